"""Pins of the float64 oracle to facts the pages and mathematics fix.

Every check here is independent of the oracle's own formula: printed numbers,
hand-worked examples, closed forms, library routines in special cases, and
invariants of the score (homogeneity, symmetry, head permutation).
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_table
from oracle import counts, indexer


# ------------------------------------------------------------ printed values


def _computed_worked_values():
    c = counts.V32
    T = 131072
    return {
        "core_flops_per_pair": counts.core_flops_per_pair(),
        "n_sel_131072_2048": counts.n_sel(T, c["k"]),
        "core_prefill_131072": counts.core_prefill_flops(T) / 1e12,
        "core_decode_token": counts.core_decode_flops(T) / 1e6,
        "indexer_linear_coeff": counts.indexer_proj_flops(1),
        "indexer_quadratic_coeff": counts.indexer_score_flops_causal(1) // 2,
        "indexer_proj_131072": counts.indexer_proj_flops(T) / 1e12,
        "indexer_score_131072": counts.indexer_score_flops_causal(T) / 1e12,
        "indexer_total_131072": counts.indexer_prefill_flops(T) / 1e12,
        "indexer_decode_const": counts.indexer_decode_flops(0),
        "indexer_decode_per_key": counts.indexer_decode_flops(1) - counts.indexer_decode_flops(0),
        "indexer_decode_131072": counts.indexer_decode_flops(T) / 1e9,
        "indexer_decode_scan_131072": (counts.indexer_decode_flops(T) - counts.indexer_decode_flops(0)) / 1e9,
        "total_prefill_131072": (counts.core_prefill_flops(T) + counts.indexer_prefill_flops(T)) / 1e12,
        "total_decode_131072": (counts.core_decode_flops(T) + counts.indexer_decode_flops(T)) / 1e9,
    }


def test_pages_worked_values():
    got = _computed_worked_values()
    rows = read_table("pages_worked_values.txt")
    assert len(rows) == len(got)
    for name, printed, _unit, decimals, _where in rows:
        d = int(decimals)
        assert round(got[name], d) == pytest.approx(float(printed), abs=10 ** (-d) / 10), name


@pytest.mark.parametrize("T,k", [(1, 1), (5, 2), (7, 7), (8, 3), (100, 17), (1024, 256), (3000, 2048)])
def test_n_sel_closed_form_vs_sum(T, k):
    assert counts.n_sel(T, k) == counts.n_sel_brute(T, k)


def test_selected_counts_of_the_workloads():
    # non-padding indices per workload: sum over rows of min(k, visible)
    assert counts.n_sel(1024, 256) == 229504
    assert counts.n_sel(32768, 2048) == 65012736
    assert 64 * 2048 == 131072
    assert counts.n_dense(1024) == 524800
    assert counts.n_dense(32768) == 536887296


# ------------------------------------------------------------ hand example


def _hand():
    rows = {r[0]: r[1] for r in read_table("hand_examples.txt")}
    mat = lambda s: np.array([[float(x) for x in row.split()] for row in s.split(";")])
    vec = lambda s: np.array([float(x) for x in s.split()])
    return rows, mat(rows["q"]), vec(rows["w"]), mat(rows["keys"]), vec(rows["scores"])


def test_hand_worked_scores():
    _, q, w, keys, want = _hand()
    got = indexer.index_score_row(q, keys, w)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("pos,key", [(3, "top2_pos3"), (2, "top2_pos2"), (0, "top2_pos0")])
def test_hand_worked_topk(pos, key):
    rows, q, w, keys, _ = _hand()
    want = sorted(int(x) for x in rows[key].split())
    qf = q[None, None]
    kf = keys[None]
    S = indexer.index_scores(qf, kf, w[None, None], np.array([[pos]]))
    n = int(indexer.visible_count(pos, keys.shape[0]))
    assert n == pos + 1
    sel = indexer.topk_row(S[0, 0, :n], 2)
    assert sorted(sel.tolist()) == want
    assert np.all(np.isneginf(S[0, 0, n:]))


# ------------------------------------------------------------ decoding


def test_fp8_codes_table():
    for code, val in read_table("fp8_e4m3fn_codes.txt"):
        got = indexer.decode_e4m3fn(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_fp8_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = indexer.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[m], ref[m])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**16, size=4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ours = indexer.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert indexer.decode_bf16(np.array([0x3F80], np.uint16))[0] == 1.0
    assert indexer.decode_bf16(np.array([0xC000], np.uint16))[0] == -2.0


# ------------------------------------------------------------ special cases


def test_single_head_unit_weight_is_relu_of_matmul():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 16))
    keys = rng.standard_normal((50, 16))
    got = indexer.index_score_row(q, keys, np.ones(1))
    want = np.clip(np.dot(keys, q[0]), 0, None)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)


def test_nonnegative_case_is_linear():
    # q, k >= 0 and w >= 0: no ReLU clips, so I = (sum_j w_j q_j) . k  (a GEMV)
    rng = np.random.default_rng(3)
    q = rng.random((64, 128))
    keys = rng.random((40, 128))
    w = rng.random(64)
    got = indexer.index_score_row(q, keys, w)
    want = keys @ (q.T @ w)
    np.testing.assert_allclose(got, want, rtol=1e-12)


def test_score_invariants():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((64, 128))
    keys = rng.standard_normal((30, 128))
    w = rng.standard_normal(64)
    base = indexer.index_score_row(q, keys, w)
    # positive homogeneity in q, k and w
    np.testing.assert_allclose(indexer.index_score_row(2.5 * q, keys, w), 2.5 * base, rtol=1e-12)
    np.testing.assert_allclose(indexer.index_score_row(q, 0.5 * keys, w), 0.5 * base, rtol=1e-12)
    np.testing.assert_allclose(indexer.index_score_row(q, keys, 3 * w), 3 * base, rtol=1e-12)
    # ReLU(q.k) is unchanged when both q and k flip sign
    np.testing.assert_allclose(indexer.index_score_row(-q, -keys, w), base, rtol=1e-12)
    # head order does not matter
    perm = rng.permutation(64)
    np.testing.assert_allclose(indexer.index_score_row(q[perm], keys, w[perm]), base, rtol=1e-12)
    # a head with w = 0 contributes nothing; a head split in two with w/2 each is the same
    q2 = np.concatenate([q, q[:1]])
    w2 = np.concatenate([w, [0.0]])
    np.testing.assert_allclose(indexer.index_score_row(q2, keys, w2), base, rtol=1e-12)
    w3 = w.copy()
    w3[0] /= 2
    q3 = np.concatenate([q, q[:1]])
    w3 = np.concatenate([w3, [w[0] / 2]])
    np.testing.assert_allclose(indexer.index_score_row(q3, keys, w3), base, rtol=1e-12, atol=1e-12)
    # only the key's own row matters (not its position among the keys)
    kp = rng.permutation(30)
    np.testing.assert_allclose(indexer.index_score_row(q, keys[kp], w), base[kp], rtol=1e-13, atol=1e-13)


def test_visibility_counts_match_closed_forms():
    T = 257
    pos = np.arange(T)
    vis = indexer.visible_count(pos, T)
    assert vis.sum() == counts.n_dense(T)
    assert np.minimum(vis, 32).sum() == counts.n_sel(T, 32)
    assert indexer.visible_count(-1, 10) == 0
    assert indexer.visible_count(100, 10) == 10


def test_full_score_matrix_visibility():
    rng = np.random.default_rng(5)
    qf = rng.standard_normal((2, 9, 3, 4))
    kf = rng.standard_normal((2, 12, 4))
    w = rng.standard_normal((2, 9, 3))
    pos = np.array([np.arange(9) + 3, np.arange(9) * 2 - 2])
    S = indexer.index_scores(qf, kf, w, pos)
    finite = np.isfinite(S)
    want = indexer.visible_count(pos, 12)
    np.testing.assert_array_equal(finite.sum(-1), want)
    for b in range(2):
        for t in range(9):
            for s in range(12):
                if s <= pos[b, t]:
                    v = sum(w[b, t, j] * max(float(qf[b, t, j] @ kf[b, s]), 0.0) for j in range(3))
                    assert S[b, t, s] == pytest.approx(v, rel=1e-12, abs=1e-14)


# ------------------------------------------------------------ Top-K


def test_topk_matches_argpartition():
    rng = np.random.default_rng(6)
    for n, k in [(1000, 10), (5000, 2048), (300, 300), (50, 100)]:
        s = rng.standard_normal(n)
        sel = indexer.topk_row(s, k)
        kk = min(k, n)
        ref = np.argpartition(-s, kk - 1)[:kk]
        assert set(sel.tolist()) == set(ref.tolist())
        # first the best, last the K-th
        assert s[sel[0]] == s.max()
        assert indexer.kth_score(s, k) == np.sort(s)[::-1][kk - 1]


def test_topk_tie_rule_zero_weights():
    # w = 0: every score is 0 and the total order keeps the k smallest indices
    rng = np.random.default_rng(7)
    q = rng.standard_normal((64, 128))
    keys = rng.standard_normal((500, 128))
    s = indexer.index_score_row(q, keys, np.zeros(64))
    assert np.all(s == 0)
    np.testing.assert_array_equal(np.sort(indexer.topk_row(s, 37)), np.arange(37))


def test_topk_fewer_visible_than_k():
    s = np.array([0.3, -1.0, 2.0])
    assert sorted(indexer.topk_row(s, 10).tolist()) == [0, 1, 2]


# ------------------------------------------------------------ acceptance check


def test_acceptance_check_accepts_exact_and_catches_mistakes():
    rng = np.random.default_rng(8)
    s = rng.standard_normal(4000)
    k = 256
    good = indexer.topk_row(s, k)
    row = np.full(300, -1)
    row[:k] = good
    assert indexer.check_topk_row(row, s, k, 2e-3, 1e-3, gpu_scores=s[good]) == []
    bad = row.copy()
    bad[0] = int(np.argmin(s))
    assert indexer.check_topk_row(bad, s, k, 2e-3, 1e-3)
    dup = row.copy()
    dup[1] = dup[0]
    assert indexer.check_topk_row(dup, s, k, 2e-3, 1e-3)
    short = row.copy()
    short[k - 1] = -1
    assert indexer.check_topk_row(short, s, k, 2e-3, 1e-3)
    off = s[good] * (1 + 1e-2)
    assert indexer.check_topk_row(row, s, k, 2e-3, 1e-3, gpu_scores=off)


# ---------------------------------------------------------------- fp32 error bound


def _fp32_score_row(q, k, w, rng):
    """One fp32 evaluation of the score (float32 products and sums in a
    random order per head, then a random-order weighted sum): a stand-in for
    any fp32 evaluation order."""
    q32, k32, w32 = q.astype(np.float32), k.astype(np.float32), w.astype(np.float32)
    n, H = k.shape[0], q.shape[0]
    out = np.zeros(n, np.float32)
    for s in range(n):
        x = np.zeros(H, np.float32)
        for j in range(H):
            prods = q32[j] * k32[s]  # exact: products of bf16 values
            acc = np.float32(0.0)
            for v in prods[rng.permutation(prods.size)]:
                acc = np.float32(acc + v)
            x[j] = acc
        terms = w32 * np.maximum(x, np.float32(0.0))
        acc = np.float32(0.0)
        for v in terms[rng.permutation(H)]:
            acc = np.float32(acc + v)
        out[s] = acc
    return out


def test_error_bound_dominates_fp32_evaluations():
    """The bound covers real fp32 evaluations (random summation orders) of
    random bf16 rows, and is not vacuous: it stays below 5e-4 of the row's
    score scale, a quarter of the bf16 acceptance band."""
    from dsa_lightning_indexer_04_amd import inputs

    rng = np.random.default_rng(5)
    d = inputs.make_inputs(1, 3, 40, "bf16", "iid", seed=5)
    qf, kf = indexer.dequantize(inputs.to_bits(d["q"]), inputs.to_bits(d["k"]), "bf16")
    w = d["w"].numpy().astype(np.float64)
    for t in range(3):
        exact = indexer.index_score_row(qf[0, t], kf[0], w[0, t])
        bound = indexer.score_error_bound_row(qf[0, t], kf[0], w[0, t])
        got = _fp32_score_row(qf[0, t], kf[0], w[0, t], rng).astype(np.float64)
        assert np.all(np.abs(got - exact) <= bound)
        assert np.all(bound < 5e-4 * np.abs(exact).max())


def test_error_bound_catches_a_scale_mistake():
    """A 2% mistake in a key's scale (an fp8 indexing or scaling slip) is
    outside the bound on every key scoring at least a quarter of the row's
    largest |score|, while the acceptance band of the fp8 comparison (3e-2
    relative) lets it pass."""
    from dsa_lightning_indexer_04_amd import inputs

    d = inputs.make_inputs(1, 2, 64, "fp8", "clustered", seed=2)
    qb, kb = inputs.to_bits(d["q"]), inputs.to_bits(d["k"])
    q8, k8 = indexer.decode_e4m3fn(qb[0, 0]), indexer.decode_e4m3fn(kb[0])
    qs, ks = float(d["q_scale"][0, 0]), d["k_scale"][0].numpy().astype(np.float64)
    w = d["w"].numpy()[0, 0].astype(np.float64)
    exact = ks * qs * indexer.index_score_row(q8, k8, w)
    bound = indexer.score_error_bound_row(q8, k8, w, scale=qs * ks)
    wrong = exact * 1.02
    big = np.abs(exact) >= 0.25 * np.abs(exact).max()
    assert big.sum() >= 5
    assert np.all(np.abs(wrong - exact)[big] > bound[big])
    rtol, atol = indexer.tolerance("fp8")
    assert np.all(np.abs(wrong - exact) <= atol + rtol * np.abs(exact))


def test_error_bound_closed_form_on_a_hand_example():
    """One head, one key: x = 0.5*2 + 0.25*(-4) + 1*3 = 3, w = -2:
    A = 2*(1 + 1 + 3) = 10, B = 2*3 = 6, bound = g128*10 + g64*(6 + g128*10)."""
    q = np.array([[0.5, 0.25, 1.0]])
    k = np.array([[2.0, -4.0, 3.0]])
    w = np.array([-2.0])
    g128, g64 = indexer.gamma(128), indexer.gamma(64)
    want = g128 * 10 + g64 * (6 + g128 * 10)
    assert indexer.score_error_bound_row(q, k, w)[0] == pytest.approx(want, rel=1e-12)
    assert indexer.gamma(1) == pytest.approx(2.0**-24, rel=1e-6)
