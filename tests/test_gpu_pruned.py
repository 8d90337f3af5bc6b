"""GPU parity of the certified-pruning Top-K (dsa_indexer_topk_pruned).

Pins: the pruned index set is bit-identical to the unpruned GPU set (and its
scores equal); every screened bound dominates the GPU's own score of that pair
and the float64 oracle score; the seed threshold tau equals the K-th best GPU
score among the row's seeds and never exceeds the row's true K-th score;
forced recovery and invalid seeds still give the same result; a raised
start that misses (fewer than K exact scores reach it) recovers the row and
still gives the same result; with seeds from anchor queries tau is the K-th
best GPU score among the anchors' Top-K keys the row sees.
"""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import OracleRows, assert_rows_ok, call_args, log, need_gpu, to_device
from oracle import indexer

pytestmark = pytest.mark.gpu


def _unpruned(dd, k):
    args, kw = call_args(dd)
    idx, sc = dsa.topk(*args, k, **kw, route="stream")
    return idx.cpu().numpy(), sc.cpu().numpy()


def _same_sets(a_idx, a_sc, b_idx, b_sc):
    B, Q, k = a_idx.shape
    for b in range(B):
        for t in range(Q):
            oa, ob = np.argsort(a_idx[b, t]), np.argsort(b_idx[b, t])
            assert np.array_equal(a_idx[b, t][oa], b_idx[b, t][ob]), (b, t)
            assert np.array_equal(a_sc[b, t][oa], b_sc[b, t][ob]), (b, t)


CASES = [
    # B, Q, N, k, dtype, dist, seeds
    (1, 16, 3000, 64, "bf16", "clustered", 512),
    (1, 24, 6000, 128, "bf16", "iid", 1024),
    (2, 12, 2500, 100, "fp8", "clustered", 400),
    (1, 9, 900, 200, "bf16", "clustered", 300),  # seeds fewer than... k < seeds < N
    (1, 10, 500, 64, "bf16", "iid", 32),  # fewer seeds than k: no threshold from seeds
    (1, 8, 12000, 4096, "bf16", "clustered", 6000),  # the largest supported k
]


@pytest.mark.parametrize("start,records", [("raised", "exact"), ("tau", "exact"), ("raised", "compact"),
                                           ("tau", "compact")])
@pytest.mark.parametrize("B,Q,N,k,dtype,dist,ns", CASES)
def test_pruned_bit_identical_and_bounds(B, Q, N, k, dtype, dist, ns, start, records):
    need_gpu()
    rng = np.random.default_rng(N)
    pos = np.sort(rng.integers(N // 2, N, size=(B, Q)), axis=1)
    pos[:, -1] = N - 1
    d = inputs.make_inputs(B, Q, N, dtype, dist, seed=N + Q, positions=pos)
    dd = to_device(d)
    log(f"pruned B={B} Q={Q} N={N} k={k} {dtype} {dist} seeds={ns} start={start} records={records}")
    args, kw = call_args(dd)
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, start=start, records=records, stats=True,
                                  upper_bound=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    st = {n: v.cpu().numpy() for n, v in st.items()}
    u_idx, u_sc = _unpruned(dd, k)
    _same_sets(idx, sc, u_idx, u_sc)
    # without scores (compact records: only the boundary code is rescored)
    idx2, _, _ = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, start=start, records=records, return_scores=False)
    idx2 = idx2.cpu().numpy()
    assert np.array_equal(np.sort(idx2, axis=-1), np.sort(u_idx, axis=-1))
    # a tau start never misses; a raised start only on a miss (code 2); the
    # compact records fit these rows (code 3 would recompute them)
    assert not (st["recovered"] == 1).any()
    assert not (st["recovered"] == 3).any()
    if start == "tau":
        assert not st["recovered"].any()
    log(f"  raised-start misses: {int((st['recovered'] == 2).sum())}")
    # bounds dominate the GPU's own scores (bitwise float compare) and the oracle
    S = dsa.scores(*args, **kw).cpu().numpy()
    U = st["upper_bound"]
    orc = OracleRows(d)
    screened = 0
    for b in range(B):
        for t in range(Q):
            v = orc.visible(b, t)
            m = ~np.isnan(U[b, t, :v])
            screened += int(m.sum())
            assert np.all(U[b, t, :v][m] >= S[b, t, :v][m]), (b, t)
            ref = orc.row(b, t)
            assert np.all(U[b, t, :v][m].astype(np.float64) >= ref[m] - 1e-6 * np.abs(ref[m]).max()), (b, t)
            assert np.all(np.isnan(U[b, t, v:]))
    assert screened == int(st["screened"].sum())
    # tau: the K-th best GPU score among the row's visible seeds
    for b in range(B):
        for t in range(Q):
            v = orc.visible(b, t)
            seeds = inputs.evenly_spaced_seeds(ns, int(min(pos[b].min(), N - 1)))
            seeds = seeds[seeds < v]
            if seeds.size >= k:
                want = np.sort(S[b, t, seeds])[::-1][k - 1]
                assert st["tau"][b, t] == want, (b, t)
                assert st["tau"][b, t] <= np.sort(S[b, t, :v])[::-1][k - 1]
            else:
                assert np.isneginf(st["tau"][b, t])
    # survivors never exceed the screened keys
    assert np.all(st["survivors"] <= st["screened"])
    log(f"  screened {st['screened'].sum()}, survivors {st['survivors'].sum()} "
        f"({100 * (1 - st['survivors'].sum() / max(1, st['screened'].sum())):.1f}% pruned)")
    assert_rows_ok(orc, idx, sc, [(b, t) for b in range(B) for t in range(Q)], k)


ANCHOR_CASES = [
    # B, Q, N, k, dtype, dist, seeds, positions from (fraction of N)
    (1, 16, 3000, 64, "bf16", "clustered", 256, 0.5),
    (2, 12, 2500, 100, "fp8", "clustered", 400, 0.5),
    (1, 24, 6000, 128, "bf16", "iid", 1024, 0.5),
    (1, 32, 2000, 64, "bf16", "clustered", 192, 0.0),  # early rows see fewer than k seeds
    (1, 8, 12000, 4096, "bf16", "clustered", 8192, 0.5),  # the largest supported k, 2 anchors
]


@pytest.mark.parametrize("records", ["exact", "compact"])
@pytest.mark.parametrize("B,Q,N,k,dtype,dist,ns,lo", ANCHOR_CASES)
def test_anchor_seeds(B, Q, N, k, dtype, dist, ns, lo, records):
    """Seeds from anchor queries: the pruned set and scores equal the
    unpruned ones, and each row's tau is the K-th best GPU score among the
    visible keys of the union of its sequence's anchor rows' Top-K sets
    (anchor rows floor((2i + 1) Q / (2A)), A = num_seeds // k)."""
    need_gpu()
    rng = np.random.default_rng(N + 7)
    pos = np.sort(rng.integers(int(lo * N), N, size=(B, Q)), axis=1)
    pos[:, -1] = N - 1
    d = inputs.make_inputs(B, Q, N, dtype, dist, seed=N + 2 * Q, positions=pos)
    dd = to_device(d)
    log(f"anchor seeds B={B} Q={Q} N={N} k={k} {dtype} {dist} seeds={ns} records={records}")
    args, kw = call_args(dd)
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, seeds="anchor", records=records, stats=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    st = {n: v.cpu().numpy() for n, v in st.items()}
    u_idx, u_sc = _unpruned(dd, k)
    _same_sets(idx, sc, u_idx, u_sc)
    assert not st["recovered"].any()
    S = dsa.scores(*args, **kw).cpu().numpy()
    A = min(Q, max(1, ns // k))
    anchors = [((2 * i + 1) * Q) // (2 * A) for i in range(A)]
    assert len(set(anchors)) == A
    for b in range(B):
        union = np.unique(np.concatenate([u_idx[b, t][u_idx[b, t] >= 0] for t in anchors]))
        assert union.size <= ns
        for t in range(Q):
            seeds = union[union <= pos[b, t]]
            if seeds.size >= k:
                want = np.sort(S[b, t, seeds])[::-1][k - 1]
                assert st["tau"][b, t] == want, (b, t)
            else:
                assert np.isneginf(st["tau"][b, t]), (b, t)
    log(f"  survivors {st['survivors'].sum()} of {st['screened'].sum()} screened")
    assert_rows_ok(OracleRows(d), idx, sc, [(b, t) for b in range(B) for t in range(Q)], k)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_forced_recovery_and_invalid_seeds(dtype):
    need_gpu()
    B, Q, N, k = 2, 16, 2000, 64
    d = inputs.make_inputs(B, Q, N, dtype, "clustered", seed=3)
    dd = to_device(d)
    args, kw = call_args(dd)
    u_idx, u_sc = _unpruned(dd, k)
    force = torch.zeros((B, Q), dtype=torch.uint8)
    force[0, ::3] = 1
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=256, force_recover=force.cuda(), stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    assert np.array_equal(st["recovered"].cpu().numpy(), force.numpy())
    # descending seeds are invalid: the whole sequence recovers
    bad = torch.arange(256, dtype=torch.int32).flip(0).repeat(B, 1).contiguous()
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=256, seed_idx=bad.cuda(), stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    assert st["recovered"].cpu().numpy().all()
    # valid custom seeds (random, ascending) are fine
    rng = np.random.default_rng(0)
    good = np.stack([np.sort(rng.choice(1984, 300, replace=False)) for _ in range(B)]).astype(np.int32)
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=300, seed_idx=torch.from_numpy(good).cuda(), stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    assert not st["recovered"].cpu().numpy().any()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_raised_start_miss_recovers(dtype):
    """Nonnegative head weights and seed keys doubled (bf16 values, or fp8
    key scales, times 2): every score is a sum of ReLUs, so doubling a key
    doubles its score and the seeds hold the best scores of every row.  The
    raised start (seed rank m = 106 < K = 256 here) is then reached by m
    keys only (checked in float64 when the case was chosen), every row must
    be recomputed unpruned (recovered = 2) and the result is still the
    exact Top-K; with a tau start the same inputs need no recovery."""
    need_gpu()
    B, Q, N, k, ns = 1, 12, 4000, 256, 1000
    d = inputs.make_inputs(B, Q, N, dtype, "iid", seed=21)
    d["w"] = d["w"].abs()
    seeds = inputs.evenly_spaced_seeds(ns, int(d["pos"].min()))
    if dtype == "bf16":
        d["k"][:, seeds] = d["k"][:, seeds] * 2
    else:
        d["k_scale"][:, seeds] = d["k_scale"][:, seeds] * 2
    dd = to_device(d)
    args, kw = call_args(dd)
    log(f"raised-start miss {dtype}")
    u_idx, u_sc = _unpruned(dd, k)
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    rec = st["recovered"].cpu().numpy()
    assert (rec == 2).all(), rec
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, records="compact", stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    assert (st["recovered"].cpu().numpy() == 2).all()
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, start="tau", stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    assert not st["recovered"].cpu().numpy().any()
    assert_rows_ok(OracleRows(d), u_idx, u_sc, [(0, t) for t in range(Q)], k)


@pytest.mark.parametrize("start,records", [("raised", "exact"), ("tau", "exact"), ("raised", "compact"),
                                           ("tau", "compact")])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_ties_and_zero_weights(dtype, start, records):
    """Rows with all-zero weights score every key 0, so their Top-K is keys
    0..k-1 by the tie rule, and every key at or below the start's key is a
    candidate.  With a tau start that is about 2480 keys (the 128th of 1024
    seeds over 20000 keys).  Exact records are cut as usual.  Compact records
    put them all in one score code, which no cut can split, so the buffer
    (4k + 640 = 1152 records) cannot make room and the row is recomputed
    unpruned (recovered = 3).  With the raised start (seed rank 21, about
    390 keys) the boundary code is rescored instead.  Every combination
    gives the unpruned sets, with and without scores."""
    need_gpu()
    B, Q, N, k = 1, 12, 20000, 128
    d = inputs.make_inputs(B, Q, N, dtype, "clustered", seed=5)
    d["w"][0, ::3] = 0.0
    dd = to_device(d)
    args, kw = call_args(dd)
    log(f"ties {dtype} {start} {records}")
    u_idx, u_sc = _unpruned(dd, k)
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=1024, start=start, records=records, stats=True)
    _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    idx2, _, st2 = dsa.topk_pruned(*args, k, **kw, num_seeds=1024, start=start, records=records,
                                   return_scores=False, stats=True)
    assert np.array_equal(np.sort(idx2.cpu().numpy(), axis=-1), np.sort(u_idx, axis=-1))
    zero_rows = np.arange(Q) % 3 == 0
    assert np.array_equal(np.sort(u_idx[0, zero_rows], axis=-1), np.tile(np.arange(k), (zero_rows.sum(), 1)))
    for s_ in (st, st2):
        rec = s_["recovered"].cpu().numpy()[0]
        assert not rec[~zero_rows].any(), rec
        want = 3 if (records == "compact" and start == "tau") else 0
        assert (rec[zero_rows] == want).all(), rec
    log(f"  recovered: {st['recovered'].cpu().numpy()[0].tolist()}")


def test_pruned_small_and_degenerate():
    need_gpu()
    # few visible keys, negative positions, zero weights, one retained head
    N, Q, k = 300, 12, 50
    pos = np.array([[-1, 0, 3, 40, 49, 50, 100, 299, 299, 150, 10, 280]])
    d = inputs.make_inputs(1, Q, N, "bf16", "iid", seed=11, positions=pos)
    d["w"][0, 5] = 0.0
    dd = to_device(d)
    args, kw = call_args(dd)
    u_idx, u_sc = _unpruned(dd, k)
    for nret in (1, 14):
        idx, sc, _ = dsa.topk_pruned(*args, k, **kw, num_seeds=64, num_retained=nret)
        _same_sets(idx.cpu().numpy(), sc.cpu().numpy(), u_idx, u_sc)
    assert_rows_ok(OracleRows(d), u_idx, u_sc, [(0, t) for t in range(Q)], k)


@pytest.mark.parametrize("dtype,dist", [("bf16", "clustered"), ("bf16", "iid"), ("fp8", "clustered")])
def test_exported_plans_certify_the_exact_scores(dtype, dist):
    """Every row's bound plan, exported from the GPU and re-evaluated in
    float64 by the oracle (oracle.prune.bound_from_plan), lies above the
    exact score of every visible key -- the certificate holds in exact
    arithmetic, not only against the GPU's own fp32 scores -- and the GPU's
    fp32 bounds of the screened keys agree with it to fp32 rounding."""
    from oracle import prune

    need_gpu()
    B, Q, N, k = 1, 12, 4000, 64
    pos = np.sort(np.random.default_rng(7).integers(N // 2, N, size=(B, Q)), axis=1)
    pos[:, -1] = N - 1
    d = inputs.make_inputs(B, Q, N, dtype, dist, seed=77, positions=pos)
    dd = to_device(d)
    args, kw = call_args(dd)
    log(f"plan export {dtype} {dist}")
    _, _, st = dsa.topk_pruned(*args, k, **kw, num_seeds=512, stats=True, upper_bound=True, plan=True)
    st = {n: v.cpu() for n, v in st.items()}
    orc = OracleRows(d)
    rows_bits = inputs.to_bits(st["plan_rows"])
    coef, misc, U = st["plan_coef"].numpy(), st["plan_misc"].numpy(), st["upper_bound"].numpy()
    for t in range(Q):
        assert not st["recovered"][0, t]
        v = orc.visible(0, t)
        if dtype == "bf16":
            prow = indexer.decode_bf16(rows_bits[0, t])
            keys, scale = orc.keys(0)[:v], None
        else:
            prow = indexer.decode_e4m3fn(rows_bits[0, t])
            keys = indexer.decode_e4m3fn(orc.kbits[0, :v])
            scale = np.float64(orc.qs[0, t]) * orc.ks[0, :v].astype(np.float64)
        Up = prune.bound_from_plan(prow, coef[0, t], misc[0, t, 0], misc[0, t, 1], keys, scale)
        exact = orc.row(0, t)
        assert np.all(Up >= exact), (t, float((exact - Up).max()))
        m = ~np.isnan(U[0, t, :v])
        assert m.sum() > 0
        # scale of the terms the fp32 evaluation rounds: sum |c_i| |rows_i| . |k| plus the |k| terms
        kn = np.linalg.norm(keys, axis=1)
        mag = np.abs(coef[0, t]) @ (np.abs(prow) @ np.abs(keys).T) + (abs(misc[0, t, 0]) + abs(misc[0, t, 1])) * kn
        if scale is not None:
            mag = mag * scale
        assert np.all(np.abs(U[0, t, :v][m] - Up[m]) <= 1e-5 * mag[m] + 1e-30), t
