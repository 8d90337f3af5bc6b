"""GPU parity of the exact Top-K (dsa_indexer_topk), both launch paths.

Two checks per row:
  * exact: the GPU index set equals a CPU sort (score desc, index asc) of the
    GPU's own scores from dsa_indexer_scores (the scores are bit-identical
    across paths, so this must hold exactly), and returned scores equal them;
  * oracle: the set passes the float64 oracle's tolerance band.
"""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import OracleRows, assert_rows_ok, call_args, lexsort_topk_of_scores, log, need_gpu, to_device

pytestmark = pytest.mark.gpu


def _exact_vs_own_scores(d, dd, idx, sc, k):
    args, kw = call_args(dd)
    S = dsa.scores(*args, **kw).cpu().numpy()
    pos = d["pos"].numpy()
    N = d["k"].shape[1]
    B, Q = pos.shape
    for b in range(B):
        for t in range(Q):
            vis = int(np.clip(pos[b, t] + 1, 0, N))
            want = lexsort_topk_of_scores(S[b, t], vis, k)
            n = want.size
            got = idx[b, t, :n]
            assert np.all(idx[b, t, n:] == -1), (b, t)
            assert np.array_equal(np.sort(got), want), (b, t)
            if sc is not None:
                assert np.array_equal(sc[b, t, :n], S[b, t, got]), (b, t)
                assert np.all(np.isneginf(sc[b, t, n:]))


CASES = [
    # B, Q, N, k, dtype, dist
    (1, 16, 700, 64, "bf16", "iid"),
    (2, 21, 1500, 100, "bf16", "clustered"),
    (1, 9, 3000, 16, "bf16", "iid"),  # many buffer compactions
    (1, 12, 400, 500, "bf16", "iid"),  # fewer visible keys than k
    (2, 10, 1100, 128, "fp8", "clustered"),
    (2, 7, 1001, 50, "bf16", "iid"),  # odd row length: unaligned score rows on the split path
    (1, 6, 9000, 4096, "bf16", "clustered"),  # the largest supported k
    (1, 5, 7000, 4096, "fp8", "iid"),  # the largest supported k, fp8 (128-key tiles)
]


@pytest.mark.parametrize("path", ["split", "stream"])
@pytest.mark.parametrize("B,Q,N,k,dtype,dist", CASES)
def test_topk_small(path, B, Q, N, k, dtype, dist):
    need_gpu()
    rng = np.random.default_rng(N + Q)
    pos = rng.integers(-2, N + 3, size=(B, Q))
    pos[0, -1] = N - 1
    d = inputs.make_inputs(B, Q, N, dtype, dist, seed=Q, positions=pos)
    dd = to_device(d)
    log(f"topk {path} B={B} Q={Q} N={N} k={k} {dtype} {dist}")
    args, kw = call_args(dd)
    idx, sc = dsa.topk(*args, k, **kw, route=path)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    _exact_vs_own_scores(d, dd, idx, sc, k)
    assert_rows_ok(OracleRows(d), idx, sc, [(b, t) for b in range(B) for t in range(Q)], k)


@pytest.mark.parametrize("path", ["split", "stream"])
def test_topk_ties_take_smallest_indices(path):
    need_gpu()
    d = inputs.make_inputs(1, 8, 900, "bf16", "iid", seed=1)
    d["w"] = torch.zeros_like(d["w"])
    args, kw = call_args(to_device(d))
    idx, _ = dsa.topk(*args, 50, **kw, route=path)
    idx = idx.cpu().numpy()
    for t in range(8):
        assert np.array_equal(np.sort(idx[0, t]), np.arange(50))


def test_topk_tiny_prefill_workload():
    need_gpu()
    wl = inputs.WORKLOADS["tiny_prefill_1k"]
    d = inputs.make_workload(wl)
    dd = to_device(d)
    log("topk tiny_prefill_1k (default path)")
    args, kw = call_args(dd)
    idx, sc = dsa.topk(*args, wl.topk, **kw)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    _exact_vs_own_scores(d, dd, idx, sc, wl.topk)
    assert_rows_ok(OracleRows(d), idx, sc, [(0, t) for t in range(wl.num_q)], wl.topk)
    # selected count closed form: sum_t min(k, t+1)
    assert int((idx >= 0).sum()) == 229504


def test_topk_paths_agree_on_a_prefill_block():
    need_gpu()
    d = inputs.make_inputs(1, 64, 5000, "bf16", "clustered", seed=5)
    dd = to_device(d)
    args, kw = call_args(dd)
    out = {}
    for path in ("split", "stream"):
        out[path] = [x.cpu() for x in dsa.topk(*args, 256, **kw, route=path)]
    a = torch.sort(out["split"][0], -1).values
    b = torch.sort(out["stream"][0], -1).values
    assert torch.equal(a, b)


@pytest.mark.parametrize("path", ["split", "stream"])
@pytest.mark.parametrize("k", [1, 2, 5, 33])
def test_topk_rising_scores_small_k(path, k):
    """Scores that rise with the key index: every fp8 key tile beats the
    running threshold, the worst case for a row's candidate buffer.  All
    codes are 1.0 and the key scales are 1 + s/1024 (exact in fp32), so
    key s scores 8192 * (1 + s/1024) and a row at position p selects the
    keys p - k + 1 .. p (those that exist)."""
    need_gpu()
    Q, N = 12, 3000
    pos = torch.tensor([[0, 1, 4, 127, 128, 129, 700, 1500, 2047, 2500, 2998, 2999]], dtype=torch.int32)
    d = {
        "q": torch.full((1, Q, 64, 128), 1.0).to(torch.float8_e4m3fn),
        "k": torch.full((1, N, 128), 1.0).to(torch.float8_e4m3fn),
        "w": torch.ones(1, Q, 64),
        "pos": pos,
        "q_scale": torch.ones(1, Q),
        "k_scale": (1.0 + torch.arange(N, dtype=torch.float32) / 1024)[None],
    }
    dd = to_device(d)
    log(f"topk rising scores {path} k={k}")
    args, kw = call_args(dd)
    idx, sc = dsa.topk(*args, k, **kw, route=path)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    for t in range(Q):
        p = int(pos[0, t])
        want = np.arange(max(0, p - k + 1), p + 1)
        n = want.size
        assert np.array_equal(np.sort(idx[0, t, :n]), want), (t, idx[0, t])
        assert np.all(idx[0, t, n:] == -1), t
        np.testing.assert_array_equal(np.sort(sc[0, t, :n]), 8192.0 * (1.0 + want / 1024).astype(np.float32))
