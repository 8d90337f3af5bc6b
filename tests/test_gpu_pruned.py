"""GPU parity of the certified-pruning Top-K (dsa_indexer_topk_pruned).

Pins: the pruned index set is bit-identical to the unpruned GPU set (and its
scores equal); every screened bound dominates the GPU's own score of that pair
and the float64 oracle score; the seed threshold tau equals the K-th best GPU
score among the row's seeds and never exceeds the row's true K-th score;
forced recovery and invalid seeds still give the same result.
"""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import OracleRows, assert_rows_ok, call_args, log, need_gpu, set_path, to_device
from oracle import indexer

pytestmark = pytest.mark.gpu


def _unpruned(dd, k):
    args, kw = call_args(dd)
    set_path("stream")
    try:
        idx, sc = dsa.topk(*args, k, **kw)
    finally:
        set_path(None)
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


@pytest.mark.parametrize("B,Q,N,k,dtype,dist,ns", CASES)
def test_pruned_bit_identical_and_bounds(B, Q, N, k, dtype, dist, ns):
    need_gpu()
    rng = np.random.default_rng(N)
    pos = np.sort(rng.integers(N // 2, N, size=(B, Q)), axis=1)
    pos[:, -1] = N - 1
    d = inputs.make_inputs(B, Q, N, dtype, dist, seed=N + Q, positions=pos)
    dd = to_device(d)
    log(f"pruned B={B} Q={Q} N={N} k={k} {dtype} {dist} seeds={ns}")
    args, kw = call_args(dd)
    idx, sc, st = dsa.topk_pruned(*args, k, **kw, num_seeds=ns, stats=True, upper_bound=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    st = {n: v.cpu().numpy() for n, v in st.items()}
    u_idx, u_sc = _unpruned(dd, k)
    _same_sets(idx, sc, u_idx, u_sc)
    assert not st["recovered"].any()
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
