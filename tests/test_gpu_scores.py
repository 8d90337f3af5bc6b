"""GPU parity of the score path (dsa_indexer_scores) against the float64 oracle."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import OracleRows, call_args, log, need_gpu, to_device, tol
from oracle import indexer

pytestmark = pytest.mark.gpu


def _check_scores(d, S):
    orc = OracleRows(d)
    rtol, atol = tol(d["dtype"])
    B, Q = d["pos"].shape
    worst = 0.0
    for b in range(B):
        for t in range(Q):
            v = orc.visible(b, t)
            assert np.all(np.isneginf(S[b, t, v:])), (b, t)
            if v == 0:
                continue
            ref = orc.row(b, t)
            got = S[b, t, :v].astype(np.float64)
            err = np.abs(got - ref)
            assert np.all(err <= atol + rtol * np.abs(ref)), (b, t, float(err.max()))
            # and within the fp32 evaluation bound (tight enough to expose a
            # wrong scale or index, unlike the fp8 acceptance band)
            bnd = orc.bound(b, t)
            assert np.all(err <= bnd + 1e-12 * np.abs(ref)), (b, t, float((err / np.maximum(bnd, 1e-30)).max()))
            worst = max(worst, float(err.max()))
    return worst


@pytest.mark.parametrize(
    "B,Q,N,dtype,dist",
    [
        (1, 1, 32, "bf16", "iid"),
        (2, 5, 300, "bf16", "iid"),
        (1, 7, 2100, "bf16", "clustered"),
        (2, 3, 517, "fp8", "iid"),
        (1, 4, 1000, "fp8", "clustered"),
    ],
)
def test_scores_small_shapes(B, Q, N, dtype, dist):
    need_gpu()
    rng = np.random.default_rng(B * 1000 + Q * 10 + N)
    pos = rng.integers(-3, N + 5, size=(B, Q))
    pos[0, 0] = N - 1
    d = inputs.make_inputs(B, Q, N, dtype, dist, seed=N, positions=pos)
    log(f"scores B={B} Q={Q} N={N} {dtype} {dist}")
    args, kw = call_args(to_device(d))
    S = dsa.scores(*args, **kw).cpu().numpy()
    worst = _check_scores(d, S)
    log(f"  worst |err| = {worst:.3e}")


def test_scores_tiny_prefill_workload():
    need_gpu()
    d = inputs.make_workload("tiny_prefill_1k")
    log("scores tiny_prefill_1k")
    args, kw = call_args(to_device(d))
    S = dsa.scores(*args, **kw).cpu().numpy()
    worst = _check_scores(d, S)
    log(f"  worst |err| = {worst:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_scores_bit_identical_under_key_permutation(dtype):
    # a pair's score must not depend on where its key sits in a tile
    need_gpu()
    N = 777
    d = inputs.make_inputs(1, 6, N, dtype, "clustered", seed=3, positions=np.full((1, 6), N - 1))
    dd = to_device(d)
    args, kw = call_args(dd)
    S = dsa.scores(*args, **kw).cpu()
    perm = torch.from_numpy(np.random.default_rng(0).permutation(N))
    k2 = dd["k"][:, perm.cuda()].contiguous()
    ks2 = None if dd["k_scale"] is None else dd["k_scale"][:, perm.cuda()].contiguous()
    S2 = dsa.scores(dd["q"], k2, dd["w"], dd["pos"], q_scale=dd["q_scale"], k_scale=ks2).cpu()
    assert torch.equal(S2, S[:, :, perm])
    # and not on which other query rows share the launch
    sub = lambda t: None if t is None else t[:, 2:4].clone()  # fresh, aligned allocations
    S3 = dsa.scores(sub(dd["q"]), dd["k"], sub(dd["w"]), sub(dd["pos"]), q_scale=sub(dd["q_scale"]),
                    k_scale=dd["k_scale"]).cpu()
    assert torch.equal(S3, S[:, 2:4])


def test_special_case_zero_weights_and_linear():
    need_gpu()
    d = inputs.make_inputs(1, 3, 200, "bf16", "iid", seed=9)
    d["w"] = torch.zeros_like(d["w"])
    args, kw = call_args(to_device(d))
    S = dsa.scores(*args, **kw).cpu().numpy()
    v = indexer.visible_count(d["pos"].numpy(), 200)
    for t in range(3):
        assert np.all(S[0, t, : v[0, t]] == 0.0)
        assert not np.signbit(S[0, t, : v[0, t]]).any()
