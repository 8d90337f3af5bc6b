"""GPU parity at full workload sizes, in the benchmark's launch configuration.

Each workload is drawn at its real size and the library is called the way
bench.py calls it (default path choice, caller-provided workspace, no score
output).  Then:
  * sampled rows (first, last, and rows drawn by rng(0)) pass the float64
    oracle's acceptance check one by one;
  * the number of selected indices equals the closed form: the sum over rows
    of min(k, visible), i.e. N_sel of the FLOPs notes for a full prefill;
  * for the 128K and 1M blocks, the pruned path returns the same index set as
    the unpruned path on every row, recovers no row, and its tau never
    exceeds the row's K-th score (on the sampled rows).
"""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import _lib, inputs
from helpers import OracleRows, assert_rows_ok, log, need_gpu
from oracle import counts

pytestmark = pytest.mark.gpu


def _device_inputs(name):
    wl = inputs.WORKLOADS[name]
    d = inputs.make_workload(wl)
    dev = torch.device("cuda:0")
    q, k, w, pos = (d[n].to(dev) for n in ("q", "k", "w", "pos"))
    qs = None if d["q_scale"] is None else d["q_scale"].to(dev)
    ks = None if d["k_scale"] is None else d["k_scale"].to(dev)
    return wl, d, (q, k, w, pos), dict(q_scale=qs, k_scale=ks)


def _unpruned(wl, args, kw):
    inp = _lib.make_inputs_struct(*args, kw["q_scale"], kw["k_scale"])
    ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK, inp, wl.topk), dtype=torch.uint8, device="cuda")
    idx, _ = dsa.topk(*args, wl.topk, **kw, return_scores=False, workspace=ws)
    torch.cuda.synchronize()
    return idx


def _pruned(wl, args, kw):
    inp = _lib.make_inputs_struct(*args, kw["q_scale"], kw["k_scale"])
    opts = _lib.PruneOpts(0, 0, None, None)
    ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK_PRUNED, inp, wl.topk, opts), dtype=torch.uint8,
                     device="cuda")
    idx, _, st = dsa.topk_pruned(*args, wl.topk, **kw, return_scores=False, workspace=ws, stats=True)
    torch.cuda.synchronize()
    return idx, st


def _expected_selected(wl) -> int:
    vis = np.clip(np.arange(wl.num_q, dtype=np.int64) + wl.pos_start + 1, 0, wl.num_k)
    return int(wl.batch * np.minimum(vis, wl.topk).sum())


def _sample_rows(wl, n_random):
    rng = np.random.default_rng(0)
    rows = {(0, 0), (wl.batch - 1, wl.num_q - 1)}
    while len(rows) < 2 + n_random:
        rows.add((int(rng.integers(wl.batch)), int(rng.integers(wl.num_q))))
    return sorted(rows)


def _check(name, idx, d, wl, n_random):
    got = int((idx >= 0).sum().item())
    want = _expected_selected(wl)
    log(f"  {name}: selected {got}, closed form {want}")
    assert got == want
    rows = _sample_rows(wl, n_random)
    log(f"  {name}: oracle rows {rows}")
    assert_rows_ok(OracleRows(d), idx.cpu().numpy(), None, rows, wl.topk)


def test_fullsize_prefill_32k():
    need_gpu()
    wl, d, args, kw = _device_inputs("prefill_32k")
    assert _expected_selected(wl) == counts.n_sel(wl.num_k, wl.topk)
    log("prefill_32k: unpruned Top-K at full size")
    idx = _unpruned(wl, args, kw)
    _check("prefill_32k", idx, d, wl, 4)


def test_fullsize_decode_64x128k():
    need_gpu()
    wl, d, args, kw = _device_inputs("decode_64x128k")
    log("decode_64x128k: Top-K at full size")
    idx = _unpruned(wl, args, kw)
    _check("decode_64x128k", idx, d, wl, 4)


@pytest.mark.parametrize("name", ["chunked_prefill_128k", "context_1m_fp8"])
def test_fullsize_pruned_equals_unpruned(name):
    need_gpu()
    wl, d, args, kw = _device_inputs(name)
    log(f"{name}: unpruned and pruned Top-K at full size")
    u_idx = _unpruned(wl, args, kw)
    p_idx, st = _pruned(wl, args, kw)
    assert torch.equal(torch.sort(u_idx, dim=-1).values, torch.sort(p_idx, dim=-1).values)
    assert not bool(st["recovered"].any().item())
    screened, surv = int(st["screened"].sum().item()), int(st["survivors"].sum().item())
    log(f"  {name}: identical sets on all {wl.batch * wl.num_q} rows; survivors {surv} of {screened} screened")
    n_random = 2 if wl.dtype == "fp8" else 3
    _check(name, p_idx, d, wl, n_random)
    # tau <= the row's K-th best score.  The sampled rows' scores come from
    # the score entry point on one-row slices of the inputs (the same score
    # routine as the Top-K paths, so bit-identical); the K-th best is the
    # lowest score in the returned exact set.
    q, k, w, pos = args
    tau = st["tau"].cpu().numpy()
    for b, t in _sample_rows(wl, n_random):
        # clone(): fresh, aligned one-row copies (a slice keeps its offset)
        sub = (q[b:b + 1, t:t + 1].clone(), k[b:b + 1], w[b:b + 1, t:t + 1].clone(), pos[b:b + 1, t:t + 1].clone())
        skw = dict(q_scale=None if kw["q_scale"] is None else kw["q_scale"][b:b + 1, t:t + 1].clone(),
                   k_scale=None if kw["k_scale"] is None else kw["k_scale"][b:b + 1])
        S = dsa.scores(*sub, **skw)[0, 0]
        kth = S[p_idx[b, t].long()].min().item()
        assert tau[b, t] <= kth, (b, t, tau[b, t], kth)
