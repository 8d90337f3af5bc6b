"""GPU parity at full workload sizes, in the benchmark's launch configuration.

Each workload is drawn at its real size and the library is called the way
bench.py calls it (default path choice, caller-provided workspace, no score
output).  Then:
  * 64 sampled rows (first, last, rows with fewer than k visible keys where
    there are such, and rows drawn by rng(0); every row of the decode batch)
    pass the float64 oracle's acceptance check one by one, and their
    returned scores lie within the fp32 evaluation bound of the oracle's;
  * the number of selected indices equals the closed form: the sum over rows
    of min(k, visible), i.e. N_sel of the FLOPs notes for a full prefill;
  * on 6 sampled rows of every workload, the returned set is exactly the
    Top-K (score descending, then index ascending) of the GPU's own scores
    of that row, from the score entry point (the same score routine);
  * for the 128K and 1M blocks, the pruned path returns the same index set as
    the unpruned path on every row, recovers no row, and its tau never
    exceeds the row's K-th score (on the sampled rows).
"""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import _lib, inputs
from helpers import OracleRows, assert_rows_ok, lexsort_topk_of_scores, log, need_gpu
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


def _unpruned(wl, args, kw, scores=False):
    inp = _lib.make_inputs_struct(*args, kw["q_scale"], kw["k_scale"])
    ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK, inp, wl.topk), dtype=torch.uint8, device="cuda")
    idx, sc = dsa.topk(*args, wl.topk, **kw, return_scores=scores, workspace=ws)
    torch.cuda.synchronize()
    return (idx, sc) if scores else idx


def _pruned(wl, args, kw, records="exact", seeds="even"):
    inp = _lib.make_inputs_struct(*args, kw["q_scale"], kw["k_scale"])
    opts = _lib.PruneOpts(wl.num_seeds, 0, None, None, _lib.PRUNE_RECORDS[records] | _lib.PRUNE_SEEDS[seeds])
    ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK_PRUNED, inp, wl.topk, opts), dtype=torch.uint8,
                     device="cuda")
    idx, _, st = dsa.topk_pruned(*args, wl.topk, **kw, num_seeds=wl.num_seeds, records=records, seeds=seeds,
                                 return_scores=False, workspace=ws, stats=True)
    torch.cuda.synchronize()
    return idx, st


def _expected_selected(wl) -> int:
    vis = np.clip(np.arange(wl.num_q, dtype=np.int64) + wl.pos_start + 1, 0, wl.num_k)
    return int(wl.batch * np.minimum(vis, wl.topk).sum())


def _sample_rows(wl, n_rows, n_short=0):
    """The first and last rows, n_short rows that see fewer than k keys (if
    the workload has such rows), then rows drawn by rng(0), n_rows in all
    (every row if the workload has at most n_rows)."""
    if wl.batch * wl.num_q <= n_rows:
        return [(b, t) for b in range(wl.batch) for t in range(wl.num_q)]
    rng = np.random.default_rng(0)
    rows = {(0, 0), (wl.batch - 1, wl.num_q - 1)}
    short = max(0, min(wl.num_q, wl.topk - 1 - wl.pos_start))  # rows t < short see fewer than k keys
    while short and len(rows) < 2 + n_short:
        rows.add((int(rng.integers(wl.batch)), int(rng.integers(short))))
    while len(rows) < n_rows:
        rows.add((int(rng.integers(wl.batch)), int(rng.integers(wl.num_q))))
    return sorted(rows)


def _check(name, idx, sc, d, wl, n_rows, n_short=0):
    """Selected count against the closed form; sampled rows against the
    oracle (acceptance band), their returned scores against the fp32 bound."""
    got = int((idx >= 0).sum().item())
    want = _expected_selected(wl)
    log(f"  {name}: selected {got}, closed form {want}")
    assert got == want
    rows = _sample_rows(wl, n_rows, n_short)
    log(f"  {name}: {len(rows)} oracle rows, e.g. {rows[:6]}")
    assert_rows_ok(OracleRows(d), idx.cpu().numpy(), None if sc is None else sc.cpu().numpy(), rows, wl.topk)


def _row_scores(args, kw, b, t):
    """The GPU's scores of row (b, t) from the score entry point on one-row
    slices of the inputs (clone(): fresh, aligned copies; a slice keeps its
    offset)."""
    q, k, w, pos = args
    sub = (q[b:b + 1, t:t + 1].clone(), k[b:b + 1], w[b:b + 1, t:t + 1].clone(), pos[b:b + 1, t:t + 1].clone())
    skw = dict(q_scale=None if kw["q_scale"] is None else kw["q_scale"][b:b + 1, t:t + 1].clone(),
               k_scale=None if kw["k_scale"] is None else kw["k_scale"][b:b + 1])
    return dsa.scores(*sub, **skw)[0, 0]


def _check_exact(name, wl, args, kw, idx, n_rows=6):
    """Sampled rows: the returned set equals the exact Top-K of the GPU's own
    scores of the row (a total order, so the set is unique)."""
    pos = args[3]
    for b, t in _sample_rows(wl, n_rows):
        vis = max(0, min(int(pos[b, t].item()) + 1, wl.num_k))
        S = _row_scores(args, kw, b, t).cpu().numpy()
        want = lexsort_topk_of_scores(S, vis, wl.topk)
        got = np.sort(idx[b, t].cpu().numpy())
        got = got[got >= 0]
        assert np.array_equal(got, want), (name, b, t)
    log(f"  {name}: {n_rows} rows exactly the Top-K of the GPU's own scores")


def test_fullsize_prefill_32k():
    need_gpu()
    wl, d, args, kw = _device_inputs("prefill_32k")
    assert _expected_selected(wl) == counts.n_sel(wl.num_k, wl.topk)
    log("prefill_32k: unpruned Top-K at full size")
    idx, sc = _unpruned(wl, args, kw, scores=True)
    _check("prefill_32k", idx, sc, d, wl, 64, n_short=16)
    _check_exact("prefill_32k", wl, args, kw, idx)


def test_fullsize_decode_64x128k():
    need_gpu()
    wl, d, args, kw = _device_inputs("decode_64x128k")
    log("decode_64x128k: Top-K at full size")
    idx, sc = _unpruned(wl, args, kw, scores=True)
    _check("decode_64x128k", idx, sc, d, wl, 64)
    _check_exact("decode_64x128k", wl, args, kw, idx)


@pytest.mark.parametrize("name", ["chunked_prefill_128k", "context_1m_fp8"])
def test_fullsize_pruned_equals_unpruned(name):
    need_gpu()
    wl, d, args, kw = _device_inputs(name)
    log(f"{name}: unpruned and pruned Top-K at full size")
    u_idx, u_sc = _unpruned(wl, args, kw, scores=True)
    u_sorted = torch.sort(u_idx, dim=-1).values
    # both candidate record formats (64-bit exact; 32-bit compact with the
    # boundary resolved by rescoring)
    for records in ("compact", "exact"):
        p_idx, st = _pruned(wl, args, kw, records)
        assert torch.equal(u_sorted, torch.sort(p_idx, dim=-1).values), records
        assert not bool(st["recovered"].any().item()), records
        screened, surv = int(st["screened"].sum().item()), int(st["survivors"].sum().item())
        log(f"  {name} ({records} records): identical sets on all {wl.batch * wl.num_q} rows; "
            f"survivors {surv} of {screened} screened")
    # seeds from anchor queries (num_seeds / k anchor rows)
    a_idx, a_st = _pruned(wl, args, kw, "exact", "anchor")
    assert torch.equal(u_sorted, torch.sort(a_idx, dim=-1).values), "anchor"
    assert not bool(a_st["recovered"].any().item()), "anchor"
    log(f"  {name} (anchor seeds): identical sets; survivors {int(a_st['survivors'].sum().item())}")
    # the unpruned rows against the oracle (the pruned sets equal them)
    _check(name, u_idx, u_sc, d, wl, 64)
    # the returned set is exactly the Top-K of the GPU's own row scores, and
    # tau <= the row's K-th best score (the lowest score in that set)
    _check_exact(name, wl, args, kw, u_idx)
    tau = st["tau"].cpu().numpy()
    for b, t in _sample_rows(wl, 6):
        S = _row_scores(args, kw, b, t)
        kth = S[p_idx[b, t].long()].min().item()
        assert tau[b, t] <= kth, (b, t, tau[b, t], kth)
