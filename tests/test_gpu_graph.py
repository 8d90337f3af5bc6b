"""The entry points are safe to capture in a HIP graph: they enqueue kernels
only (no allocation, memset or host synchronisation inside the library), so a
captured call replays to the eager result.  Each graph is replayed several
times with eager work and synchronisation between replays, and every replay
is compared bit for bit with the eager call.  (The projection entry point
runs rocBLAS and is not replayed here; its first call on a thread refuses
a capturing stream, which the last test checks.)"""
import math

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import _lib, inputs
from helpers import log, need_gpu

pytestmark = pytest.mark.gpu


def _canon(outs):
    """Top-K rows are sets (indices in no particular order, scores beside
    them): sort each row by index and carry the scores along."""
    idx, sc = outs
    order = idx.argsort(-1)
    return idx.gather(-1, order), (None if sc is None else sc.gather(-1, order))


def _replays_match(fn, eager, n=3, canon=None):
    """Capture fn() (returning a tuple of tensors), replay n times and compare."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    for i in range(n):
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        for o in outs:
            if o is not None:
                o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got, want = (canon(outs), canon(eager)) if canon else (outs, eager)
        for o, e in zip(got, want):
            if o is None:
                continue
            assert torch.equal(o.view(torch.int32) if o.dtype == torch.float32 else o,
                               e.view(torch.int32) if e.dtype == torch.float32 else e), f"replay {i} differs"
        del junk


def test_topk_and_pruned_graphs():
    need_gpu()
    d = inputs.make_inputs(1, 40, 3000, "bf16", "clustered", seed=5)
    q, k, w, pos = (d[n].cuda() for n in ("q", "k", "w", "pos"))
    topk = 64
    inp = _lib.make_inputs_struct(q, k, w, pos)
    ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK, inp, topk), dtype=torch.uint8, device="cuda")
    opts = _lib.PruneOpts(0, 0, None, None)
    wsp = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK_PRUNED, inp, topk, opts), dtype=torch.uint8,
                      device="cuda")
    log("[graph] topk")
    eager = dsa.topk(q, k, w, pos, topk, workspace=ws)
    _replays_match(lambda: dsa.topk(q, k, w, pos, topk, workspace=ws), eager, canon=_canon)
    log("[graph] pruned")
    ep = dsa.topk_pruned(q, k, w, pos, topk, num_seeds=256, workspace=wsp)[:2]
    _replays_match(lambda: dsa.topk_pruned(q, k, w, pos, topk, num_seeds=256, workspace=wsp)[:2], ep, canon=_canon)
    assert torch.equal(_canon(ep)[0], _canon(eager)[0])


def test_sparse_mla_graph_split_path():
    need_gpu()
    B, Q, N, k = 4, 1, 3000, 1024  # few rows: the split-and-merge route
    d = inputs.make_mla_inputs(B, Q, N, seed=9)
    idx = torch.from_numpy(inputs.random_selection(B, Q, N, k, np.full((B, Q), N - 1), seed=9)).cuda()
    q, kv = d["q"].cuda(), d["kv"].cuda()
    ws = torch.empty(_lib.sparse_mla_workspace_bytes(_lib.make_mla_struct(q, kv, idx)), dtype=torch.uint8,
                     device="cuda")
    log("[graph] sparse mla")
    eager = dsa.sparse_mla(q, kv, idx, 1.0 / math.sqrt(576), workspace=ws)
    _replays_match(lambda: dsa.sparse_mla(q, kv, idx, 1.0 / math.sqrt(576), workspace=ws), eager)


def test_projection_refuses_to_create_its_handle_under_capture():
    """The projection's first call on a thread creates a rocBLAS handle, which
    allocates: on a capturing stream that first call returns
    DSA_ERR_UNSUPPORTED (the capture stays clean), and a later call outside
    capture works.  Run on a fresh thread, whose handle does not exist yet."""
    import threading
    import warnings

    need_gpu()
    d = {n: v.cuda() for n, v in inputs.make_projection_inputs(16, 256, 128, seed=1).items()}
    args = (d["c_q"], d["x"], d["w_iq"], d["w_ik"], d["w_iw"])
    ws = torch.empty(_lib.project_workspace_bytes(_lib.make_proj_struct(*args)), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    seen = {}

    def body():
        try:
            s = torch.cuda.Stream()
            g = torch.cuda.CUDAGraph()
            try:
                # the refused call leaves the capture empty, which torch warns about
                with warnings.catch_warnings():
                    warnings.filterwarnings("ignore", message="The CUDA Graph is empty")
                    with torch.cuda.graph(g, stream=s):
                        dsa.project(*args, out="f32", workspace=ws)
            except _lib.IndexerError as e:
                seen["code"] = e.code
            except Exception as e:  # the capture context may re-raise on exit
                seen.setdefault("other", repr(e))
            torch.cuda.synchronize()
            out = dsa.project(*args, out="f32", workspace=ws)  # outside capture: creates the handle
            torch.cuda.synchronize()
            seen["after"] = bool(torch.isfinite(out["q"]).all().item())
        except Exception as e:
            seen["thread_error"] = repr(e)

    th = threading.Thread(target=body)
    th.start()
    th.join(timeout=120)
    log(f"[graph] projection under capture: {seen}")
    assert seen.get("code") == 2, seen  # DSA_ERR_UNSUPPORTED
    assert seen.get("after") is True
