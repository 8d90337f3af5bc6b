"""MI355X-native DSA lightning indexer with exact per-query Top-K.

Public calls (thin wrappers over the C ABI in include/dsa_indexer.h):
    scores(q, k, w, positions, q_scale=None, k_scale=None)
    topk(q, k, w, positions, topk, q_scale=None, k_scale=None)
    topk_noalloc(q, k, w, positions, topk, ...)   (fixed library scratch, no workspace)
    topk_pruned(q, k, w, positions, topk, ..., num_seeds=0, num_retained=0)
    project(c_q, x, w_iq, w_ik, w_iw, out="fp8")   (the indexer projections)
    sparse_mla(q, kv, indices, sm_scale)          (core attention over the Top-K)
The HIP library is loaded on first use; importing the package does not
touch the GPU.  Seeded synthetic inputs live in the ``inputs`` module.
"""
from __future__ import annotations


def __getattr__(name):
    if name in ("scores", "topk", "topk_noalloc", "topk_pruned", "project", "sparse_mla", "workspace_bytes", "IndexerError",
                "load"):
        from . import _lib

        return getattr(_lib, name)
    raise AttributeError(name)
