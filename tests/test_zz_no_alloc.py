"""The no-allocation Top-K entry point (dsa_indexer_topk_noalloc) against
dsa_indexer_topk on the same inputs: two calls in a row on one GPU, the
second smaller, each with identical index sets and scores, on both routes."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import call_args, log, need_gpu, to_device

pytestmark = pytest.mark.gpu


def _same(a, b):
    ia, sa = (x.cpu().numpy() for x in a)
    ib, sb = (x.cpu().numpy() for x in b)
    oa, ob = np.argsort(ia, -1), np.argsort(ib, -1)
    assert np.array_equal(np.take_along_axis(ia, oa, -1), np.take_along_axis(ib, ob, -1))
    assert np.array_equal(np.take_along_axis(sa, oa, -1), np.take_along_axis(sb, ob, -1))


@pytest.mark.parametrize("route", ["split", "stream"])
def test_noalloc_matches_topk_twice(route):
    need_gpu()
    cases = [(2, 24, 6000, 512, "bf16", "clustered"), (1, 9, 1500, 64, "fp8", "iid")]  # second call smaller
    for i, (B, Q, N, k, dtype, dist) in enumerate(cases):
        rng = np.random.default_rng(70 + i)
        pos = rng.integers(N // 3, N, size=(B, Q))
        pos[0, -1] = N - 1
        d = inputs.make_inputs(B, Q, N, dtype, dist, seed=70 + i, positions=pos)
        dd = to_device(d)
        args, kw = call_args(dd)
        log(f"noalloc {route} call {i}: B={B} Q={Q} N={N} k={k} {dtype}")
        ref = dsa.topk(*args, k, **kw, route=route)
        got = dsa.topk_noalloc(*args, k, **kw, route=route)
        torch.cuda.synchronize()
        _same(ref, got)
