"""GPU parity of the sparse MLA core attention (dsa_sparse_mla).

The GPU computes scores in fp32 (exact bf16 products), the softmax weights in
fp32, then rounds the weights to bf16 for the weighted sum (fp32 sums) and
the output to bf16.  Against the float64 oracle on the same bf16 inputs:

  |Z - Z_ref| <= 2^-7 * sum_i P_i |v_i| + 2^-8 |Z_ref| + 1e-6
      (bf16 weights: 2^-9 relative each; weights normalised by the fp32 sum of
       the unrounded ones; fp32 score error up to gamma_576 * sum|q_d k_d|,
       a few 1e-5 here; bf16 output: 2^-9 |Z|; the bound doubles the sum)
  |lse - lse_ref| <= 1e-4 * (1 + |lse_ref|) + sm_scale * gamma_576 * max_i sum_d |q_d k_d|
"""
import math

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import log, need_gpu
from oracle import indexer, sparse_mla

pytestmark = pytest.mark.gpu

G576 = 576 * 2.0**-24 / (1 - 576 * 2.0**-24)


def _dec(t):
    return indexer.decode_bf16(inputs.to_bits(t.cpu()))


def _check_rows(q_cpu, kv_cpu, idx, out, lse, sm_scale, rows):
    """q_cpu [B,Q,128,576] / kv_cpu [B,N,576] bf16 CPU tensors; idx numpy."""
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for b, t in rows:
        qf = _dec(q_cpu[b, t])
        kvf = _dec(kv_cpu[b])
        z, l_ref = sparse_mla.sparse_mla_row(qf, kvf, idx[b, t], sm_scale)
        bound = sparse_mla.value_abs_bound_row(qf, kvf, idx[b, t], sm_scale)
        tol = 2.0**-7 * bound + 2.0**-8 * np.abs(z) + 1e-6
        err = np.abs(out[b, t] - z)
        bad = np.argwhere(err > tol)
        assert bad.size == 0, f"row ({b},{t}): {bad.shape[0]} outputs off, first {bad[:3].tolist()}"
        sel = idx[b, t][(idx[b, t] >= 0) & (idx[b, t] < kvf.shape[0])]
        if sel.size == 0:
            assert np.all(np.isneginf(lse[b, t])) and np.all(out[b, t] == 0)
            continue
        smax = (np.abs(qf) @ np.abs(kvf[sel]).T).max()
        ltol = 1e-4 * (1 + np.abs(l_ref)) + sm_scale * G576 * smax
        assert np.all(np.abs(lse[b, t] - l_ref) <= ltol), (b, t, float(np.abs(lse[b, t] - l_ref).max()))


def _run(d, idx_np, sm_scale, num_splits=0):
    q, kv = d["q"].cuda(), d["kv"].cuda()
    idx = torch.from_numpy(idx_np).cuda()
    out, lse = dsa.sparse_mla(q, kv, idx, sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


# few rows split each row's tiles over several workgroups and merge the
# partial results; 1 pins the unsplit kernel, 0 lets the library choose
SPLITS = [1, 3, 0]


@pytest.mark.parametrize("split", SPLITS)
def test_small_rows_with_padding(split):
    need_gpu()
    B, Q, N, k = 2, 6, 300, 64
    d = inputs.make_mla_inputs(B, Q, N, seed=1)
    pos = np.array([[299, 40, 10, 0, -1, 63], [299, 299, 150, 31, 32, 100]])
    idx = inputs.random_selection(B, Q, N, k, pos, seed=1)
    idx[1, 2] = idx[1, 2][::-1].copy()  # padding first, then positions
    idx[1, 5, 10:20] = -1  # padding in the middle
    idx[1, 5, 3] = 400  # out of range: skipped
    log("[mla] small rows")
    out, lse = _run(d, idx, 1.0 / math.sqrt(576), split)
    _check_rows(d["q"], d["kv"], idx, out, lse, 1.0 / math.sqrt(576), [(b, t) for b in range(B) for t in range(Q)])


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("sm_scale", [1.0 / math.sqrt(576), 0.0, 0.2])
def test_full_topk_rows(sm_scale, split):
    need_gpu()
    B, Q, N, k = 1, 5, 5000, 2048
    d = inputs.make_mla_inputs(B, Q, N, seed=2)
    pos = np.array([[4999, 4999, 2047, 2048, 3000]])
    idx = inputs.random_selection(B, Q, N, k, pos, seed=2)
    log(f"[mla] topk 2048, sm_scale {sm_scale}")
    out, lse = _run(d, idx, sm_scale, split)
    _check_rows(d["q"], d["kv"], idx, out, lse, sm_scale, [(0, t) for t in range(Q)])


@pytest.mark.parametrize("split", SPLITS)
def test_second_pass_rows(split):
    """Rows whose later scores exceed the first tile's maximum by far more
    than 32 (log2 units) are recomputed by the second launch: the first 32
    selected positions get tiny latent rows, the rest full ones, and a large
    sm_scale stretches the score range."""
    need_gpu()
    B, Q, N, k = 1, 4, 600, 256
    d = inputs.make_mla_inputs(B, Q, N, seed=3)
    d["kv"][0, :100] = (d["kv"][0, :100].float() * 0.01).to(torch.bfloat16)
    idx = np.full((B, Q, k), -1, dtype=np.int32)
    rng = np.random.default_rng(3)
    for t in range(Q):
        idx[0, t, :32] = rng.choice(100, 32, replace=False)
        idx[0, t, 32:200] = 100 + rng.choice(500, 168, replace=False)
    sm_scale = 0.5
    qf, kvf = _dec(d["q"][0, 0]), _dec(d["kv"][0])
    s = sm_scale * (qf @ kvf[idx[0, 0, :200]].T) / math.log(2)
    assert (s[:, 32:].max(1) - s[:, :32].max(1)).max() > 40  # the retry path is taken
    log("[mla] second pass")
    out, lse = _run(d, idx, sm_scale, split)
    _check_rows(d["q"], d["kv"], idx, out, lse, sm_scale, [(0, t) for t in range(Q)])


def test_consumes_the_topk_output():
    """Indices straight from dsa_indexer_topk (valid first, -1 padding for
    rows that see fewer than k keys)."""
    need_gpu()
    ind = inputs.make_inputs(1, 40, 700, "bf16", "iid", pos_start=0, seed=4)  # rows see 1..40 keys
    k = 32
    idx, _ = dsa.topk(ind["q"].cuda(), ind["k"].cuda(), ind["w"].cuda(), ind["pos"].cuda(), k)
    d = inputs.make_mla_inputs(1, 40, 700, seed=4)
    out, lse = dsa.sparse_mla(d["q"].cuda(), d["kv"].cuda(), idx, 1.0 / math.sqrt(576))
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    assert (idx_np[0, 0] >= 0).sum() == 1 and (idx_np[0, 39] >= 0).sum() == 32
    _check_rows(d["q"], d["kv"], idx_np, out, lse, 1.0 / math.sqrt(576), [(0, t) for t in (0, 1, 17, 31, 32, 39)])


def test_paged_cache_matches_flat_bit_for_bit():
    """The same cache stored as shuffled pages of a pool behind a page table
    gives bit-identical outputs (the gather resolves each position to the
    same row), including positions in a partial last page."""
    need_gpu()
    B, Q, N, k, P = 2, 6, 1000, 256, 64
    d = inputs.make_mla_inputs(B, Q, N, seed=6)
    pos = np.array([[999, 998, 500, 63, 64, 0], [999, 640, 639, 1, 200, 999]])
    idx = inputs.random_selection(B, Q, N, k, pos, seed=6)
    pps = (N + P - 1) // P  # 16 pages per sequence, the last one partial
    num_pages = B * pps + 5
    rng = np.random.default_rng(6)
    phys = rng.permutation(num_pages)[: B * pps].reshape(B, pps).astype(np.int32)
    pool = torch.zeros((num_pages, P, 576), dtype=torch.bfloat16)
    for b in range(B):
        for j in range(pps):
            n = min(P, N - j * P)
            pool[phys[b, j], :n] = d["kv"][b, j * P:j * P + n]
    q = d["q"].cuda()
    idx_t = torch.from_numpy(idx).cuda()
    flat, lflat = dsa.sparse_mla(q, d["kv"].cuda(), idx_t, 1.0 / math.sqrt(576))
    paged, lpaged = dsa.sparse_mla(q, pool.cuda(), idx_t, 1.0 / math.sqrt(576), page_table=torch.from_numpy(phys).cuda(),
                                   num_k=N)
    torch.cuda.synchronize()
    assert torch.equal(flat.view(torch.int16), paged.view(torch.int16))
    assert torch.equal(lflat.view(torch.int32), lpaged.view(torch.int32))
    _check_rows(d["q"], d["kv"], idx, paged, lpaged, 1.0 / math.sqrt(576), [(0, 0), (0, 3), (1, 1), (1, 3)])


def test_decode_rows_split_and_merged():
    """Decode shape: one query row per sequence, 8 sequences, top-2048 of
    6000 keys each; the automatic split (8 ranges of a row's 64 tiles) and the
    unsplit kernel both match the oracle."""
    need_gpu()
    B, Q, N, k = 8, 1, 6000, 2048
    d = inputs.make_mla_inputs(B, Q, N, seed=8)
    pos = np.full((B, Q), N - 1)
    pos[3, 0] = 1000  # fewer visible keys than k: a shorter selection
    idx = inputs.random_selection(B, Q, N, k, pos, seed=8)
    res = {}
    for split in (0, 1):
        res[split] = _run(d, idx, 1.0 / math.sqrt(576), split)
    for out, lse in res.values():
        _check_rows(d["q"], d["kv"], idx, out, lse, 1.0 / math.sqrt(576), [(b, 0) for b in range(B)])


def test_fullsize_block_sampled_rows():
    """The 128K chunked-prefill block as the benchmark runs it: 8192 rows,
    each with the 2048 positions the indexer selects among 131072 keys;
    sampled rows against the oracle."""
    need_gpu()
    wl = inputs.WORKLOADS["chunked_prefill_128k"]
    d = inputs.make_workload(wl)
    idx, _ = dsa.topk(d["q"].cuda(), d["k"].cuda(), d["w"].cuda(), d["pos"].cuda(), wl.topk, return_scores=False)
    del d
    md = inputs.make_mla_inputs(wl.batch, wl.num_q, wl.num_k, seed=0, device="cuda")
    log("[mla] full-size block")
    out, lse = dsa.sparse_mla(md["q"], md["kv"], idx, 1.0 / math.sqrt(576))
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    assert np.all((idx_np >= 0).sum(-1) == wl.topk)
    rng = np.random.default_rng(0)
    rows = [0, wl.num_q - 1] + list(rng.choice(wl.num_q, 4, replace=False))
    q_cpu = md["q"][0, rows].cpu()[None]
    kv_cpu = md["kv"].cpu()
    sub = idx_np[:, rows]
    _check_rows(q_cpu, kv_cpu, sub, out[:, rows], lse[:, rows], 1.0 / math.sqrt(576),
                [(0, i) for i in range(len(rows))])
