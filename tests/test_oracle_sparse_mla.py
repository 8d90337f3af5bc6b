"""Pins of the sparse MLA oracle (oracle.sparse_mla).

Checks that rest on facts other than the oracle's formula: a hand-worked
two-position example, closed forms for one selected position, for identical
rows and for sm_scale = 0, the split into content and RoPE scores, padding and
order invariance, convexity of the weighted value, a library softmax
(torch.softmax) in a special case, and the pages' printed FLOP count.
"""
import math

import numpy as np
import pytest
import torch

from oracle import counts, sparse_mla


def test_hand_worked_two_positions():
    # h = 1, d_c = 2, d_r = 1.  q = [1, 0 | 1]; rows kv0 = [1, 2 | 0], kv1 = [0, 5 | 1].
    # scores: s0 = 1*1 + 0*2 + 1*0 = 1, s1 = 1*0 + 0*5 + 1*1 = 1 -> equal weights 1/2:
    # Z = [(1 + 0)/2, (2 + 5)/2] = [0.5, 3.5], lse = 1 + ln 2.
    q = np.array([[1.0, 0.0, 1.0]])
    kv = np.array([[1.0, 2.0, 0.0], [0.0, 5.0, 1.0], [9.0, 9.0, 9.0]])
    z, lse = sparse_mla.sparse_mla_row(q, kv, np.array([0, 1, -1]), 1.0, d_c=2)
    np.testing.assert_allclose(z, [[0.5, 3.5]], rtol=1e-15)
    np.testing.assert_allclose(lse, [1.0 + math.log(2.0)], rtol=1e-15)
    # sm_scale 2 with kv1's rope raised to 2: s0 = 2*1 = 2, s1 = 2*(0 + 2) = 4
    kv[1, 2] = 2.0
    z, lse = sparse_mla.sparse_mla_row(q, kv, np.array([0, 1]), 2.0, d_c=2)
    p1 = math.exp(4) / (math.exp(2) + math.exp(4))
    np.testing.assert_allclose(z, [[(1 - p1) * 1.0, (1 - p1) * 2.0 + p1 * 5.0]], rtol=1e-14)
    np.testing.assert_allclose(lse, [math.log(math.exp(2) + math.exp(4))], rtol=1e-14)


def _rand(h=8, n=50, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((h, sparse_mla.D_C + sparse_mla.D_R)), rng.standard_normal(
        (n, sparse_mla.D_C + sparse_mla.D_R))


def test_single_position_returns_its_latent_row():
    q, kv = _rand()
    z, lse = sparse_mla.sparse_mla_row(q, kv, np.array([-1, 17, -1]), 0.3)
    np.testing.assert_array_equal(z, np.tile(kv[17, :512], (8, 1)))
    np.testing.assert_allclose(lse, 0.3 * (q @ kv[17]), rtol=1e-13)


def test_identical_rows_and_zero_scale():
    q, kv = _rand()
    kv[5:9] = kv[5]
    z, lse = sparse_mla.sparse_mla_row(q, kv, np.array([5, 6, 7, 8]), 0.7)
    np.testing.assert_allclose(z, np.tile(kv[5, :512], (8, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse, 0.7 * (q @ kv[5]) + math.log(4), rtol=1e-13)
    # sm_scale = 0: uniform weights, Z = mean of the selected latent rows, lse = ln m
    _, kv2 = _rand(seed=1)
    sel = np.array([3, 10, 11, 40, 2])
    z, lse = sparse_mla.sparse_mla_row(q, kv2, sel, 0.0)
    np.testing.assert_allclose(z, np.tile(kv2[sel, :512].mean(0), (8, 1)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(5), rtol=1e-14)


def test_content_and_rope_scores_add():
    # a query with zero content part scores by the RoPE part only, and vice versa
    q, kv = _rand()
    sel = np.arange(0, 50, 3)
    q_r = q.copy()
    q_r[:, :512] = 0
    _, lse_r = sparse_mla.sparse_mla_row(q_r, kv, sel, 0.5)
    s_r = 0.5 * q[:, 512:] @ kv[sel, 512:].T
    np.testing.assert_allclose(lse_r, np.log(np.exp(s_r).sum(1)), rtol=1e-13)
    q_a = q.copy()
    q_a[:, 512:] = 0
    _, lse_a = sparse_mla.sparse_mla_row(q_a, kv, sel, 0.5)
    s_a = 0.5 * q[:, :512] @ kv[sel, :512].T
    np.testing.assert_allclose(lse_a, np.log(np.exp(s_a).sum(1)), rtol=1e-13)


def test_matches_torch_softmax_attention():
    # with one head and no RoPE part, Z is softmax(scale * q K^T) V over the selected rows
    q, kv = _rand(h=3, n=64, seed=4)
    q[:, 512:] = 0
    sel = np.array([9, 1, 33, 60, 12, 5, 47])
    z, _ = sparse_mla.sparse_mla_row(q, kv, sel, 0.05)
    qt, kt = torch.from_numpy(q[:, :512]), torch.from_numpy(kv[sel, :512])
    ref = torch.softmax(0.05 * qt @ kt.T, dim=-1) @ kt
    np.testing.assert_allclose(z, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_padding_order_and_convexity():
    q, kv = _rand(seed=2)
    sel = np.array([4, 9, 30, 31, 0, 49])
    z, lse = sparse_mla.sparse_mla_row(q, kv, sel, 0.2)
    z2, lse2 = sparse_mla.sparse_mla_row(q, kv, np.concatenate([[-1], sel[::-1], [-1, -1]]), 0.2)
    np.testing.assert_allclose(z, z2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14)
    lo, hi = kv[sel, :512].min(0), kv[sel, :512].max(0)
    assert np.all(z >= lo - 1e-12) and np.all(z <= hi + 1e-12)
    b = sparse_mla.value_abs_bound_row(q, kv, sel, 0.2)
    assert np.all(np.abs(z) <= b + 1e-12)


def test_empty_selection_and_out_of_range_entries():
    q, kv = _rand()
    z, lse = sparse_mla.sparse_mla_row(q, kv, np.array([-1, -1, 50, 99]), 1.0)  # kv has 50 rows
    assert np.all(z == 0) and np.all(np.isneginf(lse))
    z1, l1 = sparse_mla.sparse_mla_row(q, kv, np.array([7, 50, 3]), 0.3)
    z2, l2 = sparse_mla.sparse_mla_row(q, kv, np.array([7, 3]), 0.3)
    np.testing.assert_array_equal(z1, z2)
    np.testing.assert_array_equal(l1, l2)


def test_flops_per_pair_printed():
    # the FLOPs notes print 2h(2d_c + d_r) = 278,528 FLOPs per selected pair
    assert counts.core_flops_per_pair() == 278528
    assert 2 * 128 * (2 * sparse_mla.D_C + sparse_mla.D_R) == 278528
