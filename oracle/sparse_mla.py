"""Float64 reference of the sparse MLA core attention over the selected keys.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this.

Source: DeepSeek DSA FLOPs notes, section "Core Sparse Attention FLOPs".
The core attention runs in MLA's MQA mode: every query head reads the same
latent cache C^KV and RoPE key K^R of a position.  For query s with selected
set S_s (the indexer's Top-K, m_s = min(k, s) positions):

* content score  S^A = Q^A (h, d_c) x (C^KV_S)^T (d_c, m)       ("Attention score")
* RoPE score     S^R = Q^R (h, d_r) x (K^R_S)^T  (d_r, m)
* the two are added and a softmax over the m selected positions gives P (h, m)
* weighted latent value  Z = P (h, m) x C^KV_S (m, d_c)          ("Weighted latent value")

Readings (the notes leave these open):
* a query row is stored as [Q^A | Q^R] (d_c + d_r values per head) and a
  cache row as [C^KV | K^R], so S^A + S^R is one dot product of length
  d_c + d_r;
* the softmax is taken of sm_scale * (S^A + S^R) for a caller-given
  sm_scale > 0 (the notes' formula is sm_scale = 1; the benchmark uses
  1/sqrt(d_c + d_r), the usual scaled-dot-product factor for that length);
* the selected set is the index list as given: entries outside 0..N-1
  (the Top-K's -1 padding) are skipped, the others are used as they stand
  (a repeated entry counts twice); a row with no selected position outputs
  Z = 0 and log-sum-exp -inf;
* besides Z the call reports lse = log(sum_i exp(sm_scale * s_i)), natural log.
"""
from __future__ import annotations

import numpy as np

D_C = 512
D_R = 64


def sparse_mla_row(q_row: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float, d_c: int = D_C):
    """One query row.  q_row [h, d_c + d_r], kv [N, d_c + d_r] (float64),
    idx [k] int.  Returns (Z [h, d_c], lse [h])."""
    q_row = np.asarray(q_row, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    idx = np.asarray(idx)
    h = q_row.shape[0]
    sel = idx[(idx >= 0) & (idx < kv.shape[0])]
    if sel.size == 0:
        return np.zeros((h, d_c)), np.full(h, -np.inf)
    rows = kv[sel]  # (m, d_c + d_r)
    s_a = q_row[:, :d_c] @ rows[:, :d_c].T  # content score (h, m)
    s_r = q_row[:, d_c:] @ rows[:, d_c:].T  # RoPE score (h, m)
    s = sm_scale * (s_a + s_r)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    z = p @ rows[:, :d_c]
    lse = (mx + np.log(l))[:, 0]
    return z, lse


def value_abs_bound_row(q_row: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float, d_c: int = D_C):
    """sum_i P[h,i] |C^KV[s_i, :]| per head and dimension: the scale of the
    error of Z when each weight P carries a small relative error."""
    q_row = np.asarray(q_row, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    idx = np.asarray(idx)
    sel = idx[(idx >= 0) & (idx < kv.shape[0])]
    h = q_row.shape[0]
    if sel.size == 0:
        return np.zeros((h, d_c))
    rows = kv[sel]
    s = sm_scale * (q_row @ rows.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return p @ np.abs(rows[:, :d_c])
