"""Float64 reference of DoSA's certified pruning for the indexer Top-K.

TEST INFRASTRUCTURE ONLY.

Sources:
* DoSA reading notes (notes.kuangjux.top, "DoSA: Dots Sparse Attention"),
  annotation LBKERZAW, the three-step prefill flow (paper sections 2.2-2.4):
  1. seeds: at least K distinct visible keys, scored with all heads; tau is
     their K-th highest score, which cannot exceed the true K-th score;
  2. bound: exact retained-head terms, plus an upper bound on the omitted
     positive-weight heads (projection onto the retained heads plus a
     residual term prepared per query), minus a lower bound on the omitted
     negative-weight heads' penalty (their queries folded by |w| into one
     vector, then a single ReLU, which never exceeds the sum of ReLUs);
     a key is excluded only if its bound is strictly below tau;
  3. survivors are scored with all heads, those below tau are dropped, the
     rest merge with the seed Top-K and the final K is chosen by exact score.
* 机器之心 article on DoSA (163.com), section 03: the same two quantities
  (threshold lower bound, per-candidate upper bound) and strict exclusion.

The bound here is written term by term in that order.  The GPU evaluates a
folded form of it (``bound_from_plan``): per retained head one coefficient of
|d_i| plus one "linear" row E, which equals the term-by-term form when the
plan is folded from the same projection (a_i ReLU(d) + b_i ReLU(-d) =
(a_i + b_i)/2 |d| + (a_i - b_i)/2 d), while the GPU's own plans also carry
rounding margins (rows stored in the input dtype, a guard on |k|) and fit
the projection differently (nonnegative coefficients).  ``bound_from_plan``
recomputes in float64 the bound of any such plan, so that a plan the GPU
exports can be checked against the exact scores.
"""
from __future__ import annotations

import numpy as np

from .indexer import index_score_row, topk_row


def seed_threshold(seed_scores: np.ndarray, k: int) -> float:
    """tau = K-th highest full score among the seeds (-inf if fewer than K seeds)."""
    s = np.asarray(seed_scores, np.float64)
    if s.size < k:
        return -np.inf
    return float(np.sort(s)[::-1][k - 1])


def project_positive_heads(q_row: np.ndarray, retained: np.ndarray, positive: np.ndarray):
    """Least-squares coefficients C [|P|, |R|] and residuals r_j = q_j - C_j Q_R.

    Any C gives a valid bound; least squares makes the residuals small.
    """
    QR = np.asarray(q_row, np.float64)[retained]  # [|R|, d]
    QP = np.asarray(q_row, np.float64)[positive]  # [|P|, d]
    if len(positive) == 0 or len(retained) == 0:
        C = np.zeros((len(positive), len(retained)))
    else:
        C = np.linalg.lstsq(QR.T, QP.T, rcond=None)[0].T  # [|P|, |R|]
    resid = QP - C @ QR
    return C, resid


def upper_bound(
    q_row: np.ndarray,
    w_row: np.ndarray,
    keys: np.ndarray,
    retained,
    neg_fold=None,
) -> np.ndarray:
    """Certified upper bound U(s) >= I(s) for every key row in ``keys``.

    q_row [H, d], w_row [H], keys [n, d]; ``retained`` is the set R of heads
    scored exactly; ``neg_fold`` is the subset N' of omitted negative-weight
    heads folded into the penalty (default: all of them).
    """
    q = np.asarray(q_row, np.float64)
    w = np.asarray(w_row, np.float64)
    K = np.asarray(keys, np.float64)
    H = q.shape[0]
    R = np.asarray(sorted(set(int(i) for i in retained)), dtype=np.int64)
    omitted = np.setdiff1d(np.arange(H), R)
    P = omitted[w[omitted] > 0]
    Nn = omitted[w[omitted] < 0]
    Nf = Nn if neg_fold is None else np.asarray(sorted(set(int(j) for j in neg_fold)), dtype=np.int64)
    if not set(Nf.tolist()) <= set(Nn.tolist()):
        raise ValueError("the folded set must hold only omitted negative-weight heads")
    knorm = np.linalg.norm(K, axis=1)

    # retained heads, exact
    d = q[R] @ K.T  # [|R|, n]
    retained_term = w[R] @ np.maximum(d, 0.0)

    # omitted positive heads: q_j = sum_i C_ji q_i + r_j, and
    # ReLU(a + b) <= ReLU(a) + ReLU(b), ReLU(c x) = c ReLU(x) (c >= 0),
    # r_j . k <= |r_j| |k|.
    C, resid = project_positive_heads(q, R, P)
    Cp, Cm = np.maximum(C, 0.0), np.maximum(-C, 0.0)
    per_head = Cp @ np.maximum(d, 0.0) + Cm @ np.maximum(-d, 0.0)  # [|P|, n]
    per_head = per_head + np.linalg.norm(resid, axis=1)[:, None] * knorm[None, :]
    positive_term = w[P] @ per_head

    # omitted negative heads: sum_j |w_j| ReLU(x_j) >= ReLU(sum_{j in N'} |w_j| x_j)
    q_neg = np.abs(w[Nf]) @ q[Nf] if Nf.size else np.zeros(q.shape[1])
    penalty = np.maximum(K @ q_neg, 0.0)

    return retained_term + positive_term - penalty


def pruned_topk_row(
    q_row: np.ndarray,
    w_row: np.ndarray,
    keys_visible: np.ndarray,
    k: int,
    seeds: np.ndarray,
    retained,
    neg_fold=None,
):
    """The whole DoSA flow for one query row, in float64.

    Returns (selected indices, tau, survivor mask over non-seed keys).
    The selection equals ``topk_row`` of all visible scores; that identity is
    what the pruning must preserve.
    """
    n = keys_visible.shape[0]
    seeds = np.asarray(seeds, np.int64)
    seeds = seeds[seeds < n]
    seed_scores = index_score_row(q_row, keys_visible[seeds], w_row)
    tau = seed_threshold(seed_scores, k)
    seed_keep = seeds[topk_row(seed_scores, k)]

    rest = np.setdiff1d(np.arange(n), seeds)
    U = upper_bound(q_row, w_row, keys_visible[rest], retained, neg_fold)
    survive = U >= tau  # exclude only when strictly below
    cand = rest[survive]
    exact = index_score_row(q_row, keys_visible[cand], w_row)
    kept = cand[exact >= tau]

    pool = np.concatenate([seed_keep, kept])
    pool_scores = index_score_row(q_row, keys_visible[pool], w_row)
    order = np.lexsort((pool, -pool_scores))
    return pool[order[: min(int(k), n)]], tau, survive


def bound_from_plan(rows, coef, kappa: float, e_neg: float, keys, scale=None) -> np.ndarray:
    """The bound of a folded plan, in float64, for every key row in ``keys``.

    rows [32, d]: rows 0..29 the |d| rows (the retained heads' query rows,
    zero rows for unused slots, and any other row whose |dot| the plan
    adds, such as the low part of a row split in two), row 30 the folded
    negative-head row q_neg, row 31 the linear row E; coef [32]:
    c_0..c_29, the q_neg multiplier c_30, the E multiplier c_31; kappa,
    e_neg: the |k| coefficients of the residual (and any guard) and of
    q_neg's rounding.  With d_i = rows[i] . k,

        U = sum_{i<30} c_i |d_i| + c_31 d_31 - ReLU(c_30 d_30 - e_neg |k|) + kappa |k|,

    times ``scale`` (fp8: q_scale * k_scale per key) when given.  All values
    are in the units the plan was built in (fp8 code units for fp8 inputs).
    """
    R = np.asarray(rows, np.float64)
    c = np.asarray(coef, np.float64)
    K = np.asarray(keys, np.float64)
    d = R @ K.T  # [32, n]
    kn = np.linalg.norm(K, axis=1)
    U = c[:30] @ np.abs(d[:30]) + c[31] * d[31] - np.maximum(c[30] * d[30] - float(e_neg) * kn, 0.0) + float(kappa) * kn
    return U if scale is None else np.asarray(scale, np.float64) * U
