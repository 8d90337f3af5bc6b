"""Pins of the float64 pruning reference (seed threshold and upper bound).

The facts pinned: the seed threshold never exceeds the true K-th score; the
bound never falls below the true score, on random, clustered and adversarial
rows; with every head retained the bound is the score itself; the whole
seed -> bound -> refine -> merge flow returns the plain Top-K; and a planted
mistake (the residual term dropped) is caught by the same checks.
"""
import numpy as np
import pytest

from dsa_lightning_indexer_04_amd import inputs
from oracle import indexer, prune


def _row(seed, dist="iid", n=600):
    d = inputs.make_inputs(1, 1, n, "bf16", dist, pos_start=n - 1, seed=seed)
    qf, kf = indexer.dequantize(inputs.to_bits(d["q"]), inputs.to_bits(d["k"]), "bf16")
    return qf[0, 0], kf[0], d["w"].numpy()[0, 0].astype(np.float64)


def test_relu_fold_inequality():
    # ReLU(sum_j a_j x_j) <= sum_j a_j ReLU(x_j) for a_j >= 0 (the folded penalty)
    rng = np.random.default_rng(0)
    for _ in range(200):
        a = rng.random(7) * 3
        x = rng.standard_normal(7)
        assert max(a @ x, 0) <= a @ np.maximum(x, 0) + 1e-15


@pytest.mark.parametrize("seed", range(4))
def test_seed_threshold_below_true_kth(seed):
    q, K, w = _row(seed, "clustered")
    s = indexer.index_score_row(q, K, w)
    rng = np.random.default_rng(seed)
    k = 50
    for ns in (50, 120, 400):
        seeds = np.sort(rng.choice(K.shape[0], ns, replace=False))
        tau = prune.seed_threshold(s[seeds], k)
        assert tau <= indexer.kth_score(s, k)


def test_seeds_equal_all_keys_gives_exact_kth():
    q, K, w = _row(11)
    s = indexer.index_score_row(q, K, w)
    tau = prune.seed_threshold(s, 64)
    assert tau == indexer.kth_score(s, 64)
    assert prune.seed_threshold(s[:10], 64) == -np.inf


@pytest.mark.parametrize("dist", ["iid", "clustered"])
@pytest.mark.parametrize("nret", [0, 1, 8, 16, 40])
def test_upper_bound_dominates_score(dist, nret):
    rng = np.random.default_rng(nret + (100 if dist == "clustered" else 0))
    for seed in range(3):
        q, K, w = _row(seed + 20, dist)
        R = rng.choice(64, nret, replace=False)
        I = indexer.index_score_row(q, K, w)
        U = prune.upper_bound(q, w, K, R)
        scale = np.abs(w) @ np.linalg.norm(q, axis=1) * np.linalg.norm(K, axis=1)
        assert np.all(U >= I - 1e-12 * scale)
        # a random subset of the negative heads folded is still a valid bound
        omitted = np.setdiff1d(np.arange(64), R)
        neg = omitted[w[omitted] < 0]
        sub = neg[rng.random(neg.size) < 0.5]
        U2 = prune.upper_bound(q, w, K, R, neg_fold=sub)
        assert np.all(U2 >= I - 1e-12 * scale)


def test_upper_bound_adversarial_rows():
    rng = np.random.default_rng(9)
    d = 128
    K = np.concatenate([rng.standard_normal((200, d)), np.zeros((2, d)), 1e6 * rng.standard_normal((3, d))])
    base = rng.standard_normal((4, d))
    # collinear retained heads and heads that are exact combinations of them
    q = np.concatenate([base, base[:1] * 2.0, base[:2].sum(0, keepdims=True), rng.standard_normal((58, d))])
    for w in (rng.standard_normal(64), -np.abs(rng.standard_normal(64)), np.abs(rng.standard_normal(64))):
        I = indexer.index_score_row(q, K, w)
        for R in ([0, 4, 5], [0, 1, 2, 3], list(range(64))[::3], []):
            U = prune.upper_bound(q, w, K, R)
            scale = np.abs(w) @ np.linalg.norm(q, axis=1) * np.linalg.norm(K, axis=1)
            assert np.all(U >= I - 1e-12 * (scale + 1))
    # zero keys: score and bound are both 0
    assert np.all(prune.upper_bound(q, w, np.zeros((3, d)), [0, 1]) == 0)


def test_all_heads_retained_bound_is_score():
    q, K, w = _row(3)
    I = indexer.index_score_row(q, K, w)
    U = prune.upper_bound(q, w, K, np.arange(64))
    np.testing.assert_allclose(U, I, rtol=1e-12, atol=1e-12)


def test_dropping_the_residual_breaks_the_bound(monkeypatch):
    # plant a mistake in the oracle (residual norms forced to zero) and check
    # that the dominance test above would catch it
    q, K, w = _row(5, "iid")
    I = indexer.index_score_row(q, K, w)
    R = np.arange(4)
    orig = prune.project_positive_heads

    def no_residual(q_row, retained, positive):
        C, r = orig(q_row, retained, positive)
        return C, np.zeros_like(r)

    monkeypatch.setattr(prune, "project_positive_heads", no_residual)
    U = prune.upper_bound(q, w, K, R)
    assert np.any(U < I - 1e-9)


@pytest.mark.parametrize("dist,nret", [("iid", 16), ("clustered", 16), ("clustered", 4), ("iid", 0)])
def test_pruned_flow_equals_plain_topk(dist, nret):
    q, K, w = _row(30 + nret, dist, n=2000)
    k = 64
    seeds = inputs.evenly_spaced_seeds(384, K.shape[0] - 1)
    R = np.argsort(-np.abs(w))[:nret]
    sel, tau, survive = prune.pruned_topk_row(q, w, K, k, seeds, R)
    ref = indexer.topk_row(indexer.index_score_row(q, K, w), k)
    assert sorted(sel.tolist()) == sorted(ref.tolist())
    assert tau <= indexer.kth_score(indexer.index_score_row(q, K, w), k)


def _folded_plan(q, w, R, Nf):
    """A plan folded from the term-by-term bound's own projection: rows = the
    retained query rows, q_neg = sum_{N'} |w_j| q_j, E = sum_i e_i q_i with
    a_i = w_i + sum_P w_j C_ji^+, b_i = sum_P w_j C_ji^-, c_i = (a_i + b_i)/2,
    e_i = (a_i - b_i)/2, kappa = rho = sum_P w_j |r_j|, e_neg = 0."""
    H = q.shape[0]
    omitted = np.setdiff1d(np.arange(H), R)
    P = omitted[w[omitted] > 0]
    C, resid = prune.project_positive_heads(q, R, P)
    a = w[R] + w[P] @ np.maximum(C, 0.0)
    b = w[P] @ np.maximum(-C, 0.0)
    rows = np.zeros((32, q.shape[1]))
    rows[: len(R)] = q[R]
    rows[30] = np.abs(w[Nf]) @ q[Nf]
    rows[31] = ((a - b) / 2) @ q[R]
    coef = np.zeros(32)
    coef[: len(R)] = (a + b) / 2
    coef[30] = coef[31] = 1.0
    rho = w[P] @ np.linalg.norm(resid, axis=1)
    return rows, coef, rho


@pytest.mark.parametrize("dist", ["iid", "clustered"])
@pytest.mark.parametrize("nret", [1, 12, 30])
def test_plan_form_equals_the_term_by_term_bound(dist, nret):
    """A plan folded from the same projection evaluates to the term-by-term
    bound (the GPU's folded form is that bound, not a different one), and
    dominates the exact scores; dropping the b_i half of the fold (a planted
    mistake) changes it."""
    q, K, w = _row(40 + nret, dist)
    pos = np.nonzero(w > 0)[0]
    R = pos[: min(nret, pos.size)]
    Nf = np.nonzero(w < 0)[0]
    rows, coef, rho = _folded_plan(q, w, R, Nf)
    Up = prune.bound_from_plan(rows, coef, rho, 0.0, K)
    Ut = prune.upper_bound(q, w, K, R, Nf)
    scale = np.abs(w) @ np.linalg.norm(q, axis=1) * np.linalg.norm(K, axis=1)
    assert np.allclose(Up, Ut, rtol=0, atol=1e-10 * scale.max())
    assert np.all(Up >= indexer.index_score_row(q, K, w) - 1e-10 * scale)
    # planted mistake: c_i = a_i / 2 (the ReLU(-d) half dropped)
    H = q.shape[0]
    omitted = np.setdiff1d(np.arange(H), R)
    P = omitted[w[omitted] > 0]
    C, _ = prune.project_positive_heads(q, R, P)
    if P.size and np.any(C < 0):
        bad = coef.copy()
        bad[: len(R)] = (w[R] + w[P] @ np.maximum(C, 0.0)) / 2
        assert not np.allclose(prune.bound_from_plan(rows, bad, rho, 0.0, K), Ut, rtol=0, atol=1e-10 * scale.max())


def test_plan_margins_keep_the_bound_valid():
    """Rounding the folded rows to bf16 and putting the rounding error on
    |k| (|E - E_bf16| into kappa, |q_neg - q_neg_bf16| into e_neg) keeps the
    plan's bound above every exact score."""
    q, K, w = _row(77, "clustered")
    R = np.nonzero(w > 0)[0][:20]
    Nf = np.nonzero(w < 0)[0]
    rows, coef, rho = _folded_plan(q, w, R, Nf)
    r16 = indexer.decode_bf16(inputs.to_bits(torch_bf16(rows)))
    e_lin = np.linalg.norm(rows[31] - r16[31]) * abs(coef[31])
    e_neg = np.linalg.norm(rows[30] - r16[30])
    Up = prune.bound_from_plan(r16, coef, rho + e_lin, e_neg, K)
    assert np.all(Up >= indexer.index_score_row(q, K, w) - 1e-9)


def torch_bf16(x):
    import torch

    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
