"""Closed forms printed in the DeepSeek DSA FLOPs notes.

TEST INFRASTRUCTURE ONLY.

Convention (section "Notation"): a multiply-add is 2 FLOPs and only matrix
products are counted; ReLU, head weights, the head sum and Top-K selection
are not.
"""
from __future__ import annotations

# DeepSeek-V3.2 sizes from the notation table of the same notes.
V32 = dict(d=7168, h=128, d_c=512, d_r=64, d_qc=1536, H_I=64, d_I=128, k=2048)


def n_dense(T: int) -> int:
    """Visible causal query-key pairs, diagonal included ("Causal token-pair 数")."""
    return T * (T + 1) // 2


def n_sel(T: int, k: int) -> int:
    """sum over the T queries of min(k, s), s = 1..T (the N_sel equation)."""
    if T <= k:
        return T * (T + 1) // 2
    return k * T - k * (k - 1) // 2


def n_sel_brute(T: int, k: int) -> int:
    return sum(min(k, s) for s in range(1, T + 1))


def indexer_score_flops_causal(T: int, H: int = 64, d: int = 128) -> int:
    """Causal full-prefix scoring: H^I d^I T (T+1) ("Full-prefix index scoring")."""
    return H * d * T * (T + 1)


def indexer_score_flops_square(T: int, H: int = 64, d: int = 128) -> int:
    """Square (masked) scoring: 2 H^I T^2 d^I."""
    return 2 * H * T * T * d


def indexer_proj_flops(T: int, c=V32) -> int:
    """The three indexer projections: 2T(d_qc H^I d^I + d d^I + d H^I)."""
    return 2 * T * (c["d_qc"] * c["H_I"] * c["d_I"] + c["d"] * c["d_I"] + c["d"] * c["H_I"])


def indexer_prefill_flops(T: int, c=V32) -> int:
    return indexer_proj_flops(T, c) + indexer_score_flops_causal(T, c["H_I"], c["d_I"])


def indexer_decode_flops(t: int, c=V32) -> int:
    """One decode token against a key cache of length t (section "Decode")."""
    return indexer_proj_flops(1, c) + 2 * c["H_I"] * t * c["d_I"]


def core_flops_per_pair(c=V32) -> int:
    """Sparse MLA core attention per selected pair: 2h(2d_c + d_r)."""
    return 2 * c["h"] * (2 * c["d_c"] + c["d_r"])


def core_prefill_flops(T: int, c=V32) -> int:
    return core_flops_per_pair(c) * n_sel(T, c["k"])


def core_decode_flops(t: int, c=V32) -> int:
    return core_flops_per_pair(c) * min(c["k"], t)


def pair_flops(H: int = 64, d: int = 128) -> int:
    """Matrix-product FLOPs per scored (query, key) pair: 2 H^I d^I."""
    return 2 * H * d
