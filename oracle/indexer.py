"""Float64 reference of the lightning-indexer score and exact Top-K.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this.

Sources (the pages' own notation: query s, key r; here query t, key s):

* Index score -- DeepSeek DSA FLOPs notes, section "Lightning Indexer FLOPs",
  the displayed equation I_{s,r} = sum_j w_{s,j} ReLU(q_{s,j} . k_r): a signed
  weighted sum over the H^I indexer heads of the ReLU of each head's query
  dotted with the one key vector that all heads share (section "Notation",
  remark that K^I is shared by all heads).
* Visibility -- same notes, section "Causal token-pair 数": the causal count
  T(T+1)/2 includes the diagonal, so the query at absolute position p sees
  keys 0..p inclusive, and a query keeps at most min(k, visible) keys
  (the N_sel equation).
* Top-K -- the k highest index scores among the visible keys.  The pages fix
  no tie rule (the DoSA reading notes, annotation GAL4HV37, say ties need not
  match); this oracle breaks ties by the smaller key index, the total order
  the GPU path also uses.
* FP8 -- the FLOPs notes say the indexer runs in FP8 ("Lightning Indexer
  FLOPs", remark after the score equation).  Codes are OCP e4m3fn; values are
  decoded exactly from their bits here and multiplied by the per-row fp32
  scale in float64.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- decoding


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no infinities) codes -> float64, exactly.

    sign(1) | exponent(4, bias 7) | mantissa(3).  Exponent field 0 is
    subnormal: m * 2^-9.  Code S.1111.111 is NaN; every other code is finite,
    the largest being 1.75 * 2^8 = 448.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0**-9
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((b & 0x7) == 7), np.nan, val)
    return sign * val


def dequantize(q_bits, k_bits, dtype: str, q_scale=None, k_scale=None):
    """Exact float64 values of the indexer inputs.

    q_bits [..., H, d], k_bits [..., d].  For fp8 the per-row fp32 scales
    multiply every element of their row (q_scale indexes the query token,
    shared by all its heads; k_scale indexes the key row).
    """
    if dtype == "bf16":
        return decode_bf16(q_bits), decode_bf16(k_bits)
    if dtype == "fp8":
        qf = decode_e4m3fn(q_bits) * np.asarray(q_scale, dtype=np.float64)[..., None, None]
        kf = decode_e4m3fn(k_bits) * np.asarray(k_scale, dtype=np.float64)[..., None]
        return qf, kf
    raise ValueError(dtype)


# ---------------------------------------------------------------- score


def visible_count(pos, num_k: int) -> np.ndarray:
    """Number of keys the row at absolute position ``pos`` sees: keys 0..pos."""
    return np.clip(np.asarray(pos, dtype=np.int64) + 1, 0, int(num_k))


def index_score_row(q_row: np.ndarray, keys: np.ndarray, w_row: np.ndarray) -> np.ndarray:
    """I[s] = sum_j w_j * ReLU(q_j . k_s) for one query row, float64.

    q_row [H, d], keys [n, d], w_row [H]  ->  [n]
    """
    head_dots = np.asarray(q_row, np.float64) @ np.asarray(keys, np.float64).T  # [H, n]
    return np.asarray(w_row, np.float64) @ np.maximum(head_dots, 0.0)


def index_scores(qf: np.ndarray, kf: np.ndarray, w: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Full [B, Q, N] float64 score array, -inf where the key is not visible.

    qf [B,Q,H,d], kf [B,N,d], w [B,Q,H], pos [B,Q].  Small inputs only.
    """
    B, Q = qf.shape[:2]
    N = kf.shape[1]
    out = np.full((B, Q, N), -np.inf)
    vis = visible_count(pos, N)
    for b in range(B):
        for t in range(Q):
            v = int(vis[b, t])
            if v:
                out[b, t, :v] = index_score_row(qf[b, t], kf[b, :v], w[b, t])
    return out


# ---------------------------------------------------------------- fp32 error bound

U32 = 2.0**-24  # unit roundoff of fp32 (round to nearest)


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u): the relative error bound of n fp32 roundings
    in a sum or product chain (standard floating-point error analysis)."""
    return n * U32 / (1.0 - n * U32)


def score_error_bound_row(q_row: np.ndarray, keys: np.ndarray, w_row: np.ndarray, scale=None) -> np.ndarray:
    """Bound on |I_fp32 - I| for one query row, for any evaluation that forms
    each head's 128-term dot product and the 64-term weighted sum of ReLUs in
    fp32 arithmetic (any summation order), from exact products of the input
    values (bf16 x bf16 and e4m3 x e4m3 products are exact in fp32).

    q_row [H, d], keys [n, d] in the units the products are formed in (bf16
    values, or e4m3 code values for fp8), w_row [H].  ``scale`` (fp8 only):
    q_scale * k_scale per key ([n] or scalar), applied to the fp32 sum by two
    more roundings (the product of the scales, then the scaling).

    With x_j the exact head dots and X_j their fp32 values,
    |X_j - x_j| <= gamma_128 sum_d |q_jd k_d|; ReLU is 1-Lipschitz, so the
    weighted sum of the ReLUs moves by at most gamma_128 A,
    A = sum_j |w_j| sum_d |q_jd| |k_d|; its own fp32 evaluation adds at most
    gamma_64 (B + gamma_128 A), B = sum_j |w_j| ReLU(x_j).
    """
    q = np.asarray(q_row, np.float64)
    k = np.asarray(keys, np.float64)
    w = np.asarray(w_row, np.float64)
    A = (np.abs(w) @ np.abs(q)) @ np.abs(k).T  # [n]
    B = np.abs(w) @ np.maximum(q @ k.T, 0.0)  # [n]
    code = gamma(128) * A + gamma(64) * (B + gamma(128) * A)
    if scale is None:
        return code
    sc = np.asarray(scale, np.float64)
    exact = sc * (w @ np.maximum(q @ k.T, 0.0))
    return sc * code * (1.0 + gamma(2)) + gamma(2) * np.abs(exact)


# ---------------------------------------------------------------- Top-K


def topk_row(scores_visible: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, n) best keys: score descending, then index ascending."""
    s = np.asarray(scores_visible, np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    return order[: min(int(k), n)]


def kth_score(scores_visible: np.ndarray, k: int) -> float:
    """The K-th highest score of a row (the lowest score that Top-K keeps)."""
    sel = topk_row(scores_visible, k)
    return float(scores_visible[sel[-1]]) if sel.size else -np.inf


# ---------------------------------------------------------------- acceptance

BF16_TOL = (2e-3, 1e-3)  # (relative, absolute)
FP8_TOL = (3e-2, 1e-3)


def tolerance(dtype: str) -> tuple[float, float]:
    return BF16_TOL if dtype == "bf16" else FP8_TOL


def check_topk_row(
    gpu_idx: np.ndarray,
    oracle_scores: np.ndarray,
    k: int,
    rtol: float,
    atol: float,
    gpu_scores: np.ndarray | None = None,
) -> list[str]:
    """Acceptance of one GPU Top-K row against float64 oracle scores.

    ``oracle_scores`` are the row's visible scores (length = visible count).
    The GPU row must hold exactly min(k, visible) distinct visible indices
    followed by -1 padding; it must contain every key whose oracle score
    exceeds the K-th oracle score by more than the tolerance band and no key
    below it by more than the band.  Returned scores (if given) must match
    the oracle within the tolerance.  Returns a list of failure messages.
    """
    errs: list[str] = []
    n = oracle_scores.shape[0]
    want = min(int(k), n)
    g = np.asarray(gpu_idx, np.int64)
    valid, pad = g[:want], g[want:]
    if np.any(pad != -1):
        errs.append(f"padding not -1: {pad[pad != -1][:8]}")
    if np.any((valid < 0) | (valid >= n)):
        errs.append(f"indices out of visible range [0,{n}): {valid[(valid < 0) | (valid >= n)][:8]}")
        return errs
    if np.unique(valid).size != valid.size:
        errs.append("duplicate indices")
    if want == 0:
        return errs
    sK = kth_score(oracle_scores, k)
    band = atol + rtol * abs(sK)
    must_in = np.nonzero(oracle_scores > sK + band)[0]
    missing = np.setdiff1d(must_in, valid)
    if missing.size:
        errs.append(f"{missing.size} keys above K-th+band missing, e.g. {missing[:8]}")
    low = valid[oracle_scores[valid] < sK - band]
    if low.size:
        errs.append(f"{low.size} keys below K-th-band selected, e.g. {low[:8]}")
    if gpu_scores is not None:
        gs = np.asarray(gpu_scores, np.float64)[:want]
        ref = oracle_scores[valid]
        bad = np.abs(gs - ref) > atol + rtol * np.abs(ref)
        if np.any(bad):
            errs.append(f"{int(bad.sum())} returned scores off tolerance, worst |d|={np.max(np.abs(gs-ref)):.3e}")
    return errs
