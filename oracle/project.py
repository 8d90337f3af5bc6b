"""Float64 reference of the indexer projections and their fp8 quantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this.

Sources:

* Projections -- DeepSeek DSA FLOPs notes, section "Indexer projections":
  the indexer queries come from the MLA query latent, Q^I = C^Q W_IQ with
  C^Q (T, d_qc) and W_IQ (d_qc, H^I d^I), read as (T, H^I, d^I); the shared
  key K^I = X W_IK with X (T, d), W_IK (d, d^I); the head weights
  W^I = X W_IW with W_IW (d, H^I).  The weights are stored here out-feature
  major (row o holds column o of the matrix above), the layout the library
  takes: the product is then y[t, o] = sum_i a[t, i] * wt[o, i].
* FP8 -- the same notes ("Lightning Indexer FLOPs", remark after the score
  equation) say the indexer runs in FP8 but fix no scaling rule.  The reading
  taken: one fp32 scale per query token shared by its 64 heads and one per
  key row, scale = amax / 448 (448 is the largest finite e4m3fn value), codes
  = e4m3fn round-to-nearest-even of x * (448 / amax) saturated to +-448.
  Every fp32 step (the division, the product) is taken in fp32 with IEEE
  round-to-nearest-even, so a code is a function of the fp32 input alone.
  A row whose amax is 0 gets scale 1 and codes of +-0.
* bf16 output -- round-to-nearest-even of the fp32 projection.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def project(c_q: np.ndarray, x: np.ndarray, w_iq: np.ndarray, w_ik: np.ndarray, w_iw: np.ndarray, heads: int = 64):
    """Exact-as-float64 projections (Q^I [T,H,d], K^I [T,d], W^I [T,H]).

    c_q [T, d_qc], x [T, d] and the out-feature-major weights w_iq [H*d, d_qc],
    w_ik [d^I, d], w_iw [H, d] are float64 arrays (decoded bf16 values).
    """
    c_q, x = np.asarray(c_q, np.float64), np.asarray(x, np.float64)
    q = c_q @ np.asarray(w_iq, np.float64).T
    k = x @ np.asarray(w_ik, np.float64).T
    w = x @ np.asarray(w_iw, np.float64).T
    T = c_q.shape[0]
    return q.reshape(T, heads, -1), k, w


def projection_abs_bound(c_q, x, w_iq, w_ik, w_iw, heads: int = 64):
    """sum_i |a[t,i] * wt[o,i]| for every output: the scale of the rounding error
    of an fp32 accumulation of that output (the classic bound for a sum of n
    terms in any order is gamma_{n-1} times this)."""
    q = np.abs(np.asarray(c_q, np.float64)) @ np.abs(np.asarray(w_iq, np.float64)).T
    k = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w_ik, np.float64)).T
    w = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w_iw, np.float64)).T
    return q.reshape(q.shape[0], heads, -1), k, w


def e4m3fn_rne(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code of each value (ties to even mantissa), saturating.

    e4m3fn (OCP 8-bit floating point specification): sign, 4 exponent bits of
    bias 7, 3 mantissa bits.  Binade [2^e, 2^(e+1)) for e >= -6 holds 8 codes
    spaced 2^(e-3); below 2^-6 the codes are the subnormals m * 2^-9.
    Magnitudes at or above 448 map to 448.  Inputs must not be NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1)  ->  floor(log2 a) = ex - 1
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.ldexp(1.0, e - 3)  # spacing of codes around a
    r = np.round(a / quantum)  # exact division by a power of two; numpy rounds halves to even
    val = r * quantum
    val = np.minimum(val, FP8_MAX)  # only reachable from a >= 448 (432 < a < 448 rounds to 448 exactly)
    val = np.where(a >= FP8_MAX, FP8_MAX, val)
    # encode the (now representable) value
    sub = val < 2.0**-6
    _, vex = np.frexp(np.where(sub, 1.0, val))
    ve = vex.astype(np.int64) - 1
    mant_n = np.round((np.where(sub, 1.0, val) / np.ldexp(1.0, ve) - 1.0) * 8.0).astype(np.int64)
    code_n = ((ve + 7) << 3) | mant_n
    code_s = np.round(val / 2.0**-9).astype(np.int64)  # 0..7 (8 would be 2^-6, a normal)
    code = np.where(sub, code_s, code_n)
    return (sign | code).astype(np.uint8)


def quantize_rows_fp8(v32: np.ndarray):
    """Per-row e4m3fn quantisation of fp32 values [R, n] -> (codes uint8 [R, n], scales fp32 [R]).

    All arithmetic that decides a code is fp32: amax (exact), inv = 448 / amax
    and x * inv, each rounded to nearest even by numpy's IEEE fp32 operations.
    """
    v32 = np.asarray(v32, dtype=np.float32)
    amax = np.abs(v32).max(axis=1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(FP8_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(FP8_MAX) / safe).astype(np.float32)
    x = (v32 * inv[:, None]).astype(np.float32)
    return e4m3fn_rne(x.astype(np.float64)), scale


def bf16_rne(v32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    v = np.asarray(v32, dtype=np.float64)
    v32 = np.asarray(v32, dtype=np.float32)
    # the two bf16 neighbours of v: truncation and one ulp further from zero
    u = v32.view(np.uint32)
    lo = (u >> np.uint32(16)).astype(np.uint32)
    hi = lo + np.uint32(1)
    vlo = (lo << np.uint32(16)).view(np.float32).astype(np.float64)
    vhi = (hi << np.uint32(16)).view(np.float32).astype(np.float64)
    dlo, dhi = np.abs(v - vlo), np.abs(vhi - v)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & np.uint32(1)) == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def quantize_projection(q32: np.ndarray, k32: np.ndarray, out: str):
    """The prologue's output step applied to fp32 projections.

    q32 [T, H, d], k32 [T, d].  out = "fp8": (q codes, q_scale [T], k codes,
    k_scale [T]); out = "bf16": (q bits, None, k bits, None).
    """
    T = q32.shape[0]
    if out == "fp8":
        qc, qs = quantize_rows_fp8(q32.reshape(T, -1))
        kc, ks = quantize_rows_fp8(k32.reshape(T, -1))
        return qc.reshape(q32.shape), qs, kc.reshape(k32.shape), ks
    if out == "bf16":
        return bf16_rne(q32), None, bf16_rne(k32), None
    raise ValueError(out)
