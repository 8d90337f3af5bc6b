"""Shared helpers of the tests: device transfer, oracle rows, checks."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_04_amd import inputs
from oracle import indexer


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def to_device(d: dict, dev="cuda") -> dict:
    out = {}
    for key, v in d.items():
        out[key] = v.to(dev) if isinstance(v, torch.Tensor) else v
    return out


def call_args(dd: dict):
    return (dd["q"], dd["k"], dd["w"], dd["pos"]), dict(q_scale=dd["q_scale"], k_scale=dd["k_scale"])


class OracleRows:
    """Float64 oracle scores of selected rows of one CPU input set."""

    def __init__(self, d: dict):
        self.d = d
        self.dtype = d["dtype"]
        self.qbits = inputs.to_bits(d["q"])
        self.kbits = inputs.to_bits(d["k"])
        self.w = d["w"].numpy().astype(np.float64)
        self.pos = d["pos"].numpy()
        self.qs = None if d["q_scale"] is None else d["q_scale"].numpy()
        self.ks = None if d["k_scale"] is None else d["k_scale"].numpy()
        self.N = self.kbits.shape[1]
        self._kf = {}
        self._k8 = {}

    def keys(self, b: int) -> np.ndarray:
        if b not in self._kf:
            if self.dtype == "bf16":
                self._kf[b] = indexer.decode_bf16(self.kbits[b])
            else:
                self._kf[b] = self.codes(b) * self.ks[b].astype(np.float64)[:, None]
        return self._kf[b]

    def visible(self, b: int, t: int) -> int:
        return int(indexer.visible_count(self.pos[b, t], self.N))

    def row(self, b: int, t: int) -> np.ndarray:
        """Visible scores of row (b, t), float64."""
        v = self.visible(b, t)
        if self.dtype == "bf16":
            q = indexer.decode_bf16(self.qbits[b, t])
        else:
            q = indexer.decode_e4m3fn(self.qbits[b, t]) * float(self.qs[b, t])
        return indexer.index_score_row(q, self.keys(b)[:v], self.w[b, t])

    def codes(self, b: int) -> np.ndarray:
        """e4m3 code values of sequence b's keys (fp8 inputs), decoded once."""
        if b not in self._k8:
            self._k8[b] = indexer.decode_e4m3fn(self.kbits[b])
        return self._k8[b]

    def bound(self, b: int, t: int, keys=None) -> np.ndarray:
        """fp32 evaluation error bound of row (b, t)'s visible scores
        (oracle.indexer.score_error_bound_row; fp8 in code units, scaled),
        or of the visible keys ``keys`` only (the bound is per key)."""
        v = self.visible(b, t)
        sel = np.arange(v) if keys is None else np.asarray(keys, np.int64)
        assert sel.size == 0 or (sel.min() >= 0 and sel.max() < v)
        if self.dtype == "bf16":
            return indexer.score_error_bound_row(indexer.decode_bf16(self.qbits[b, t]), self.keys(b)[sel], self.w[b, t])
        q8 = indexer.decode_e4m3fn(self.qbits[b, t])
        scale = np.float64(np.float32(self.qs[b, t])) * self.ks[b, sel].astype(np.float64)
        return indexer.score_error_bound_row(q8, self.codes(b)[sel], self.w[b, t], scale=scale)


def tol(dtype: str):
    return indexer.tolerance(dtype)


def assert_rows_ok(orc: OracleRows, idx: np.ndarray, sc: np.ndarray | None, rows, k: int):
    """Oracle acceptance of GPU Top-K rows; with returned scores, also each
    score within the fp32 evaluation bound of its oracle score."""
    rtol, atol = tol(orc.dtype)
    for b, t in rows:
        ref = orc.row(b, t)
        errs = indexer.check_topk_row(idx[b, t], ref, k, rtol, atol, None if sc is None else sc[b, t])
        assert not errs, f"row ({b},{t}): {errs}"
        if sc is not None:
            assert_within_bound(orc, b, t, idx[b, t], sc[b, t], ref)


def assert_within_bound(orc: OracleRows, b: int, t: int, idx_row, sc_row, ref=None):
    """GPU scores of the valid entries of a row within the fp32 error bound
    of the oracle (plus 1e-12 relative for the oracle's own rounding)."""
    ref = orc.row(b, t) if ref is None else ref
    valid = np.asarray(idx_row) >= 0
    keys = np.asarray(idx_row)[valid].astype(np.int64)
    if keys.size == 0:
        return
    bnd = orc.bound(b, t, keys)
    err = np.abs(np.asarray(sc_row, np.float64)[valid] - ref[keys])
    ok = err <= bnd + 1e-12 * np.abs(ref[keys])
    assert ok.all(), f"row ({b},{t}): {int((~ok).sum())} scores outside the fp32 bound, worst err/bound " \
        f"{float((err / np.maximum(bnd, 1e-30)).max()):.3g}"


def lexsort_topk_of_scores(S_row: np.ndarray, vis: int, k: int) -> np.ndarray:
    """Exact Top-K by sort over one row of (GPU) scores; total order score desc, idx asc."""
    s = S_row[:vis].astype(np.float64)
    order = np.lexsort((np.arange(vis), -s))
    return np.sort(order[: min(k, vis)])
