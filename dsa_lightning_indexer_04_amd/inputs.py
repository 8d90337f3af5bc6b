"""Seeded synthetic inputs for the lightning indexer.

This module only draws and stores inputs.  It holds none of the indexer's
arithmetic (no dot products, no ReLU, no head sums, no selection), so the CPU
oracle and the HIP path can both consume what it makes without sharing any of
the method's code.

Tensor layout (DeepSeek DSA FLOPs notes, section "Notation", indexer tensors
Q^I (T,H^I,d^I), K^I (T,d^I), W^I (T,H^I)), with a leading batch axis B:

* ``q``   [B, Q, H, d]  bf16, or fp8 e4m3fn codes
* ``k``   [B, N, d]     bf16, or fp8 e4m3fn codes (one key shared by all heads)
* ``w``   [B, Q, H]     fp32, signed
* ``q_scale`` [B, Q], ``k_scale`` [B, N]  fp32 > 0 (fp8 only, else None)
* ``pos`` [B, Q]        int32 absolute position of each query row; key s is
  visible to the row iff s <= pos.

Two value distributions are provided:

``iid``        q and k entries i.i.d. N(0,1)/sqrt(128), w i.i.d. N(0,1).
``clustered``  16 shared key centroids of norm 3; each key is one centroid
               plus N(0, 0.3^2) noise per coordinate; each query row mixes 4
               distinct centroids with |N(0,1)| weights per head plus a small
               isotropic term; head weights |N(0,1)| with a random sign that is
               negative with probability 0.3.

fp8 inputs use one fp32 scale per key row and one per query token (shared by
its 64 heads): scale = amax / 448, codes = RNE(x / scale) saturated to +-448.

Around the indexer: ``make_projection_inputs`` draws the bf16 operands of the
indexer projections (activations N(0,1), weights N(0, 1/fan_in)), and
``make_mla_inputs`` / ``random_selection`` draw the sparse MLA attention's
query block, latent cache and selected positions.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEADS = 64
HEAD_DIM = 128
FP8_MAX = 448.0
NUM_CENTROIDS = 16
CENTROID_NORM = 3.0
KEY_NOISE = 0.3
QUERY_MIX = 4
QUERY_NOISE = 0.05
NEG_HEAD_PROB = 0.3


@dataclasses.dataclass(frozen=True)
class Workload:
    """One input shape: B sequences, Q query rows each, N keys each."""

    name: str
    batch: int
    num_q: int
    num_k: int
    topk: int
    dtype: str  # "bf16" or "fp8"
    dist: str  # "iid" or "clustered"
    pos_start: int  # row t sits at absolute position pos_start + t
    pruned: bool = False
    num_seeds: int = 12288
    query_noise: float = QUERY_NOISE  # clustered queries: per-coordinate noise scale (sigma_q)

    @property
    def visible_pairs(self) -> int:
        p = self.pos_start + np.arange(self.num_q, dtype=np.int64)
        return int(self.batch * np.minimum(p + 1, self.num_k).clip(min=0).sum())


# The five workloads the indexer is measured on (sizes of the DSA indexer as
# deployed in DeepSeek-V3.2: 64 heads of 128, k = 2048).
WORKLOADS = {
    "tiny_prefill_1k": Workload("tiny_prefill_1k", 1, 1024, 1024, 256, "bf16", "iid", 0),
    "prefill_32k": Workload("prefill_32k", 1, 32768, 32768, 2048, "bf16", "iid", 0),
    "decode_64x128k": Workload("decode_64x128k", 64, 1, 131072, 2048, "bf16", "iid", 131071),
    # the 128K block's seed count is not given; 2048 seeds (= k, the fewest
    # that still fix a start) is the measured best there with the raised start
    "chunked_prefill_128k": Workload(
        "chunked_prefill_128k", 1, 8192, 131072, 2048, "bf16", "clustered", 122880, pruned=True, num_seeds=2048
    ),
    "context_1m_fp8": Workload(
        "context_1m_fp8", 1, 16384, 1048576, 2048, "fp8", "clustered", 1032192, pruned=True
    ),
    # the 128K block with noisier queries (sigma_q = 0.2 instead of 0.05): the
    # filter-rate sensitivity of the pruned path
    "chunked_prefill_128k_noise02": Workload(
        "chunked_prefill_128k_noise02", 1, 8192, 131072, 2048, "bf16", "clustered", 122880, pruned=True,
        num_seeds=2048, query_noise=0.2,
    ),
}


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def quantize_fp8_rows(x: np.ndarray, row_axes: int) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-row e4m3fn quantisation: the leading ``row_axes`` axes index rows.

    Returns (codes as torch.float8_e4m3fn, fp32 scales with the row shape).
    """
    x = np.asarray(x, dtype=np.float32)
    rshape = x.shape[:row_axes]
    flat = x.reshape(int(np.prod(rshape)), -1)
    amax = np.abs(flat).max(axis=1)
    amax = np.where(amax > 0, amax, 1.0).astype(np.float32)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    y = np.clip(flat / scale[:, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).reshape(x.shape)
    return codes, torch.from_numpy(scale.reshape(rshape))


def _draw_iid(rng: np.random.Generator, B: int, Q: int, N: int):
    inv = np.float32(1.0 / math.sqrt(HEAD_DIM))
    # keys first, one sequence at a time to bound peak host memory
    ks = []
    for _ in range(B):
        ks.append(rng.standard_normal((N, HEAD_DIM), dtype=np.float32) * inv)
    q = rng.standard_normal((B, Q, HEADS, HEAD_DIM), dtype=np.float32) * inv
    w = rng.standard_normal((B, Q, HEADS), dtype=np.float32)
    return q, ks, w


def _draw_clustered(rng: np.random.Generator, B: int, Q: int, N: int, query_noise: float = QUERY_NOISE):
    ks, qs, ws = [], [], []
    for _ in range(B):
        g = rng.standard_normal((NUM_CENTROIDS, HEAD_DIM))
        cent = (CENTROID_NORM * g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)
        member = rng.integers(0, NUM_CENTROIDS, size=N)
        k = cent[member] + np.float32(KEY_NOISE) * rng.standard_normal((N, HEAD_DIM), dtype=np.float32)
        ks.append(k.astype(np.float32))
        # queries: 4 distinct centroids per row, |N(0,1)| mixing weight per head
        order = np.argsort(rng.random((Q, NUM_CENTROIDS)), axis=1)[:, :QUERY_MIX]
        a = np.abs(rng.standard_normal((Q, HEADS, QUERY_MIX))).astype(np.float32)
        mix = np.zeros((Q, HEADS, NUM_CENTROIDS), dtype=np.float32)
        rows = np.arange(Q)[:, None, None]
        heads = np.arange(HEADS)[None, :, None]
        mix[rows, heads, order[:, None, :]] = a
        q = np.einsum("thm,md->thd", mix, cent / np.float32(CENTROID_NORM)).astype(np.float32)
        q += np.float32(query_noise / math.sqrt(HEAD_DIM)) * rng.standard_normal(
            (Q, HEADS, HEAD_DIM), dtype=np.float32
        )
        qs.append(q)
        mag = np.abs(rng.standard_normal((Q, HEADS))).astype(np.float32)
        neg = rng.random((Q, HEADS)) < NEG_HEAD_PROB
        ws.append(np.where(neg, -mag, mag).astype(np.float32))
    return np.stack(qs), ks, np.stack(ws)


def make_inputs(
    batch: int,
    num_q: int,
    num_k: int,
    dtype: str = "bf16",
    dist: str = "iid",
    pos_start: int | None = None,
    seed: int = 0,
    positions: np.ndarray | None = None,
    query_noise: float = QUERY_NOISE,
) -> dict:
    """Draw one seeded input set as CPU torch tensors.

    ``pos_start`` defaults to N - Q (the query block sits at the tail of the
    sequence, which is plain causal prefill when Q == N).  ``positions``
    overrides it with an explicit [B, Q] int array.  ``query_noise`` is the
    clustered generator's query noise scale sigma_q.
    """
    if dtype not in ("bf16", "fp8"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    if dist == "iid":
        q, ks, w = _draw_iid(rng, batch, num_q, num_k)
    elif dist == "clustered":
        q, ks, w = _draw_clustered(rng, batch, num_q, num_k, query_noise)
    else:
        raise ValueError(dist)
    if positions is None:
        if pos_start is None:
            pos_start = num_k - num_q
        positions = np.broadcast_to(pos_start + np.arange(num_q), (batch, num_q))
    pos = torch.from_numpy(np.ascontiguousarray(positions, dtype=np.int32))
    out = {"w": torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)), "pos": pos, "dtype": dtype}
    if dtype == "bf16":
        out["q"] = _to_bf16(q)
        out["k"] = torch.stack([_to_bf16(k) for k in ks])
        out["q_scale"] = None
        out["k_scale"] = None
    else:
        out["q"], out["q_scale"] = quantize_fp8_rows(q, 2)
        kc, kscale = [], []
        for k in ks:
            c, s = quantize_fp8_rows(k, 1)
            kc.append(c)
            kscale.append(s)
        out["k"] = torch.stack(kc)
        out["k_scale"] = torch.stack(kscale)
    return out


def make_workload(wl: Workload | str, seed: int = 0) -> dict:
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    return make_inputs(wl.batch, wl.num_q, wl.num_k, wl.dtype, wl.dist, wl.pos_start, seed,
                       query_noise=wl.query_noise)


def evenly_spaced_seeds(num_seeds: int, common_prefix_end: int) -> np.ndarray:
    """Seed key indices floor(i * (p0 + 1) / S), i < S, over keys 0..p0.

    Distinct and ascending when S <= p0 + 1; every row whose position is at
    least p0 sees all of them.
    """
    p1 = int(common_prefix_end) + 1
    s = min(int(num_seeds), p1)
    return ((np.arange(s, dtype=np.int64) * p1) // s).astype(np.int32)


# DeepSeek-V3.2 sizes of the indexer projections (hidden d, query latent d_qc).
PROJ_HIDDEN = 7168
PROJ_Q_LATENT = 1536


def make_projection_inputs(T: int, hidden: int = PROJ_HIDDEN, q_latent: int = PROJ_Q_LATENT, seed: int = 0,
                           device="cpu") -> dict:
    """Seeded bf16 operands of the indexer projections.

    c_q [T, q_latent] and x [T, hidden] have i.i.d. N(0,1) entries (the
    normalised query latent and hidden state); the out-feature-major weights
    w_iq [64*128, q_latent], w_ik [128, hidden], w_iw [64, hidden] have
    i.i.d. N(0, 1/fan_in) entries, so every projection output has unit
    variance.  Drawn with torch's generator on ``device`` (draws on the GPU
    and on the CPU differ); T can be large on a GPU.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape, std):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        step = max(1, (1 << 26) // shape[1])  # bound the fp32 temporary
        for r in range(0, shape[0], step):
            n = min(step, shape[0] - r)
            x = torch.randn((n, shape[1]), generator=g, device=device, dtype=torch.float32)
            out[r:r + n] = (x * std).to(torch.bfloat16)
        return out

    return {
        "c_q": draw((T, q_latent), 1.0),
        "x": draw((T, hidden), 1.0),
        "w_iq": draw((HEADS * HEAD_DIM, q_latent), 1.0 / math.sqrt(q_latent)),
        "w_ik": draw((HEAD_DIM, hidden), 1.0 / math.sqrt(hidden)),
        "w_iw": draw((HEADS, hidden), 1.0 / math.sqrt(hidden)),
    }


# Sizes of the sparse MLA core attention (DeepSeek-V3.2: 128 heads, latent 512, RoPE 64).
MLA_HEADS = 128
MLA_LATENT = 512
MLA_ROPE = 64


def make_mla_inputs(B: int, Q: int, N: int, seed: int = 0, device="cpu") -> dict:
    """Seeded bf16 operands of the sparse MLA attention: q [B,Q,128,576]
    ([Q^A | Q^R] per head) and kv [B,N,576] ([C^KV | K^R] per position), all
    entries i.i.d. N(0,1) (normalised latents; with sm_scale = 1/sqrt(576) a
    score is N(0,1)).  Drawn with torch's generator on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    d = MLA_LATENT + MLA_ROPE

    def draw(shape):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = out.view(-1, d)
        step = 1 << 16
        for r in range(0, flat.shape[0], step):
            n = min(step, flat.shape[0] - r)
            flat[r:r + n] = torch.randn((n, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        return out

    return {"q": draw((B, Q, MLA_HEADS, d)), "kv": draw((B, N, d))}


def random_selection(B: int, Q: int, N: int, topk: int, pos: np.ndarray, seed: int = 0) -> np.ndarray:
    """[B,Q,topk] int32: for each row, min(topk, visible) distinct random
    positions in 0..pos (in random order), then -1 padding."""
    rng = np.random.default_rng(seed)
    out = np.full((B, Q, topk), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Q):
            vis = int(min(max(pos[b, t] + 1, 0), N))
            m = min(topk, vis)
            if m:
                out[b, t, :m] = rng.choice(vis, size=m, replace=False)
    return out


def to_bits(x: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 (uint16) or fp8 (uint8) tensor as numpy."""
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float8_e4m3fn:
        return x.contiguous().view(torch.uint8).numpy()
    raise TypeError(x.dtype)
