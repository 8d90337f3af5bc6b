"""ctypes binding of libdsa_indexer.so.

Argument marshalling only: tensors supply device pointers, torch's current
HIP stream supplies the stream, and torch allocates outputs and workspace.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_indexer.so")

DSA_BF16, DSA_FP8_E4M3, DSA_F32 = 0, 1, 2
DSA_OP_SCORES, DSA_OP_TOPK, DSA_OP_TOPK_PRUNED = 0, 1, 2
DSA_FLAG_ROUTE_STREAM, DSA_FLAG_ROUTE_SPLIT = 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20  # DSA_NOALLOC_SCRATCH_BYTES
ROUTES = {None: 0, "auto": 0, "stream": DSA_FLAG_ROUTE_STREAM, "split": DSA_FLAG_ROUTE_SPLIT}
ERR = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}


class Inputs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q", ctypes.c_int32),
        ("num_k", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("w", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("positions", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


class PruneOpts(ctypes.Structure):
    _fields_ = [
        ("num_seeds", ctypes.c_int32),
        ("num_retained", ctypes.c_int32),
        ("seed_idx", ctypes.c_void_p),
        ("force_recover", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


# Pruning flags (dsa_prune_opts.flags): the row's starting threshold and the
# candidate record format they select.
DSA_PRUNE_START_AT_TAU = 1 << 0
DSA_PRUNE_COMPACT_RECORDS = 1 << 1
DSA_PRUNE_ANCHOR_SEEDS = 1 << 2
PRUNE_STARTS = {"raised": 0, "tau": DSA_PRUNE_START_AT_TAU}
PRUNE_RECORDS = {"exact": 0, "compact": DSA_PRUNE_COMPACT_RECORDS}
PRUNE_SEEDS = {"even": 0, "anchor": DSA_PRUNE_ANCHOR_SEEDS}


class PruneStats(ctypes.Structure):
    _fields_ = [
        ("tau", ctypes.c_void_p),
        ("screened", ctypes.c_void_p),
        ("survivors", ctypes.c_void_p),
        ("recovered", ctypes.c_void_p),
        ("upper_bound", ctypes.c_void_p),
        ("plan_rows", ctypes.c_void_p),
        ("plan_coef", ctypes.c_void_p),
        ("plan_misc", ctypes.c_void_p),
    ]


class ProjInputs(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("q_latent", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("c_q", ctypes.c_void_p),
        ("x", ctypes.c_void_p),
        ("w_iq", ctypes.c_void_p),
        ("w_ik", ctypes.c_void_p),
        ("w_iw", ctypes.c_void_p),
    ]


class MlaInputs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q", ctypes.c_int32),
        ("num_k", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("kv", ctypes.c_void_p),
        ("indices", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]


EXPORTED = [
    "dsa_indexer_scores",
    "dsa_indexer_topk",
    "dsa_indexer_topk_pruned",
    "dsa_indexer_topk_noalloc",
    "dsa_indexer_workspace_bytes",
    "dsa_indexer_project",
    "dsa_indexer_project_workspace_bytes",
    "dsa_sparse_mla",
    "dsa_sparse_mla_workspace_bytes",
    "dsa_indexer_error_string",
    "dsa_indexer_last_error",
    "dsa_indexer_profile_begin",
    "dsa_indexer_profile_end",
    "dsa_indexer_mfma_ceiling",
]

_lib = None


def load() -> ctypes.CDLL:
    """Load the library (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m dsa_lightning_indexer_04_amd.build_lib` "
            "(the indexer has no non-HIP fallback)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.dsa_indexer_scores.argtypes = [ctypes.POINTER(Inputs), P, P]
    lib.dsa_indexer_scores.restype = ctypes.c_int
    lib.dsa_indexer_topk.argtypes = [ctypes.POINTER(Inputs), I32, P, P, P, SZ, P]
    lib.dsa_indexer_topk.restype = ctypes.c_int
    lib.dsa_indexer_topk_noalloc.argtypes = [ctypes.POINTER(Inputs), I32, P, P, P]
    lib.dsa_indexer_topk_noalloc.restype = ctypes.c_int
    lib.dsa_indexer_topk_pruned.argtypes = [
        ctypes.POINTER(Inputs),
        I32,
        ctypes.POINTER(PruneOpts),
        P,
        P,
        ctypes.POINTER(PruneStats),
        P,
        SZ,
        P,
    ]
    lib.dsa_indexer_topk_pruned.restype = ctypes.c_int
    lib.dsa_indexer_workspace_bytes.argtypes = [ctypes.c_int, ctypes.POINTER(Inputs), I32, ctypes.POINTER(PruneOpts)]
    lib.dsa_indexer_workspace_bytes.restype = SZ
    lib.dsa_indexer_project.argtypes = [ctypes.POINTER(ProjInputs), I32, P, P, P, P, P, P, SZ, P]
    lib.dsa_indexer_project.restype = ctypes.c_int
    lib.dsa_indexer_project_workspace_bytes.argtypes = [ctypes.POINTER(ProjInputs)]
    lib.dsa_indexer_project_workspace_bytes.restype = SZ
    lib.dsa_sparse_mla.argtypes = [ctypes.POINTER(MlaInputs), ctypes.c_float, P, P, P, SZ, P]
    lib.dsa_sparse_mla.restype = ctypes.c_int
    lib.dsa_sparse_mla_workspace_bytes.argtypes = [ctypes.POINTER(MlaInputs)]
    lib.dsa_sparse_mla_workspace_bytes.restype = SZ
    lib.dsa_indexer_error_string.argtypes = [ctypes.c_int]
    lib.dsa_indexer_error_string.restype = ctypes.c_char_p
    lib.dsa_indexer_last_error.argtypes = []
    lib.dsa_indexer_last_error.restype = ctypes.c_char_p
    lib.dsa_indexer_profile_begin.argtypes = []
    lib.dsa_indexer_profile_begin.restype = ctypes.c_int
    lib.dsa_indexer_profile_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(I32),
                                            ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.dsa_indexer_profile_end.restype = ctypes.c_int
    lib.dsa_indexer_mfma_ceiling.argtypes = [I32, I32, I32, P, SZ, P, ctypes.POINTER(I32)]
    lib.dsa_indexer_mfma_ceiling.restype = ctypes.c_int
    _lib = lib
    return lib


class IndexerError(RuntimeError):
    def __init__(self, code: int, detail: str):
        super().__init__(f"{ERR.get(code, code)}: {detail}")
        self.code = code


def _check(rc: int):
    if rc != 0:
        lib = load()
        raise IndexerError(rc, lib.dsa_indexer_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_device(named, device=None):
    """All tensors on one CUDA device (the current one unless `device` is given)."""
    dev = device
    for name, t in named:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor (got device {t.device})")
        if dev is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _check_shape(name, t, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def check_index_args(q, k, w, positions, q_scale=None, k_scale=None):
    """Dtype, layout and shape checks of the indexer inputs (no device check):
    q [B,Q,H,d] bf16 or float8_e4m3fn, k [B,N,d] of q's dtype, w [B,Q,H] fp32,
    positions [B,Q] int32, and for fp8 q_scale [B,Q] / k_scale [B,N] fp32
    (absent for bf16).  Returns (B, Q, H, d, N, dtype code)."""
    if q.dtype == torch.bfloat16:
        dt = DSA_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dt = DSA_FP8_E4M3
    else:
        raise TypeError(f"unsupported q dtype {q.dtype}")
    if k.dtype != q.dtype:
        raise TypeError("q and k must share a dtype")
    for name, t in (("q", q), ("k", k), ("w", w), ("positions", positions), ("q_scale", q_scale), ("k_scale", k_scale)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if w.dtype != torch.float32 or positions.dtype != torch.int32:
        raise TypeError("w must be float32 and positions int32")
    if q.dim() != 4 or k.dim() != 3:
        raise ValueError("q must be [B,Q,H,d] and k [B,N,d]")
    B, Q, H, D = q.shape
    N = k.shape[1]
    _check_shape("k", k, (B, N, D))
    _check_shape("w", w, (B, Q, H))
    _check_shape("positions", positions, (B, Q))
    if dt == DSA_FP8_E4M3:
        if q_scale is None or k_scale is None:
            raise ValueError("fp8 inputs need q_scale and k_scale")
        for name, t in (("q_scale", q_scale), ("k_scale", k_scale)):
            if t.dtype != torch.float32:
                raise TypeError(f"{name} must be float32")
        _check_shape("q_scale", q_scale, (B, Q))
        _check_shape("k_scale", k_scale, (B, N))
    elif q_scale is not None or k_scale is not None:
        raise ValueError("bf16 inputs take no scales")
    return B, Q, H, D, N, dt


def make_inputs_struct(q, k, w, positions, q_scale=None, k_scale=None, *, heads=None, head_dim=None,
                       flags: int = 0) -> Inputs:
    """Build the C inputs struct from device tensors, after checking them.

    q [B,Q,H,d] (bf16 or float8_e4m3fn), k [B,N,d], w [B,Q,H] fp32,
    positions [B,Q] int32, q_scale [B,Q] / k_scale [B,N] fp32 (fp8 only), all
    on the current CUDA device.  heads / head_dim override the sizes the
    struct declares (the library rejects any other than 64 / 128).
    """
    B, Q, H, D, N, dt = check_index_args(q, k, w, positions, q_scale, k_scale)
    _check_device((("q", q), ("k", k), ("w", w), ("positions", positions), ("q_scale", q_scale),
                   ("k_scale", k_scale)))
    return Inputs(
        B,
        Q,
        N,
        H if heads is None else heads,
        D if head_dim is None else head_dim,
        dt,
        _ptr(q),
        _ptr(k),
        _ptr(w),
        _ptr(q_scale),
        _ptr(k_scale),
        _ptr(positions),
        flags,
    )


def check_prune_args(seed_idx, force_recover, B: int, Q: int, num_seeds: int):
    """The pruned path's optional device arrays: seed_idx int32 with B*num_seeds
    elements (num_seeds > 0), force_recover uint8 or bool with B*Q elements,
    both contiguous."""
    if seed_idx is not None:
        if seed_idx.dtype != torch.int32:
            raise TypeError("seed_idx must be int32")
        if num_seeds <= 0:
            raise ValueError("seed_idx needs num_seeds > 0")
        if seed_idx.numel() != B * num_seeds:
            raise ValueError(f"seed_idx must hold batch * num_seeds = {B * num_seeds} entries, got {seed_idx.numel()}")
        if not seed_idx.is_contiguous():
            raise ValueError("seed_idx must be contiguous")
    if force_recover is not None:
        if force_recover.dtype not in (torch.uint8, torch.bool):
            raise TypeError("force_recover must be uint8 or bool")
        if force_recover.numel() != B * Q:
            raise ValueError(f"force_recover must hold batch * num_q = {B * Q} entries, got {force_recover.numel()}")
        if not force_recover.is_contiguous():
            raise ValueError("force_recover must be contiguous")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(op: int, inp: Inputs, topk: int = 0, opts: PruneOpts | None = None) -> int:
    lib = load()
    n = lib.dsa_indexer_workspace_bytes(op, ctypes.byref(inp), topk, ctypes.byref(opts) if opts else None)
    if n == 0 and op != DSA_OP_SCORES:
        detail = lib.dsa_indexer_last_error().decode()
        if detail:
            raise IndexerError(1, detail)
    return n


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte (or better) aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def scores(q, k, w, positions, q_scale=None, k_scale=None) -> torch.Tensor:
    """[B,Q,N] fp32 index scores, -inf where the key is not visible."""
    lib = load()
    inp = make_inputs_struct(q, k, w, positions, q_scale, k_scale)
    out = torch.empty((q.shape[0], q.shape[1], k.shape[1]), dtype=torch.float32, device=q.device)
    _check(lib.dsa_indexer_scores(ctypes.byref(inp), _ptr(out), _stream()))
    return out


def _route_flags(route):
    if route not in ROUTES:
        raise ValueError(f"route must be one of {sorted(r for r in ROUTES if r)} or None")
    return ROUTES[route]


def topk(q, k, w, positions, topk: int, q_scale=None, k_scale=None, return_scores: bool = True, workspace=None,
         route=None):
    """Exact per-row Top-K: (idx [B,Q,topk] int32 with -1 padding, scores or None).
    route: None (the library chooses), "stream" or "split" (DSA_FLAG_ROUTE_*)."""
    lib = load()
    inp = make_inputs_struct(q, k, w, positions, q_scale, k_scale, flags=_route_flags(route))
    nbytes = workspace_bytes(DSA_OP_TOPK, inp, topk)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    B, Q = q.shape[:2]
    idx = torch.empty((B, Q, topk), dtype=torch.int32, device=q.device)
    sc = torch.empty((B, Q, topk), dtype=torch.float32, device=q.device) if return_scores else None
    _check(lib.dsa_indexer_topk(ctypes.byref(inp), topk, _ptr(idx), _ptr(sc), _ptr(ws), ws.numel(), _stream()))
    return idx, sc


def topk_noalloc(q, k, w, positions, topk: int, q_scale=None, k_scale=None, return_scores: bool = True,
                 route=None):
    """dsa_indexer_topk_noalloc: the same Top-K with the library's fixed
    per-GPU scratch instead of a workspace (the outputs are still allocated
    here; the library call allocates nothing)."""
    lib = load()
    inp = make_inputs_struct(q, k, w, positions, q_scale, k_scale, flags=_route_flags(route))
    B, Q = q.shape[:2]
    idx = torch.empty((B, Q, topk), dtype=torch.int32, device=q.device)
    sc = torch.empty((B, Q, topk), dtype=torch.float32, device=q.device) if return_scores else None
    _check(lib.dsa_indexer_topk_noalloc(ctypes.byref(inp), topk, _ptr(idx), _ptr(sc), _stream()))
    return idx, sc


def topk_pruned(
    q,
    k,
    w,
    positions,
    topk: int,
    q_scale=None,
    k_scale=None,
    *,
    num_seeds: int = 0,
    num_retained: int = 0,
    seed_idx=None,
    force_recover=None,
    start: str | None = None,
    records: str = "exact",
    seeds: str = "even",
    return_scores: bool = True,
    stats: bool = False,
    upper_bound: bool = False,
    plan: bool = False,
    workspace=None,
):
    """Exact per-row Top-K with certified pruning; same index set as topk().

    start: "raised" (the default with even seeds) starts each row's running
    threshold at a seed record above tau, verified at the end (a row short of
    K records at its start is recomputed unpruned); "tau" (the default, and
    the only start, with anchor seeds) starts at tau, the K-th seed score.
    seeds: "even" (default) spaces num_seeds seeds evenly over the keys every
    row sees, or takes seed_idx; "anchor" takes the distinct keys of the
    exact Top-K of num_seeds // topk anchor rows per sequence (num_seeds >=
    topk, no seed_idx).
    records: "exact" (default) keeps 64-bit candidate records; "compact"
    keeps 32-bit records (row-relative score code + key index) and resolves
    the Top-K boundary by rescoring.
    Returns (idx, scores or None, stats dict or None).  stats holds per-row
    tau, screened, survivors, recovered (1: plan/seeds/forced, 2: raised
    start missed, 3: compact records did not fit), the debug upper bounds,
    and with plan=True each row's
    exported bound plan: plan_rows [B,Q,32,128] in q's dtype, plan_coef
    [B,Q,32], plan_misc [B,Q,2] = kappa, e_neg.
    """
    if seeds not in PRUNE_SEEDS:
        raise ValueError(f"seeds must be one of {sorted(PRUNE_SEEDS)}, not {seeds!r}")
    if start is None:
        start = "tau" if seeds == "anchor" else "raised"
    if start not in PRUNE_STARTS:
        raise ValueError(f"start must be one of {sorted(PRUNE_STARTS)}, not {start!r}")
    if seeds == "anchor":
        if start != "tau":
            raise ValueError("anchor seeds start every row at tau (start='tau')")
        if seed_idx is not None:
            raise ValueError("anchor seeds take no seed_idx")
        if (num_seeds or 12288) < topk:
            raise ValueError(f"anchor seeds need num_seeds >= topk ({num_seeds} < {topk})")
    if records not in PRUNE_RECORDS:
        raise ValueError(f"records must be one of {sorted(PRUNE_RECORDS)}, not {records!r}")
    lib = load()
    inp = make_inputs_struct(q, k, w, positions, q_scale, k_scale)
    check_prune_args(seed_idx, force_recover, q.shape[0], q.shape[1], num_seeds)
    _check_device((("seed_idx", seed_idx), ("force_recover", force_recover)), q.device)
    opts = PruneOpts(num_seeds, num_retained, _ptr(seed_idx), _ptr(force_recover),
                     PRUNE_STARTS[start] | PRUNE_RECORDS[records] | PRUNE_SEEDS[seeds])
    nbytes = workspace_bytes(DSA_OP_TOPK_PRUNED, inp, topk, opts)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    B, Q = q.shape[:2]
    dev = q.device
    idx = torch.empty((B, Q, topk), dtype=torch.int32, device=dev)
    sc = torch.empty((B, Q, topk), dtype=torch.float32, device=dev) if return_scores else None
    st = None
    cst = PruneStats()
    if stats or upper_bound or plan:
        st = {
            "tau": torch.empty((B, Q), dtype=torch.float32, device=dev),
            "screened": torch.empty((B, Q), dtype=torch.int32, device=dev),
            "survivors": torch.empty((B, Q), dtype=torch.int32, device=dev),
            "recovered": torch.empty((B, Q), dtype=torch.uint8, device=dev),
        }
        if upper_bound:
            st["upper_bound"] = torch.empty((B, Q, k.shape[1]), dtype=torch.float32, device=dev)
        if plan:
            st["plan_rows"] = torch.empty((B, Q, 32, 128), dtype=q.dtype, device=dev)
            st["plan_coef"] = torch.empty((B, Q, 32), dtype=torch.float32, device=dev)
            st["plan_misc"] = torch.empty((B, Q, 2), dtype=torch.float32, device=dev)
        cst = PruneStats(*(_ptr(st.get(n)) for n in ("tau", "screened", "survivors", "recovered", "upper_bound",
                                                      "plan_rows", "plan_coef", "plan_misc")))
    _check(
        lib.dsa_indexer_topk_pruned(
            ctypes.byref(inp),
            topk,
            ctypes.byref(opts),
            _ptr(idx),
            _ptr(sc),
            ctypes.byref(cst),
            _ptr(ws),
            ws.numel(),
            _stream(),
        )
    )
    return idx, sc, st


def make_proj_struct(c_q, x, w_iq, w_ik, w_iw, block_tokens: int = 0) -> ProjInputs:
    """C struct of the projection inputs: bf16 device tensors c_q [T, q_latent],
    x [T, hidden] and out-feature-major weights w_iq [64*128, q_latent],
    w_ik [128, hidden], w_iw [64, hidden]."""
    for name, t in (("c_q", c_q), ("x", x), ("w_iq", w_iq), ("w_ik", w_ik), ("w_iw", w_iw)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    T, L = c_q.shape
    if x.shape[0] != T:
        raise ValueError("c_q and x must have the same number of tokens")
    D = x.shape[1]
    if tuple(w_iq.shape) != (64 * 128, L) or tuple(w_ik.shape) != (128, D) or tuple(w_iw.shape) != (64, D):
        raise ValueError("weights must be w_iq [8192, q_latent], w_ik [128, hidden], w_iw [64, hidden]")
    _check_device((("c_q", c_q), ("x", x), ("w_iq", w_iq), ("w_ik", w_ik), ("w_iw", w_iw)))
    return ProjInputs(T, D, L, 64, 128, block_tokens, _ptr(c_q), _ptr(x), _ptr(w_iq), _ptr(w_ik), _ptr(w_iw))


_PROJ_OUT = {"fp8": (DSA_FP8_E4M3, torch.float8_e4m3fn), "bf16": (DSA_BF16, torch.bfloat16), "f32": (DSA_F32, torch.float32)}


def project(c_q, x, w_iq, w_ik, w_iw, out: str = "fp8", workspace=None, block_tokens: int = 0) -> dict:
    """Indexer projections Q^I = C^Q W_IQ, K^I = X W_IK, W^I = X W_IW and the
    output conversion.  Returns {"q" [T,64,128], "k" [T,128], "w" [T,64] fp32,
    "q_scale" [T], "k_scale" [T] (fp8 only, else None)}: for one sequence,
    the q, k, w and scales the scoring calls take.  block_tokens: tokens per
    query-GEMM block (0: the library's 65536)."""
    lib = load()
    if out not in _PROJ_OUT:
        raise ValueError(f"out must be one of {sorted(_PROJ_OUT)}")
    code, dt = _PROJ_OUT[out]
    inp = make_proj_struct(c_q, x, w_iq, w_ik, w_iw, block_tokens)
    need = lib.dsa_indexer_project_workspace_bytes(ctypes.byref(inp))
    if need == 0:
        raise IndexerError(1, lib.dsa_indexer_last_error().decode())
    ws = workspace if workspace is not None else _workspace(need, c_q.device)
    T, dev = c_q.shape[0], c_q.device
    q = torch.empty((T, 64, 128), dtype=dt, device=dev)
    k = torch.empty((T, 128), dtype=dt, device=dev)
    w = torch.empty((T, 64), dtype=torch.float32, device=dev)
    qs = torch.empty((T,), dtype=torch.float32, device=dev) if out == "fp8" else None
    ks = torch.empty((T,), dtype=torch.float32, device=dev) if out == "fp8" else None
    _check(lib.dsa_indexer_project(ctypes.byref(inp), code, _ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(w), _ptr(ws),
                                   ws.numel(), _stream()))
    return {"q": q, "k": k, "w": w, "q_scale": qs, "k_scale": ks}


def project_workspace_bytes(inp: ProjInputs) -> int:
    lib = load()
    n = lib.dsa_indexer_project_workspace_bytes(ctypes.byref(inp))
    if n == 0:
        raise IndexerError(1, lib.dsa_indexer_last_error().decode())
    return n


def make_mla_struct(q, kv, indices, page_table=None, num_k=None, num_splits: int = 0) -> MlaInputs:
    """C struct of the sparse MLA inputs: q [B,Q,128,576] bf16, indices
    [B,Q,topk] int32 and either kv [B,N,576] bf16, or (paged) a page pool kv
    [num_pages,page_size,576] with page_table [B,pages_per_seq] int32 and the
    sequence length num_k (device tensors)."""
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16:
        raise TypeError("q and kv must be bfloat16")
    if indices.dtype != torch.int32 or (page_table is not None and page_table.dtype != torch.int32):
        raise TypeError("indices and page_table must be int32")
    for name, t in (("q", q), ("kv", kv), ("indices", indices), ("page_table", page_table)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or indices.dim() != 3 or kv.dim() != 3:
        raise ValueError("shapes must be q [B,Q,H,576], kv [..,..,576], indices [B,Q,topk]")
    B, Q, H, D = q.shape
    if kv.shape[-1] != D or tuple(indices.shape[:2]) != (B, Q):
        raise ValueError("shapes must be q [B,Q,H,576], kv [..,576], indices [B,Q,topk]")
    _check_device((("q", q), ("kv", kv), ("indices", indices), ("page_table", page_table)))
    if page_table is None:
        if kv.shape[0] != B:
            raise ValueError("a flat kv is [B,N,576]")
        return MlaInputs(B, Q, kv.shape[1], H, 512, D - 512, indices.shape[2], num_splits, _ptr(q), _ptr(kv),
                         _ptr(indices), None, 0, 0, 0)
    if num_k is None or page_table.shape[0] != B:
        raise ValueError("a paged kv needs num_k and page_table [B,pages_per_seq]")
    return MlaInputs(B, Q, num_k, H, 512, D - 512, indices.shape[2], num_splits, _ptr(q), _ptr(kv), _ptr(indices),
                     _ptr(page_table), kv.shape[1], page_table.shape[1], kv.shape[0])


def sparse_mla(q, kv, indices, sm_scale: float, return_lse: bool = True, workspace=None, *, page_table=None,
               num_k=None, num_splits: int = 0):
    """MLA core attention (MQA mode) over the selected positions: returns
    (out [B,Q,128,512] bf16, lse [B,Q,128] fp32 or None).  With page_table,
    kv is a page pool [num_pages,page_size,576] and num_k the sequence length.
    num_splits: work units per row (0: the library chooses)."""
    lib = load()
    inp = make_mla_struct(q, kv, indices, page_table, num_k, num_splits)
    need = lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(inp))
    if need == 0:
        raise IndexerError(1, lib.dsa_indexer_last_error().decode())
    ws = workspace if workspace is not None else _workspace(need, q.device)
    B, Q = q.shape[:2]
    out = torch.empty((B, Q, 128, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Q, 128), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.dsa_sparse_mla(ctypes.byref(inp), float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                              _stream()))
    return out, lse


def sparse_mla_workspace_bytes(inp: MlaInputs) -> int:
    lib = load()
    n = lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(inp))
    if n == 0:
        raise IndexerError(1, lib.dsa_indexer_last_error().decode())
    return n


def profile_begin():
    """Open a per-kernel timing window (events on the launch stream)."""
    load().dsa_indexer_profile_begin()


def profile_end(max_kernels: int = 16) -> dict:
    """Close the window: {kernel name: (launches, mean ms)}."""
    lib = load()
    names = (ctypes.c_char_p * max_kernels)()
    counts = (ctypes.c_int32 * max_kernels)()
    means = (ctypes.c_double * max_kernels)()
    n = lib.dsa_indexer_profile_end(names, counts, means, max_kernels)
    if n < 0:
        raise IndexerError(4, "profile window: HIP error")
    return {names[i].decode(): (int(counts[i]), float(means[i])) for i in range(min(n, max_kernels))}


def mfma_ceiling(dtype: str, mode: int, iters: int, out=None) -> int:
    """The score step on synthetic operands (dsa_indexer_mfma_ceiling) on the
    current stream; returns the launch's workgroup count.  With out=None only
    the count is returned, nothing is launched."""
    if dtype not in ("bf16", "fp8"):
        raise ValueError(f"dtype must be bf16 or fp8, got {dtype!r}")
    lib = load()
    wg = ctypes.c_int32(0)
    if out is not None:
        _check_device([("out", out)])
        if out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor")
    rc = lib.dsa_indexer_mfma_ceiling(DSA_BF16 if dtype == "bf16" else DSA_FP8_E4M3, mode, iters, _ptr(out),
                                      0 if out is None else out.numel(), _stream(), ctypes.byref(wg))
    _check(rc)
    return int(wg.value)
