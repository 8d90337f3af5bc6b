"""The C-ABI library builds, loads and exports every declared symbol, and
rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h")]
LIB = os.path.join(ROOT, "dsa_lightning_indexer_04_amd", "libdsa_indexer.so")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdsa_indexer.so not built (run __graft_entry__.build())")
    import torch  # noqa: F401  (share torch's HIP runtime)
    from dsa_lightning_indexer_04_amd import _lib

    return _lib.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dsa_indexer_scores", "dsa_indexer_topk", "dsa_indexer_topk_pruned", "dsa_indexer_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


FAKE = 1 << 20  # aligned, never dereferenced: every case below fails validation first


def _inputs(_lib, **kw):
    d = dict(batch=1, num_q=4, num_k=64, heads=64, head_dim=128, dtype=0, q=FAKE, k=FAKE * 2, w=FAKE * 3,
             q_scale=None, k_scale=None, positions=FAKE * 4)
    d.update(kw)
    return _lib.Inputs(**d)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(heads=32), 2),
        (dict(head_dim=64), 2),
        (dict(dtype=7), 2),
        (dict(num_q=0), 1),
        (dict(batch=-1), 1),
        (dict(q=None), 1),
        (dict(q=FAKE + 4), 1),
        (dict(dtype=1), 1),  # fp8 without scales
        (dict(q_scale=FAKE * 5), 1),  # bf16 with a scale
    ],
)
def test_invalid_inputs_are_rejected(lib, kw, code):
    from dsa_lightning_indexer_04_amd import _lib

    inp = _inputs(_lib, **kw)
    rc = lib.dsa_indexer_scores(ctypes.byref(inp), ctypes.c_void_p(FAKE * 8), None)
    assert rc == code
    assert lib.dsa_indexer_last_error()
    rc = lib.dsa_indexer_topk(ctypes.byref(inp), 16, ctypes.c_void_p(FAKE * 8), None, None, 0, None)
    assert rc == code


def test_topk_argument_errors(lib):
    from dsa_lightning_indexer_04_amd import _lib

    inp = _inputs(_lib)
    out = ctypes.c_void_p(FAKE * 8)
    assert lib.dsa_indexer_topk(ctypes.byref(inp), 0, out, None, None, 0, None) == 1
    assert lib.dsa_indexer_topk(ctypes.byref(inp), 5000, out, None, None, 0, None) == 2
    assert lib.dsa_indexer_topk(ctypes.byref(inp), 16, None, None, None, 0, None) == 1
    # workspace too small
    need = lib.dsa_indexer_workspace_bytes(1, ctypes.byref(inp), 16, None)
    assert need > 0
    assert lib.dsa_indexer_topk(ctypes.byref(inp), 16, out, None, ctypes.c_void_p(FAKE * 64), need - 1, None) == 3
    # an output aliasing an input
    assert lib.dsa_indexer_topk(ctypes.byref(inp), 16, ctypes.c_void_p(FAKE * 3), None, None, need, None) == 1
    assert lib.dsa_indexer_error_string(3) == b"workspace too small"


def _proj(_lib, **kw):
    d = dict(num_tokens=16, hidden=7168, q_latent=1536, heads=64, head_dim=128, c_q=FAKE, x=FAKE * 2,
             w_iq=FAKE * 3, w_ik=FAKE * 4, w_iw=FAKE * 5)
    d.update(kw)
    return _lib.ProjInputs(**d)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(heads=32), 2),
        (dict(head_dim=64), 2),
        (dict(num_tokens=0), 1),
        (dict(hidden=7170), 1),
        (dict(q_latent=0), 1),
        (dict(x=None), 1),
        (dict(w_iq=FAKE + 2), 1),
    ],
)
def test_projection_inputs_are_rejected(lib, kw, code):
    from dsa_lightning_indexer_04_amd import _lib

    inp = _proj(_lib, **kw)
    o = ctypes.c_void_p
    rc = lib.dsa_indexer_project(ctypes.byref(inp), 0, o(FAKE * 8), None, o(FAKE * 9), None, o(FAKE * 10),
                                 o(FAKE * 64), 1 << 40, None)
    assert rc == code
    assert lib.dsa_indexer_last_error()
    assert lib.dsa_indexer_project_workspace_bytes(ctypes.byref(inp)) == 0


def test_projection_argument_errors(lib):
    from dsa_lightning_indexer_04_amd import _lib

    inp = _proj(_lib)
    o = ctypes.c_void_p
    need = lib.dsa_indexer_project_workspace_bytes(ctypes.byref(inp))
    # the fp32 staging block of 16 tokens, the concatenated key/weight matrix and the GEMM scratch
    assert need >= 16 * (8192 + 192) * 4 + 192 * 7168 * 2 + (32 << 20)
    # outputs clear of every input span (w_iq alone spans 24 MiB from FAKE * 3)
    qo, ko, wo, ws = o(FAKE * 64), o(FAKE * 65), o(FAKE * 66), o(FAKE * 128)
    qs, ks = o(FAKE * 67), o(FAKE * 68)
    call = lib.dsa_indexer_project
    assert call(ctypes.byref(inp), 5, qo, None, ko, None, wo, ws, need, None) == 2  # unknown out dtype
    assert call(ctypes.byref(inp), 1, qo, None, ko, None, wo, ws, need, None) == 1  # fp8 without scales
    assert call(ctypes.byref(inp), 0, qo, qs, ko, ks, wo, ws, need, None) == 1  # bf16 with scales
    assert call(ctypes.byref(inp), 2, None, None, ko, None, wo, ws, need, None) == 1  # missing q_out
    assert call(ctypes.byref(inp), 2, qo, None, ko, None, wo, ws, need - 1, None) == 3  # workspace too small
    assert call(ctypes.byref(inp), 2, qo, None, ko, None, wo, o(FAKE * 128 + 16), need, None) == 1  # misaligned
    assert b"256-byte" in lib.dsa_indexer_last_error()
    assert call(ctypes.byref(inp), 2, o(FAKE * 2), None, ko, None, wo, ws, need, None) == 1  # q_out aliases x
    assert b"aliases an input" in lib.dsa_indexer_last_error()
    assert call(ctypes.byref(inp), 2, qo, None, qo, None, wo, ws, need, None) == 1  # outputs overlap
    assert b"must not overlap" in lib.dsa_indexer_last_error()
    assert call(ctypes.byref(inp), 1, qo, qs, ko, ks, wo, o(FAKE * 67), need, None) == 1  # workspace over a scale
    assert b"must not overlap" in lib.dsa_indexer_last_error()


def _mla(_lib, **kw):
    d = dict(batch=1, num_q=8, num_k=4096, heads=128, latent_dim=512, rope_dim=64, topk=2048, q=FAKE * 256,
             kv=FAKE * 512, indices=FAKE * 600, page_table=None, page_size=0, pages_per_seq=0, num_pages=0)
    d.update(kw)
    return _lib.MlaInputs(**d)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(heads=64), 2),
        (dict(latent_dim=256), 2),
        (dict(rope_dim=0), 2),
        (dict(topk=4096), 2),
        (dict(topk=0), 1),
        (dict(num_k=0), 1),
        (dict(kv=None), 1),
        (dict(indices=FAKE * 600 + 4), 1),
        (dict(page_table=FAKE * 650, page_size=64, pages_per_seq=63, num_pages=100), 1),  # 63*64 < 4096
        (dict(page_table=FAKE * 650, page_size=0, pages_per_seq=64, num_pages=100), 1),
        (dict(page_table=FAKE * 650 + 8, page_size=64, pages_per_seq=64, num_pages=100), 1),
        (dict(page_table=FAKE * 650, page_size=1 << 16, pages_per_seq=1, num_pages=1 << 16), 1),  # pool > 2^31 rows
    ],
)
def test_sparse_mla_inputs_are_rejected(lib, kw, code):
    from dsa_lightning_indexer_04_amd import _lib

    inp = _mla(_lib, **kw)
    o = ctypes.c_void_p
    rc = lib.dsa_sparse_mla(ctypes.byref(inp), 0.04, o(FAKE * 700), None, o(FAKE * 800), 1 << 30, None)
    assert rc == code
    assert lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(inp)) == 0


def test_sparse_mla_argument_errors(lib):
    from dsa_lightning_indexer_04_amd import _lib

    inp = _mla(_lib)
    o = ctypes.c_void_p
    need = lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(inp))
    assert need >= 8 * 128 * 4 + 8 * 4
    out, ws = o(FAKE * 700), o(FAKE * 800)
    call = lib.dsa_sparse_mla
    assert call(ctypes.byref(inp), -1.0, out, None, ws, need, None) == 1
    assert call(ctypes.byref(inp), float("inf"), out, None, ws, need, None) == 1
    assert call(ctypes.byref(inp), 0.04, None, None, ws, need, None) == 1
    assert call(ctypes.byref(inp), 0.04, out, None, ws, need - 1, None) == 3
    assert call(ctypes.byref(inp), 0.04, o(FAKE * 512), None, ws, need, None) == 1  # out aliases kv
    assert b"aliases an input" in lib.dsa_indexer_last_error()
    assert call(ctypes.byref(inp), 0.04, out, None, out, need, None) == 1  # workspace over out
    assert b"must not overlap" in lib.dsa_indexer_last_error()


@pytest.mark.parametrize("flags", [4, 1 << 31, 3])
def test_bad_flags_are_rejected(lib, flags):
    """Unknown flag bits, and both Top-K routes at once."""
    from dsa_lightning_indexer_04_amd import _lib

    inp = _inputs(_lib, flags=flags)
    assert lib.dsa_indexer_topk(ctypes.byref(inp), 16, ctypes.c_void_p(FAKE * 8), None, None, 0, None) == 1
    assert lib.dsa_indexer_workspace_bytes(1, ctypes.byref(inp), 16, None) == 0
    assert lib.dsa_indexer_last_error()


@pytest.mark.parametrize("flags,ok", [(0, True), (1, True), (2, True), (3, True), (4, True), (7, True), (8, False),
                                      (1 << 31, False)])
def test_prune_flags(lib, flags, ok):
    """dsa_prune_opts.flags: DSA_PRUNE_START_AT_TAU, DSA_PRUNE_COMPACT_RECORDS
    and DSA_PRUNE_ANCHOR_SEEDS are known; none changes the workspace."""
    import torch

    from dsa_lightning_indexer_04_amd import _lib

    inp = _inputs(_lib)
    base = lib.dsa_indexer_workspace_bytes(2, ctypes.byref(inp), 16, ctypes.byref(_lib.PruneOpts(0, 0, None, None, 0)))
    got = lib.dsa_indexer_workspace_bytes(2, ctypes.byref(inp), 16, ctypes.byref(_lib.PruneOpts(0, 0, None, None, flags)))
    assert base > 0
    assert got == (base if ok else 0)
    if not ok:
        assert b"flags" in lib.dsa_indexer_last_error()
    with pytest.raises(ValueError, match="start"):
        _lib.topk_pruned(*[torch.zeros(1)] * 4, 16, start="high")
    with pytest.raises(ValueError, match="records"):
        _lib.topk_pruned(*[torch.zeros(1)] * 4, 16, records="short")


def test_compact_records_need_at_most_2_24_keys(lib):
    """Compact records keep the key index in the low bits of 32 (at most 24
    of them)."""
    from dsa_lightning_indexer_04_amd import _lib

    opts = _lib.PruneOpts(0, 0, None, None, _lib.DSA_PRUNE_COMPACT_RECORDS)
    assert lib.dsa_indexer_workspace_bytes(2, ctypes.byref(_inputs(_lib, num_q=4, num_k=1 << 24)), 16,
                                           ctypes.byref(opts)) > 0
    assert lib.dsa_indexer_workspace_bytes(2, ctypes.byref(_inputs(_lib, num_q=4, num_k=(1 << 24) + 1)), 16,
                                           ctypes.byref(opts)) == 0
    assert b"2^24" in lib.dsa_indexer_last_error()


def test_route_flags_set_the_workspace(lib):
    """The key-split route stores [B*Q, N] fp32 score rows plus a 2048-bin
    histogram per row; the streaming route (4*topk + 640) 8-byte records per
    row; with no flag, 4 rows pick the split route."""
    from dsa_lightning_indexer_04_amd import _lib

    split = lib.dsa_indexer_workspace_bytes(1, ctypes.byref(_inputs(_lib, flags=_lib.DSA_FLAG_ROUTE_SPLIT)), 16, None)
    stream = lib.dsa_indexer_workspace_bytes(1, ctypes.byref(_inputs(_lib, flags=_lib.DSA_FLAG_ROUTE_STREAM)), 16, None)
    auto = lib.dsa_indexer_workspace_bytes(1, ctypes.byref(_inputs(_lib)), 16, None)
    assert split == 4 * 64 * 4 + 4 * 2048 * 4
    assert stream == ((4 * (4 * 16 + 640) * 8 + 255) // 256) * 256
    assert auto == split


@pytest.mark.parametrize("block,ok", [(0, True), (64, True), (100, True), (1 << 18, True), (63, False),
                                      ((1 << 18) + 1, False), (-5, False)])
def test_projection_block_tokens(lib, block, ok):
    """block_tokens sets the fp32 staging block of the query GEMM (and so the
    workspace); outside 64..262144 (0: default) it is an argument error."""
    from dsa_lightning_indexer_04_amd import _lib

    inp = _proj(_lib, num_tokens=5000, block_tokens=block)
    need = lib.dsa_indexer_project_workspace_bytes(ctypes.byref(inp))
    if not ok:
        assert need == 0 and b"block_tokens" in lib.dsa_indexer_last_error()
        return
    blk = min(5000, block or 65536)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need == up(blk * 8192 * 4) + up(5000 * 192 * 4) + up(192 * 7168 * 2) + (32 << 20)


@pytest.mark.parametrize("splits,ok", [(0, True), (1, True), (8, True), (9, False), (-1, False)])
def test_sparse_mla_num_splits(lib, splits, ok):
    """num_splits pins the work units per row (and the partial-output
    workspace); 0 lets the library choose (8 rows: 8 units per row)."""
    from dsa_lightning_indexer_04_amd import _lib

    inp = _mla(_lib, num_splits=splits)
    need = lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(inp))
    if not ok:
        assert need == 0 and b"num_splits" in lib.dsa_indexer_last_error()
        return
    units = 8 * (splits or 8)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = up(units * 128 * 4) + up(units * 4)
    if units > 8:
        want += up(units * 128 * 512 * 4) + up(units * 128 * 2 * 4)
    assert need == want


# ---------------------------------------------------------------- Python wrapper checks (no GPU needed)


def _cpu_inputs(dtype="bf16", B=2, Q=3, N=40):
    import torch

    from dsa_lightning_indexer_04_amd import inputs

    d = inputs.make_inputs(B, Q, N, dtype, "iid", seed=0)
    return d, torch


def test_wrapper_rejects_host_tensors():
    """Tensors must be CUDA tensors: a host pointer handed to a kernel would fault."""
    from dsa_lightning_indexer_04_amd import _lib

    d, _ = _cpu_inputs()
    with pytest.raises(ValueError, match="CUDA tensor"):
        _lib.make_inputs_struct(d["q"], d["k"], d["w"], d["pos"])


@pytest.mark.parametrize(
    "change,exc,msg",
    [
        (lambda d, t: d.update(k=d["k"][:1]), ValueError, "k must have shape"),
        (lambda d, t: d.update(k=d["k"][:, :, :64].contiguous()), ValueError, "k must have shape"),
        (lambda d, t: d.update(w=d["w"][:, :, :32].contiguous()), ValueError, "w must have shape"),
        (lambda d, t: d.update(pos=d["pos"][:, :2].contiguous()), ValueError, "positions must have shape"),
        (lambda d, t: d.update(pos=d["pos"].long()), TypeError, "int32"),
        (lambda d, t: d.update(w=d["w"].double()), TypeError, "float32"),
        (lambda d, t: d.update(q=d["q"].float()), TypeError, "unsupported q dtype"),
        (lambda d, t: d.update(k=d["k"].transpose(1, 2)), ValueError, "contiguous"),
        (lambda d, t: d.update(q_scale=t.ones(2, 3)), ValueError, "bf16 inputs take no scales"),
    ],
)
def test_wrapper_rejects_bad_shapes_and_dtypes(change, exc, msg):
    from dsa_lightning_indexer_04_amd import _lib

    d, torch = _cpu_inputs()
    change(d, torch)
    with pytest.raises(exc, match=msg):
        _lib.check_index_args(d["q"], d["k"], d["w"], d["pos"], d.get("q_scale"), d.get("k_scale"))


def test_wrapper_checks_fp8_scales():
    from dsa_lightning_indexer_04_amd import _lib

    d, torch = _cpu_inputs("fp8")
    assert _lib.check_index_args(d["q"], d["k"], d["w"], d["pos"], d["q_scale"], d["k_scale"])[5] == 1
    with pytest.raises(ValueError, match="need q_scale"):
        _lib.check_index_args(d["q"], d["k"], d["w"], d["pos"], None, d["k_scale"])
    with pytest.raises(ValueError, match="k_scale must have shape"):
        _lib.check_index_args(d["q"], d["k"], d["w"], d["pos"], d["q_scale"], d["k_scale"][:, :10].contiguous())
    with pytest.raises(TypeError, match="q_scale must be float32"):
        _lib.check_index_args(d["q"], d["k"], d["w"], d["pos"], d["q_scale"].double(), d["k_scale"])


@pytest.mark.parametrize(
    "seed,force,num_seeds,exc,msg",
    [
        ("i64", None, 8, TypeError, "seed_idx must be int32"),
        ("short", None, 8, ValueError, "batch \\* num_seeds"),
        ("ok", None, 0, ValueError, "num_seeds > 0"),
        (None, "f32", 0, TypeError, "force_recover must be uint8"),
        (None, "short", 0, ValueError, "batch \\* num_q"),
    ],
)
def test_wrapper_checks_prune_arrays(seed, force, num_seeds, exc, msg):
    """seed_idx: int32 with batch * num_seeds entries (a seed list without its
    batch axis is too short); force_recover: uint8/bool with batch * num_q."""
    import torch

    from dsa_lightning_indexer_04_amd import _lib

    B, Q = 2, 3
    seeds = {"i64": torch.arange(B * 8, dtype=torch.int64), "short": torch.arange(8, dtype=torch.int32),
             "ok": torch.arange(B * 8, dtype=torch.int32), None: None}[seed]
    fr = {"f32": torch.zeros(B * Q), "short": torch.zeros(Q, dtype=torch.uint8), None: None}[force]
    with pytest.raises(exc, match=msg):
        _lib.check_prune_args(seeds, fr, B, Q, num_seeds)
    _lib.check_prune_args(torch.arange(B * 8, dtype=torch.int32), torch.zeros(B, Q, dtype=torch.bool), B, Q, 8)


def test_wrapper_rejects_host_tensors_in_other_calls():
    import torch

    from dsa_lightning_indexer_04_amd import _lib

    bf = torch.bfloat16
    with pytest.raises(ValueError, match="CUDA tensor"):
        _lib.make_proj_struct(torch.zeros(4, 64, dtype=bf), torch.zeros(4, 64, dtype=bf), torch.zeros(8192, 64, dtype=bf),
                              torch.zeros(128, 64, dtype=bf), torch.zeros(64, 64, dtype=bf))
    with pytest.raises(ValueError, match="CUDA tensor"):
        _lib.make_mla_struct(torch.zeros(1, 2, 128, 576, dtype=bf), torch.zeros(1, 50, 576, dtype=bf),
                             torch.zeros(1, 2, 16, dtype=torch.int32))
    with pytest.raises(ValueError, match="route"):
        _lib._route_flags("fast")


def test_noalloc_rejects_calls_beyond_the_fixed_scratch(lib):
    """The no-allocation Top-K refuses, before any GPU call, a call whose
    workspace exceeds the fixed 64 MiB scratch: 8192 streaming rows at top-2048
    need 8192 * 8832 * 8 bytes."""
    from dsa_lightning_indexer_04_amd import _lib

    inp = _inputs(_lib, num_q=8192, num_k=131072, flags=_lib.DSA_FLAG_ROUTE_STREAM)
    need = lib.dsa_indexer_workspace_bytes(1, ctypes.byref(inp), 2048, None)
    assert need == 8192 * (4 * 2048 + 640) * 8 > _lib.NOALLOC_SCRATCH_BYTES
    rc = lib.dsa_indexer_topk_noalloc(ctypes.byref(inp), 2048, ctypes.c_void_p(FAKE * 8), None, None)
    assert rc == 3 and b"fixed scratch" in lib.dsa_indexer_last_error()
    # the decode batch fits: 64 rows x 131072 keys of score rows + histograms
    dec = _inputs(_lib, batch=64, num_q=1, num_k=131072)
    assert lib.dsa_indexer_workspace_bytes(1, ctypes.byref(dec), 2048, None) <= _lib.NOALLOC_SCRATCH_BYTES
    # argument errors come first, as for dsa_indexer_topk
    assert lib.dsa_indexer_topk_noalloc(ctypes.byref(_inputs(_lib, heads=32)), 16, None, None, None) == 2
    assert lib.dsa_indexer_topk_noalloc(ctypes.byref(_inputs(_lib)), 0, None, None, None) == 1


@pytest.mark.parametrize("dtype,mode,iters,wg_null", [
    (2, 0, 16, False),   # unknown dtype
    (0, 3, 16, False),   # unknown mode
    (1, 2, 16, False),   # the |x| form is bf16 only
    (0, 1, 15, False),   # odd iteration count
    (1, 0, 0, False),    # no iterations
    (0, 0, 16, True),    # nowhere to report the workgroup count
])
def test_mfma_ceiling_arguments(lib, dtype, mode, iters, wg_null):
    """The sustained-rate probe checks its arguments before any device query."""
    wg = ctypes.c_int32(-7)
    rc = lib.dsa_indexer_mfma_ceiling(dtype, mode, iters, None, 0, None, None if wg_null else ctypes.byref(wg))
    assert rc == 1
    assert wg.value == -7
    assert lib.dsa_indexer_last_error()


def test_anchor_seed_arguments(lib):
    """Anchor seeds need num_seeds >= topk and exclude seed_idx, in the C ABI
    and in the wrapper (which also refuses a raised start with them)."""
    import torch

    from dsa_lightning_indexer_04_amd import _lib

    inp = _inputs(_lib)
    A = _lib.DSA_PRUNE_ANCHOR_SEEDS
    assert lib.dsa_indexer_workspace_bytes(2, ctypes.byref(inp), 16, ctypes.byref(_lib.PruneOpts(16, 0, None, None, A))) > 0
    assert lib.dsa_indexer_workspace_bytes(2, ctypes.byref(inp), 16, ctypes.byref(_lib.PruneOpts(15, 0, None, None, A))) == 0
    assert b"num_seeds" in lib.dsa_indexer_last_error()
    fake = ctypes.c_void_p(FAKE * 4)
    assert lib.dsa_indexer_workspace_bytes(2, ctypes.byref(inp), 16, ctypes.byref(_lib.PruneOpts(16, 0, fake, None, A))) == 0
    assert b"seed_idx" in lib.dsa_indexer_last_error()
    z = [torch.zeros(1)] * 4
    with pytest.raises(ValueError, match="seeds must be"):
        _lib.topk_pruned(*z, 16, seeds="history")
    with pytest.raises(ValueError, match="tau"):
        _lib.topk_pruned(*z, 16, seeds="anchor", start="raised")
    with pytest.raises(ValueError, match="seed_idx"):
        _lib.topk_pruned(*z, 16, seeds="anchor", seed_idx=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="num_seeds"):
        _lib.topk_pruned(*z, 2048, seeds="anchor", num_seeds=1024)
