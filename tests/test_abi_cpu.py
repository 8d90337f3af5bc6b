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
