"""GPU parity of the indexer projections (dsa_indexer_project).

Checks, on the same seeded bf16 operands:
  * products: the fp32 projections (out="f32") lie within the fp32
    accumulation bound gamma_n * sum|a*w| of the float64 oracle, n = the
    contraction length (any summation order satisfies it);
  * conversion: fp8 codes and scales, and bf16 bits, equal bit for bit the
    oracle's conversion of the GPU's own fp32 projections (every decision
    taken in fp32 on both sides); the head weights equal the fp32 ones;
  * rounding of the conversion instruction: one-hot latent rows read chosen
    weights back, so rows hold e4m3 midpoints, subnormals and signed values;
  * composition: projected fp8 q/k/w of one sequence give, through
    dsa_indexer_topk, a Top-K that passes the oracle's check.
"""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_04_amd as dsa
from dsa_lightning_indexer_04_amd import inputs
from helpers import OracleRows, assert_rows_ok, log, need_gpu
from oracle import indexer, project

pytestmark = pytest.mark.gpu

U32 = 2.0**-24


def gamma(n: int) -> float:
    return n * U32 / (1 - n * U32)


def _dec(t: torch.Tensor) -> np.ndarray:
    return indexer.decode_bf16(inputs.to_bits(t.cpu()))


def _run(d: dict, modes=("f32", "fp8", "bf16"), block_tokens: int = 0) -> dict:
    dev = {k: v.cuda() for k, v in d.items()}
    args = (dev["c_q"], dev["x"], dev["w_iq"], dev["w_ik"], dev["w_iw"])
    out = {m: dsa.project(*args, out=m, block_tokens=block_tokens) for m in modes}
    torch.cuda.synchronize()
    return {m: {k: (None if v is None else v.cpu()) for k, v in r.items()} for m, r in out.items()}


def _check_products(d: dict, res: dict, tokens: np.ndarray):
    cq, x = _dec(d["c_q"][tokens]), _dec(d["x"][tokens])
    wq, wk, ww = _dec(d["w_iq"]), _dec(d["w_ik"]), _dec(d["w_iw"])
    q, k, w = project.project(cq, x, wq, wk, ww)
    bq, bk, bw = project.projection_abs_bound(cq, x, wq, wk, ww)
    L, D = cq.shape[1], x.shape[1]
    f = res["f32"]
    for name, got, ref, bnd, n in (
        ("q", f["q"].numpy()[tokens], q, bq, L),
        ("k", f["k"].numpy()[tokens], k, bk, D),
        ("w", f["w"].numpy()[tokens], w, bw, D),
    ):
        err = np.abs(got.astype(np.float64) - ref)
        lim = gamma(n) * bnd
        bad = np.argwhere(err > lim)
        assert bad.size == 0, f"{name}: {bad.shape[0]} outputs outside the fp32 bound, first {bad[:3].tolist()}"
        log(f"  {name}: max |err| / bound = {float((err / np.maximum(lim, 1e-300)).max()):.3e}")


def _check_conversion(res: dict):
    f = res["f32"]
    q32, k32 = f["q"].numpy(), f["k"].numpy()
    qc, qs, kc, ks = project.quantize_projection(q32, k32, "fp8")
    g = res["fp8"]
    np.testing.assert_array_equal(g["q_scale"].numpy(), qs)
    np.testing.assert_array_equal(g["k_scale"].numpy(), ks)
    gq, gk = inputs.to_bits(g["q"]), inputs.to_bits(g["k"])
    bad = np.argwhere(gq != qc)
    assert bad.size == 0, f"{bad.shape[0]} q codes differ, first {[(tuple(i), float(q32[tuple(i)])) for i in bad[:3]]}"
    np.testing.assert_array_equal(gk, kc)
    qb, _, kb, _ = project.quantize_projection(q32, k32, "bf16")
    np.testing.assert_array_equal(inputs.to_bits(res["bf16"]["q"]), qb)
    np.testing.assert_array_equal(inputs.to_bits(res["bf16"]["k"]), kb)
    for m in ("fp8", "bf16"):
        np.testing.assert_array_equal(res[m]["w"].numpy().view(np.uint32), f["w"].numpy().view(np.uint32))


@pytest.mark.parametrize(
    "T,hidden,q_latent,block",
    [
        (300, 1024, 512, None),  # one block
        (1, 7168, 1536, None),  # one decode token
        (4396, 7168, 1536, None),  # DeepSeek-V3.2 sizes, one block
        (4396, 7168, 1536, 1024),  # five token blocks, the last one ragged
    ],
)
def test_projection_parity(T, hidden, q_latent, block):
    need_gpu()
    log(f"[project] T={T} hidden={hidden} q_latent={q_latent} block={block}")
    d = inputs.make_projection_inputs(T, hidden, q_latent, seed=T)
    res = _run(d, block_tokens=block or 0)
    if T <= 512:
        tokens = np.arange(T)
    else:
        rng = np.random.default_rng(0)
        tokens = np.unique(np.concatenate([[0, 1023, 1024, 4095, 4096, T - 1], rng.choice(T, 60, replace=False)]))
    _check_products(d, res, tokens)
    _check_conversion(res)


def test_projection_zero_rows():
    need_gpu()
    d = inputs.make_projection_inputs(70, 256, 128, seed=3)
    d["c_q"][5] = 0
    d["x"][7] = 0
    d["c_q"][9] = 0
    d["x"][9] = 0
    res = _run(d)
    _check_products(d, res, np.arange(70))
    _check_conversion(res)
    g = res["fp8"]
    assert g["q_scale"][5].item() == 1.0 and g["k_scale"][7].item() == 1.0
    assert not inputs.to_bits(g["q"][9]).any() and not inputs.to_bits(g["k"][9]).any()


def test_conversion_rounding_of_chosen_values():
    """Latent row t is one-hot at column t, so query row t reads column t of
    the stored W_IQ back: each row carries 448 (so its scale is 1 and codes are
    the plain e4m3 rounding) and a set of bf16 values at and beside e4m3
    midpoints, in both signs, including subnormal ones."""
    need_gpu()
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo, hi = indexer.decode_e4m3fn(codes), indexer.decode_e4m3fn(codes + 1)
    m = (lo + hi) / 2
    # keep the midpoints a bf16 can hold exactly, and their bf16 neighbours
    mb = torch.from_numpy(m.astype(np.float32)).to(torch.bfloat16).double().numpy()
    mids = m[mb == m]
    # one bf16 ulp above and below each (positive) midpoint
    mb16 = torch.from_numpy(mids.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    up = (mb16 + 1).view(torch.bfloat16).double().numpy()
    down = (mb16 - 1).view(torch.bfloat16).double().numpy()
    vals = np.concatenate([[448.0], mids, -mids, up, -down, [2.0**-10, -(2.0**-10), 3 * 2.0**-10, 0.0]])
    assert np.all(up > mids) and np.all(down < mids)
    n = vals.size
    assert n <= 8192
    T, L, D = 64, 64, 64
    d = inputs.make_projection_inputs(T, D, L, seed=1)
    d["c_q"].zero_()
    for t in range(T):
        d["c_q"][t, t % L] = 1.0
    col = np.zeros(8192)
    col[:n] = vals
    wq = torch.from_numpy(np.tile(col[:, None], (1, L))).to(torch.bfloat16)
    # vary the row order per latent column so codes land in every lane position
    for c in range(L):
        wq[:, c] = wq[:, c].roll(c * 37)
    d["w_iq"] = wq.contiguous()
    res = _run(d, modes=("f32", "fp8"))
    g = res["fp8"]
    assert np.all(g["q_scale"].numpy() == 1.0)
    q32 = res["f32"]["q"].numpy().reshape(T, -1)
    np.testing.assert_array_equal(q32, wq.double().numpy()[:, np.arange(T) % L].T.astype(np.float32))
    want = project.e4m3fn_rne(q32.astype(np.float64))
    got = inputs.to_bits(g["q"]).reshape(T, -1)
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(float(q32[tuple(i)]), hex(got[tuple(i)]), hex(want[tuple(i)])) for i in bad[:5]]


def test_projected_inputs_feed_the_topk():
    need_gpu()
    T, k = 600, 64
    d = inputs.make_projection_inputs(T, 512, 256, seed=11)
    dev = {n: v.cuda() for n, v in d.items()}
    r = dsa.project(dev["c_q"], dev["x"], dev["w_iq"], dev["w_ik"], dev["w_iw"], out="fp8")
    pos = torch.arange(T, dtype=torch.int32, device="cuda")[None]
    q, kk, w = r["q"][None], r["k"][None], r["w"][None]
    qs, ks = r["q_scale"][None], r["k_scale"][None]
    idx, sc = dsa.topk(q, kk, w, pos, k, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    cpu = {"q": q.cpu(), "k": kk.cpu(), "w": w.cpu(), "pos": pos.cpu(), "q_scale": qs.cpu(), "k_scale": ks.cpu(),
           "dtype": "fp8"}
    orc = OracleRows(cpu)
    rows = [(0, t) for t in (0, 1, 63, 64, 65, 300, T - 1)]
    assert_rows_ok(orc, idx.cpu().numpy(), sc.cpu().numpy(), rows, k)
