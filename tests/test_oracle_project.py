"""Pins of the projection / quantisation oracle (oracle.project).

Each check rests on something other than the oracle's own formula: a
hand-worked product, one-hot inputs that read single weights back, exact
scaling identities, torch's CPU casts to bfloat16 and float8_e4m3fn (library
routines), the golden e4m3fn code table and round trips through the
already-pinned decoder.
"""
import numpy as np
import pytest
import torch

from conftest import read_table
from oracle import indexer, project

# --------------------------------------------------------------- projections


def test_hand_worked_projection():
    # Q^I = C^Q W_IQ with T=1, d_qc=2, H=1, d=2: C^Q = [1, 2],
    # W_IQ = [[1, 0], [3, -1]]  ->  Q^I = [1*1 + 2*3, 1*0 + 2*(-1)] = [7, -2].
    # K^I = X W_IK with X = [2, -1, 1], W_IK columns (1,0,1) and (0,1,1) -> [3, 0];
    # W^I = X W_IW with W_IW column (1, 1, 1) -> [2].
    c_q = np.array([[1.0, 2.0]])
    w_iq = np.array([[1.0, 0.0], [3.0, -1.0]]).T  # stored out-feature major
    x = np.array([[2.0, -1.0, 1.0]])
    w_ik = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).T
    w_iw = np.array([[1.0], [1.0], [1.0]]).T
    q, k, w = project.project(c_q, x, w_iq, w_ik, w_iw, heads=1)
    assert q.shape == (1, 1, 2) and k.shape == (1, 2) and w.shape == (1, 1)
    assert q.ravel().tolist() == [7.0, -2.0]
    assert k.ravel().tolist() == [3.0, 0.0]
    assert w.ravel().tolist() == [2.0]


def test_one_hot_rows_read_weights_back():
    # a one-hot input row e_i picks input feature i: output o equals the stored
    # weight wt[o, i] (non-square shapes, so a transposed operand cannot pass)
    rng = np.random.default_rng(1)
    H, d, dq, dh, dI = 4, 8, 6, 10, 8
    w_iq = rng.standard_normal((H * d, dq))
    w_ik = rng.standard_normal((dI, dh))
    w_iw = rng.standard_normal((H, dh))
    c_q = np.eye(dq)
    x = np.eye(dh)
    q, k, w = project.project(c_q, x, w_iq, w_ik, w_iw, heads=H)
    assert q.shape == (dq, H, d) and k.shape == (dh, dI) and w.shape == (dh, H)
    np.testing.assert_array_equal(q.reshape(dq, H * d), w_iq.T)
    np.testing.assert_array_equal(k, w_ik.T)
    np.testing.assert_array_equal(w, w_iw.T)
    # head j of query t holds outputs j*d .. j*d+d-1
    np.testing.assert_array_equal(q[3, 2], w_iq[2 * d:3 * d, 3])


def test_projection_homogeneity_and_additivity():
    rng = np.random.default_rng(2)
    c_q, x = rng.standard_normal((5, 6)), rng.standard_normal((5, 10))
    w_iq, w_ik, w_iw = rng.standard_normal((16, 6)), rng.standard_normal((4, 10)), rng.standard_normal((2, 10))
    base = project.project(c_q, x, w_iq, w_ik, w_iw, heads=2)
    twice = project.project(2 * c_q, 2 * x, w_iq, w_ik, w_iw, heads=2)
    for a, b in zip(base, twice):
        np.testing.assert_array_equal(2 * a, b)  # scaling by 2 is exact
    # rows are independent: the projection of a stacked pair is the stack
    top = project.project(c_q[:2], x[:2], w_iq, w_ik, w_iw, heads=2)
    for a, b in zip(base, top):
        np.testing.assert_allclose(a[:2], b, rtol=1e-15, atol=1e-15)


def test_abs_bound_dominates_and_is_tight_for_nonnegative():
    rng = np.random.default_rng(3)
    c_q, x = rng.standard_normal((3, 6)), rng.standard_normal((3, 10))
    w_iq, w_ik, w_iw = rng.standard_normal((8, 6)), rng.standard_normal((4, 10)), rng.standard_normal((2, 10))
    vals = project.project(c_q, x, w_iq, w_ik, w_iw, heads=2)
    bnds = project.projection_abs_bound(c_q, x, w_iq, w_ik, w_iw, heads=2)
    for v, b in zip(vals, bnds):
        assert np.all(np.abs(v) <= b * (1 + 1e-12))
    pos = [np.abs(a) for a in (c_q, x, w_iq, w_ik, w_iw)]
    for v, b in zip(project.project(*pos, heads=2), project.projection_abs_bound(*pos, heads=2)):
        np.testing.assert_allclose(v, b, rtol=1e-14)


# -------------------------------------------------------------------- e4m3fn


def test_e4m3_golden_codes():
    # the OCP code table: every finite value encodes to its own code
    for code_s, val_s in read_table("fp8_e4m3fn_codes.txt"):
        code = int(code_s, 16)
        val = float(val_s)
        if np.isnan(val):
            continue
        got = int(project.e4m3fn_rne(np.array([val]))[0])
        assert got == code, (code_s, val_s, hex(got))


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = indexer.decode_e4m3fn(codes)
    np.testing.assert_array_equal(project.e4m3fn_rne(vals), codes)


def test_e4m3_matches_torch_cast_in_range():
    # torch's CPU float8_e4m3fn cast rounds to nearest even; compare on a dense
    # sweep of fp32 values inside the finite range, plus every midpoint
    rng = np.random.default_rng(4)
    pos_codes = np.arange(0, 0x7E + 1, dtype=np.uint8)
    pv = indexer.decode_e4m3fn(pos_codes)
    mids = (pv[:-1] + pv[1:]) / 2  # exact in float64 and in float32
    sweep = np.concatenate([
        rng.uniform(-448, 448, 20000),
        np.exp2(rng.uniform(-14, 8.8, 20000)) * rng.choice([-1, 1], 20000),
        mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)).astype(np.float64),
    ])
    sweep = sweep[np.abs(sweep) <= 448].astype(np.float32)
    want = torch.from_numpy(sweep).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = project.e4m3fn_rne(sweep.astype(np.float64))
    bad = np.nonzero(want != got)[0]
    assert bad.size == 0, [(float(sweep[i]), hex(want[i]), hex(got[i])) for i in bad[:5]]


def test_e4m3_midpoints_round_to_even_and_saturate():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo, hi = indexer.decode_e4m3fn(codes), indexer.decode_e4m3fn(codes + 1)
    got = project.e4m3fn_rne((lo + hi) / 2)
    even = np.where(codes % 2 == 0, codes, codes + 1)
    np.testing.assert_array_equal(got, even)
    sat = project.e4m3fn_rne(np.array([448.0, 449.0, 464.0, 480.0, 1e30, -500.0, -448.0]))
    assert sat.tolist() == [0x7E] * 5 + [0xFE, 0xFE]
    # signed zeros and underflow keep the sign
    z = project.e4m3fn_rne(np.array([0.0, -0.0, 1e-9, -1e-9, 2.0**-10, 2.0**-10 * 1.0001]))
    assert z.tolist() == [0x00, 0x80, 0x00, 0x80, 0x00, 0x01]


# ----------------------------------------------------------- row quantisation


def test_quantize_rows_invariants():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((64, 8192)) * np.exp2(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    codes, scale = project.quantize_rows_fp8(v)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    dec = indexer.decode_e4m3fn(codes)
    # the amax element of every row maps to the top code
    np.testing.assert_array_equal(np.abs(dec).max(axis=1), 448.0)
    amax = np.abs(v).max(axis=1).astype(np.float64)
    np.testing.assert_allclose(scale, amax / 448.0, rtol=2.0**-23)
    # reconstruction: half an e4m3 quantum (relative 2^-4 for normals, 2^-10
    # absolute in code units below 2^-6) plus the fp32 rounding of x*inv
    err = np.abs(dec * scale[:, None].astype(np.float64) - v)
    code_units = np.abs(v) / scale[:, None]
    bound = np.maximum(code_units * 2.0**-4, 2.0**-10) * (1 + 2.0**-20) + code_units * 2.0**-22
    assert np.all(err <= bound * scale[:, None])
    # odd symmetry
    c_neg, s_neg = project.quantize_rows_fp8(-v)
    np.testing.assert_array_equal(s_neg, scale)
    np.testing.assert_array_equal(c_neg, codes ^ np.uint8(0x80))


def test_quantize_rows_zero_and_exact_rows():
    codes, scale = project.quantize_rows_fp8(np.zeros((2, 16), np.float32))
    assert scale.tolist() == [1.0, 1.0] and codes.tolist() == [[0] * 16] * 2
    # a row whose amax is 448 has inv = 1: codes are the plain e4m3 rounding,
    # which torch's cast gives independently
    row = np.array([[448.0, 1.0625, 1.1875, -3.3, 0.0009765625, 200.0]], np.float32)
    codes, scale = project.quantize_rows_fp8(row)
    assert scale.tolist() == [1.0]
    want = torch.from_numpy(row).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, want)
    assert codes[0, 1] == 0x38 and codes[0, 2] == 0x3A  # 1.0625 -> 1.0, 1.1875 -> 1.25


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(6)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        # exact ties: bf16 value plus half an ulp
        (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
        -(np.arange(1, 2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(project.bf16_rne(v), want)


def test_quantize_projection_shapes():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 4, 8)).astype(np.float32)
    k = rng.standard_normal((3, 8)).astype(np.float32)
    qc, qs, kc, ks = project.quantize_projection(q, k, "fp8")
    assert qc.shape == (3, 4, 8) and qs.shape == (3,) and kc.shape == (3, 8) and ks.shape == (3,)
    # one scale per token over all its heads
    np.testing.assert_array_equal(qs, (np.abs(q).reshape(3, -1).max(1) / np.float32(448)).astype(np.float32))
    qb, none1, kb, none2 = project.quantize_projection(q, k, "bf16")
    assert none1 is None and none2 is None and qb.dtype == np.uint16 and kb.shape == (3, 8)
    with pytest.raises(ValueError):
        project.quantize_projection(q, k, "fp16")
