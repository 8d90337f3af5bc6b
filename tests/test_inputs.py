"""The seeded input generators: determinism, shapes, fp8 scaling, seeds."""
import numpy as np
import torch

from dsa_lightning_indexer_04_amd import inputs
from oracle import indexer


def test_deterministic_and_shaped():
    a = inputs.make_inputs(2, 5, 40, "bf16", "iid", seed=3)
    b = inputs.make_inputs(2, 5, 40, "bf16", "iid", seed=3)
    for key in ("q", "k", "w", "pos"):
        assert torch.equal(a[key], b[key])
    assert a["q"].shape == (2, 5, 64, 128) and a["q"].dtype == torch.bfloat16
    assert a["k"].shape == (2, 40, 128)
    assert a["w"].shape == (2, 5, 64) and a["w"].dtype == torch.float32
    assert a["pos"].tolist() == [[35, 36, 37, 38, 39]] * 2
    c = inputs.make_inputs(2, 5, 40, "bf16", "iid", seed=4)
    assert not torch.equal(a["q"], c["q"])


def test_fp8_quantisation():
    d = inputs.make_inputs(1, 3, 50, "fp8", "clustered", seed=0)
    assert d["q"].dtype == torch.float8_e4m3fn and d["k"].dtype == torch.float8_e4m3fn
    assert torch.all(d["q_scale"] > 0) and torch.all(d["k_scale"] > 0)
    assert d["q_scale"].shape == (1, 3) and d["k_scale"].shape == (1, 50)
    # decoded codes stay within the e4m3 range and the per-row max hits 448
    kc = indexer.decode_e4m3fn(inputs.to_bits(d["k"]))
    assert np.all(np.isfinite(kc)) and np.abs(kc).max() <= 448
    assert np.allclose(np.abs(kc).max(axis=-1), 448)
    # dequantised values are close to the fp32 draw (relative error of e4m3 is <= 2^-4)
    ref = inputs.make_inputs(1, 3, 50, "bf16", "clustered", seed=0)
    kf = indexer.decode_bf16(inputs.to_bits(ref["k"]))
    deq = kc * d["k_scale"].numpy()[..., None]
    assert np.max(np.abs(deq - kf)) <= 2.0**-4 * np.abs(kf).max() + 1e-6


def test_clustered_structure():
    d = inputs.make_inputs(1, 8, 2000, "bf16", "clustered", seed=0)
    k = d["k"].float().numpy()[0]
    norms = np.linalg.norm(k, axis=1)
    # centroid norm 3 plus noise 0.3 per coordinate: norm near sqrt(9 + 0.09*128)
    assert 3.5 < norms.mean() < 5.5
    w = d["w"].numpy()
    assert 0.15 < (w < 0).mean() < 0.45


def test_evenly_spaced_seeds():
    s = inputs.evenly_spaced_seeds(12288, 1032191)
    assert s.size == 12288 and s[0] == 0 and s[-1] <= 1032191
    assert np.all(np.diff(s) > 0)
    s2 = inputs.evenly_spaced_seeds(100, 49)
    np.testing.assert_array_equal(s2, np.arange(50))


def test_workload_pair_counts():
    wl = inputs.WORKLOADS
    assert wl["tiny_prefill_1k"].visible_pairs == 524800
    assert wl["prefill_32k"].visible_pairs == 536887296
    assert wl["decode_64x128k"].visible_pairs == 8388608
    assert wl["chunked_prefill_128k"].visible_pairs == 1040191488
    assert wl["context_1m_fp8"].visible_pairs == 17045659648


def test_projection_inputs():
    a = inputs.make_projection_inputs(6, 256, 128, seed=2)
    b = inputs.make_projection_inputs(6, 256, 128, seed=2)
    for key in ("c_q", "x", "w_iq", "w_ik", "w_iw"):
        assert torch.equal(a[key], b[key]) and a[key].dtype == torch.bfloat16
    assert a["c_q"].shape == (6, 128) and a["x"].shape == (6, 256)
    assert a["w_iq"].shape == (64 * 128, 128) and a["w_ik"].shape == (128, 256) and a["w_iw"].shape == (64, 256)
    # N(0, 1/fan_in) weights: the projections have about unit variance
    q = a["c_q"].float() @ a["w_iq"].float().T
    assert 0.7 < float(q.std()) < 1.3


def test_mla_inputs_and_selection():
    d = inputs.make_mla_inputs(2, 3, 100, seed=1)
    assert d["q"].shape == (2, 3, 128, 576) and d["kv"].shape == (2, 100, 576)
    assert d["q"].dtype == torch.bfloat16 and 0.9 < float(d["kv"].float().std()) < 1.1
    pos = np.array([[99, 5, -1], [10, 99, 0]])
    sel = inputs.random_selection(2, 3, 100, 16, pos, seed=1)
    assert sel.shape == (2, 3, 16) and sel.dtype == np.int32
    for b in range(2):
        for t in range(3):
            vis = max(0, min(pos[b, t] + 1, 100))
            m = min(16, vis)
            row = sel[b, t]
            assert np.all(row[m:] == -1)
            assert len(set(row[:m].tolist())) == m and np.all((row[:m] >= 0) & (row[:m] < vis))
