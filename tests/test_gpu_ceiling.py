"""The benchmark aids of dsa_indexer_profile.h.  The sustained-rate probe
(dsa_indexer_mfma_ceiling) runs the score step on synthetic operands: it
launches two workgroups per compute unit, is deterministic, and rejects an
output buffer that is too small.  Timing windows count each launch once."""
import pytest
import torch

from dsa_lightning_indexer_04_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,mode", [("bf16", 0), ("bf16", 1), ("bf16", 2), ("fp8", 0), ("fp8", 1)])
def test_probe_runs_and_is_deterministic(dtype, mode):
    wg = _lib.mfma_ceiling(dtype, mode, 64)
    assert wg == 2 * torch.cuda.get_device_properties(0).multi_processor_count
    a = torch.full((wg * 256,), float("nan"), device="cuda")
    b = torch.full((wg * 256,), float("nan"), device="cuda")
    assert _lib.mfma_ceiling(dtype, mode, 64, a) == wg
    assert _lib.mfma_ceiling(dtype, mode, 64, b) == wg
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)


def test_probe_rejects_a_short_buffer():
    wg = _lib.mfma_ceiling("bf16", 0, 2)
    out = torch.zeros(wg * 256 - 1, device="cuda")
    with pytest.raises(_lib.IndexerError, match="256"):
        _lib.mfma_ceiling("bf16", 0, 2, out)


def test_profile_windows_count_launches_and_reuse_events():
    """Per-kernel timing windows: each launch in a window is counted once with
    a positive mean duration, and a second window (reusing the first one's
    events) counts its own launches only."""
    import numpy as np

    import dsa_lightning_indexer_04_amd as dsa
    from dsa_lightning_indexer_04_amd import inputs

    d = inputs.make_inputs(1, 8, 3000, "bf16", "iid", seed=5)
    q, k, w, pos = (d[n].cuda() for n in ("q", "k", "w", "pos"))
    want = dsa.topk(q, k, w, pos, 64, route="stream")[0].cpu().numpy()
    for calls in (3, 2):
        _lib.profile_begin()
        for _ in range(calls):
            got = dsa.topk(q, k, w, pos, 64, route="stream")[0]
        prof = _lib.profile_end()
        assert set(prof) == {"k_topk_stream"}, prof
        n, ms = prof["k_topk_stream"]
        assert n == calls and ms > 0.0
        assert np.array_equal(got.cpu().numpy(), want)
