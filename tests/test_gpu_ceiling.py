"""The sustained-rate probe (dsa_indexer_mfma_ceiling) runs the score step on
synthetic operands: it launches two workgroups per compute unit, is
deterministic, and rejects an output buffer that is too small."""
import pytest
import torch

from dsa_lightning_indexer_04_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", [0, 1])
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
