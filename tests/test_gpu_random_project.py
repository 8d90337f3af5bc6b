"""GPU parity of the indexer projections on seeded random shapes (each case
drawn from rng(case)): 1..2499 tokens, hidden and q_latent any multiple of 8
up to 4096 / 2048, and a token block of 64..1024 tokens or the default.  The
checks are those of test_gpu_project: fp32 products within the fp32
accumulation bound of the float64 oracle (on up to 40 sampled tokens), fp8
and bf16 conversion bit for bit equal to the oracle's conversion of the
GPU's own fp32 products."""
import numpy as np
import pytest

from dsa_lightning_indexer_04_amd import inputs
from helpers import log, need_gpu
from test_gpu_project import _check_conversion, _check_products, _run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", range(8))
def test_random_projection(case):
    need_gpu()
    rng = np.random.default_rng(3000 + case)
    T = int(rng.integers(1, 2500))
    hidden = 8 * int(rng.integers(1, 513))
    q_latent = 8 * int(rng.integers(1, 257))
    block = int(rng.choice([0, 64, 100, 1024]))
    log(f"random projection case {case}: T={T} hidden={hidden} q_latent={q_latent} block={block or 'default'}")
    d = inputs.make_projection_inputs(T, hidden, q_latent, seed=case)
    res = _run(d, block_tokens=block)
    tokens = np.arange(T) if T <= 40 else np.unique(np.concatenate([[0, T - 1], rng.choice(T, 38, replace=False)]))
    _check_products(d, res, tokens)
    _check_conversion(res)
