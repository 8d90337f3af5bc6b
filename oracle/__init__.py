"""CPU oracle for the DSA lightning indexer and its exact per-query Top-K.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code written from the
pages' definitions.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import or run anything in this package; the library
and its Python binding never do.  Nothing here shares code with the HIP path.

Modules:
    indexer  -- exact input decoding, the index score, visibility, Top-K by sort,
                and the acceptance check used against GPU results.
    counts   -- the closed forms the pages print (pair counts, FLOP counts).
    prune    -- the DoSA certificate pieces: seed threshold and the score
                upper bound built from retained heads, projected positive
                heads with a residual term, and a folded negative-head penalty.
    project  -- the indexer projections (Q^I, K^I, W^I) and the per-token
                e4m3fn quantisation of their fp32 results.
    sparse_mla -- the core attention over the selected keys (MLA, MQA mode).
"""
from . import counts, indexer, project, prune, sparse_mla  # noqa: F401
