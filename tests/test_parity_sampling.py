"""The stratified row sample the full-size parity tests check: every stratum
the comparison protocol names is present at the 32K, 128K and 1M-context
sizes (host only)."""
import numpy as np
import pytest

from block_sparse_gqa_02_amd.configs import CHUNK_1M, PREFILL_128K, PREFILL_32K
import parity as PAR


@pytest.mark.parametrize("w", [PREFILL_32K, PREFILL_128K, CHUNK_1M], ids=lambda w: w.name)
def test_sample_covers_every_stratum(w):
    rows = PAR.sample_rows(w.seq_q, w.q_start, w.block_size, seed=5, n_uniform=2048, n_log=32)
    assert np.all(np.diff(rows) > 0) and rows[0] >= 0 and rows[-1] < w.seq_q
    rs = set(rows.tolist())
    bs, q0 = w.block_size, w.q_start
    # all rows of the first two blocks, the last 64 rows
    first_two = range(0, 2 * bs - q0 % bs)
    assert set(first_two) <= rs
    assert set(range(w.seq_q - 64, w.seq_q)) <= rs
    # both boundary rows of >= 32 distinct blocks past the first two
    blocks = PAR.boundary_blocks(w.seq_q, q0, bs, 32)
    assert len(set(blocks)) >= 32
    first_block = q0 // bs
    assert min(blocks) >= first_block + 2
    for c in blocks:
        assert c * bs - q0 in rs and c * bs + bs - 1 - q0 in rs
    # the boundary blocks spread over the whole range (log-spaced up to the last)
    assert max(blocks) == (q0 + w.seq_q - 1) // bs
    # >= 2048 distinct uniform rows on top of the structured strata
    assert len(rows) >= 2048


def test_uniform_rows_are_distinct_draws():
    rows = PAR.sample_rows(8192, 1040384, 64, seed=1024, n_uniform=2048, n_log=32)
    rng = np.random.default_rng(1024)
    uni = rng.choice(8192, size=2048, replace=False)
    assert len(set(uni.tolist())) == 2048 and set(uni.tolist()) <= set(rows.tolist())
