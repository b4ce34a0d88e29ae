"""The seeded input generator (CPU): the diagnostic shared-index-query recipe."""
import torch

from block_sparse_gqa_02_amd.configs import PREFILL_32K, PREFILL_32K_SHARED_IQ
from block_sparse_gqa_02_amd.inputs import generate


def test_shared_index_queries_repeat_per_run():
    w = PREFILL_32K_SHARED_IQ.shrink(seq_q=200, seq_kv=200)
    iq = generate(w, "cpu").iq
    for r0 in range(0, 200, 64):
        run = iq[0, r0:min(r0 + 64, 200)]
        assert bool((run == run[0]).all()), f"rows of run {r0} differ"
    assert not bool((iq[0, 0] == iq[0, 64]).all()), "consecutive runs share a draw"


def test_independent_rows_by_default():
    w = PREFILL_32K.shrink(seq_q=128, seq_kv=128)
    iq = generate(w, "cpu").iq
    assert not bool((iq[0, 0] == iq[0, 1]).all())
    # Q, K and V do not depend on the index-query recipe
    a = generate(w, "cpu")
    b = generate(w.shrink(iq_shared_rows=64), "cpu")
    for n in ("q", "k", "v"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
