"""Host-side logic of bench.py (no GPU): the one-GPU rule, the algorithmic
work counters against brute force, and the measured-traffic table's
bookkeeping."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_gqa_02_amd.configs import ALL, TINY_PREFILL_2K  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "one MI355X" in r.stderr, r.stderr


def _brute_force(w):
    """Attended (row, KV head, key) triples and scored (row, key) pairs by
    walking every row's blocks: a row keeps min(k, cur + 1) blocks, every kept
    block other than its own contributes 64 keys and the own block pos % 64 + 1;
    the index branch scores every key of the blocks before the own block."""
    att = idx = dense = 0
    for t in range(w.seq_q):
        pos = w.q_start + t
        cur = pos // w.block_size
        kept = min(w.top_k, cur + 1)
        keys = 0
        for i in range(kept):
            keys += (pos % w.block_size + 1) if i == 0 else w.block_size
        att += keys
        idx += cur * w.block_size
        dense += pos + 1
    return att * w.batch * w.n_kv_heads, idx * w.batch, dense * w.batch


@pytest.mark.parametrize("shape", [
    dict(seq_q=130, seq_kv=130, q_start=0, top_k=1),
    dict(seq_q=200, seq_kv=900, q_start=700, top_k=3),
    dict(seq_q=64, seq_kv=64, q_start=0, top_k=8),
    dict(seq_q=77, seq_kv=5000, q_start=4923, top_k=40, batch=2),
])
def test_work_counters_match_brute_force(shape):
    w = TINY_PREFILL_2K.shrink(**shape)
    att, idx, dense = _brute_force(w)
    assert bench.attended_keys(w) == att
    assert bench.index_keys(w) == idx
    assert bench.dense_pairs(w) == dense


def test_compulsory_bytes_cover_q_o_and_the_attendable_context():
    for w in ALL:
        if w.decode:
            continue
        b = bench.k4_compulsory_bytes(w)
        q_and_o = 2 * w.batch * w.seq_q * w.n_q_heads * w.head_dim * 2
        assert b > q_and_o


def test_traffic_table_names_known_ops_and_existing_sources():
    for (workload, op), e in bench.MEASURED_TRAFFIC.items():
        assert workload in {w.name for w in ALL}, workload
        assert op in bench.KERNEL_SOURCES, op
        for f in bench.KERNEL_SOURCES[op]:
            assert os.path.exists(os.path.join(bench.CSRC, f)), f
        assert len(e["sha256"]) == 64
        assert e["fetch_bytes"] > 0 and e["write_bytes"] >= 0
        # an entry that matches the sources reports both parts and their sum
        tr = bench.measured_traffic(workload, op)
        if tr is not None:
            assert tr["bytes"] == e["fetch_bytes"] + e["write_bytes"]
