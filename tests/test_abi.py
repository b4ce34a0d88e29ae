"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import block_sparse_gqa_02_amd as msa
from block_sparse_gqa_02_amd import binding
from block_sparse_gqa_02_amd.configs import ALL, CHUNK_1M, DECODE_32x256K, PREFILL_128K, PREFILL_32K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

A = ctypes.c_void_p(0x10000)       # dummy, 16-byte aligned, never dereferenced
A4 = ctypes.c_void_p(0x10004)      # 4-byte aligned only
NULL = None


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:msa_status|const char\s*\*|int|void)\s+(msa_\w+)\s*\(",
                                 src, re.M)))


def test_header_declares_entry_points():
    names = declared()
    for n in ["msa_index_block_scores", "msa_topk_blocks", "msa_index_topk_fused",
              "msa_sparse_attn_prefill", "msa_sparse_attn_decode", "msa_dense_attn_prefill",
              "msa_dense_attn_decode", "msa_workspace_bytes", "msa_status_string",
              "msa_last_error", "msa_abi_version", "msa_index_block_scores_paged",
              "msa_sparse_attn_decode_paged", "msa_sparse_attn_prefill_backward",
              "msa_index_kl_backward"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    for n in declared():
        assert hasattr(L, n), f"libmsa.so does not export {n}"


def test_abi_version_and_status_strings():
    L = binding.lib()
    assert L.msa_abi_version() == 6
    for code, name in binding.STATUS.items():
        assert L.msa_status_string(code).decode() == name


def prob(w=PREFILL_128K, **kw):
    return msa.Problem.from_workload(w, **kw).c()


def call(name, *args):
    L = binding.lib()
    return getattr(L, name)(*args), L.msa_last_error().decode()


def P(p):
    return ctypes.byref(p)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, 2), ("idx_head_dim", 128, 2), ("block_size", 128, 2),
    ("n_idx_heads", 8, 2), ("n_kv_heads", 8, 2), ("n_q_heads", 30, 1),
    ("top_k", 0, 1), ("top_k", 257, 2), ("batch", 0, 1), ("seq_kv", 100, 1),
    ("q_start", -1, 1), ("n_q_heads", 4 * 17, 2),
])
def test_topk_validation(field, value, code):
    p = prob(**{field: value})
    st, msg = call("msa_topk_blocks", P(p), A, NULL, A, NULL)
    assert st == code, (st, msg)
    assert msg


def test_null_and_misaligned_pointers():
    p = prob()
    assert call("msa_index_block_scores", P(p), NULL, A, NULL, A, NULL)[0] == 1
    assert call("msa_index_block_scores", P(p), A4, A, NULL, A, NULL)[0] == 1  # bf16: 16 B
    assert call("msa_sparse_attn_prefill", P(p), A, A, A, NULL, A, NULL, NULL, 0, NULL)[0] == 1
    assert call("msa_sparse_attn_prefill", P(p), A, A, A, A4, A4, NULL, NULL, 0, NULL)[0] == 1
    assert call("msa_dense_attn_prefill", P(p), A, NULL, A, A, NULL, NULL, 0, NULL)[0] == 1
    assert call("msa_index_block_scores", None, A, A, NULL, A, NULL)[0] == 1


def test_decode_shape_rules():
    p = prob(DECODE_32x256K)
    # decode needs seq_q == 1
    bad = prob(DECODE_32x256K, seq_q=2)
    assert call("msa_sparse_attn_decode", P(bad), A, A, A, A4, A4, A, NULL, A, 1 << 30, NULL)[0] == 1
    # workspace too small
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(p), 4, ctypes.byref(need))[0] == 0 and need.value > 0
    st, msg = call("msa_sparse_attn_decode", P(p), A, A, A, A4, A4, A, NULL, A, need.value - 1, NULL)
    assert st == 3 and "workspace" in msg
    st, _ = call("msa_dense_attn_decode", P(p), A, A, A, NULL, A, NULL, A, 1 << 40, NULL)
    assert st == 1  # seq_lens required


def test_paged_decode_rules():
    p = prob(DECODE_32x256K)
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(p), 4, ctypes.byref(need))[0] == 0
    # index scores: page table, pool size, decode shape
    assert call("msa_index_block_scores_paged", P(p), A, A, NULL, 8, A4, A4, NULL)[0] == 1
    st, msg = call("msa_index_block_scores_paged", P(p), A, A, A4, 0, A4, A4, NULL)
    assert st == 1 and "num_pages" in msg
    bad = prob(DECODE_32x256K, seq_q=2)
    assert call("msa_index_block_scores_paged", P(bad), A, A, A4, 8, A4, A4, NULL)[0] == 1
    assert call("msa_index_block_scores_paged", P(p), A, A4, A4, 8, A4, A4, NULL)[0] == 1  # pool: 16 B
    # attention: every pointer, pool size, workspace
    args = [A, A, A, A4, 8, A4, A4, A, NULL, A, need.value, NULL]
    for i in (0, 1, 2, 3, 5, 6, 7, 9):
        a = list(args)
        a[i] = NULL
        assert call("msa_sparse_attn_decode_paged", P(p), *a)[0] == 1, i
    a = list(args)
    a[4] = -1
    assert call("msa_sparse_attn_decode_paged", P(p), *a)[0] == 1
    a = list(args)
    a[10] = need.value - 1
    st, msg = call("msa_sparse_attn_decode_paged", P(p), *a)
    assert st == 3 and "workspace" in msg


def test_fused_rules():
    p = prob(CHUNK_1M)
    # seq_lens selects the decode form, which needs a decode problem (seq_q == 1)
    st, msg = call("msa_index_topk_fused", P(p), A, A, A4, A4, A, 1 << 40, NULL)
    assert st == 1 and "decode" in msg, msg
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(p), 2, ctypes.byref(need))[0] == 0
    if need.value:
        st, msg = call("msa_index_topk_fused", P(p), A, A, NULL, A4, A, need.value - 1, NULL)
        assert st == 3, msg


def test_fused_decode_rules():
    """Decode form of the fused index + top-k: block scores, then B arrival
    counters at the end of the workspace; pointers and size checked first."""
    d = prob(DECODE_32x256K)
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(d), 8, ctypes.byref(need))[0] == 0
    assert need.value == (1 << 20) + 32 * 4 * 4096 * 4
    st, msg = call("msa_index_topk_fused", P(d), A, A, A4, A4, A, need.value - 1, NULL)
    assert st == 3 and "workspace" in msg, msg
    st, msg = call("msa_index_topk_fused", P(d), A, A, A4, A4, NULL, need.value, NULL)
    assert st == 1, msg
    st, msg = call("msa_index_topk_fused_paged", P(d), A, A, A4, 0, A4, A4, A, need.value, NULL)
    assert st == 1 and "num_pages" in msg, msg
    st, msg = call("msa_index_topk_fused_paged", P(d), A, A, NULL, 5, A4, A4, A, need.value, NULL)
    assert st == 1, msg
    # more sequences than the fixed counter region holds
    big = prob(DECODE_32x256K, batch=65535)  # 9 counters per sequence
    st, msg = call("msa_index_topk_fused", P(big), A, A, A4, A4, A, 1 << 60, NULL)
    assert st == 2 and "counters" in msg, msg
    # prefill problems have no decode workspace
    assert call("msa_workspace_bytes", P(prob(PREFILL_32K)), 8, ctypes.byref(need))[0] != 0


def test_workspace_bytes_every_op_and_workload():
    for w in ALL:
        p = prob(w)
        for op in range(9):
            is_decode_op = op in (4, 6, 8)
            out = ctypes.c_size_t(12345)
            st, msg = call("msa_workspace_bytes", P(p), op, ctypes.byref(out))
            if is_decode_op and not w.decode:
                continue  # decode ops need seq_q == 1
            if op in (2, 7) and w.decode:
                continue
            assert st == 0, (w.name, op, msg)
    assert call("msa_workspace_bytes", P(prob()), 99, ctypes.byref(ctypes.c_size_t()))[0] == 1
    assert call("msa_workspace_bytes", P(prob()), 0, None)[0] == 1


def test_sparse_prefill_workspace_rules():
    """The tiled sparse prefill (G = 4 or 8) needs a workspace of one 16 KiB
    transposed V tile per (sequence, KV head, context block); the row-wise
    kernel (other G) and token-level selection need none."""
    p = prob()  # 128K, G = 8
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(p), 3, ctypes.byref(need))[0] == 0
    assert need.value == 1 * 4 * (131072 // 64) * 16384 + 256
    off = ctypes.c_size_t()
    assert call("msa_sparse_attn_prefill_status_offset", P(p), ctypes.byref(off))[0] == 0
    assert off.value == need.value - 256 and off.value % 256 == 0
    st, msg = call("msa_sparse_attn_prefill", P(p), A, A, A, A4, A, NULL, A, need.value - 1, NULL)
    assert st == 3 and "workspace" in msg, msg
    st, msg = call("msa_sparse_attn_prefill", P(p), A, A, A, A4, A, NULL, NULL, need.value, NULL)
    assert st == 1, msg
    chunk = prob(CHUNK_1M)  # context = q_start + seq_q = 1048576 tokens
    assert call("msa_workspace_bytes", P(chunk), 3, ctypes.byref(need))[0] == 0
    assert need.value >= 4 * (1048576 // 64) * 16384 + 256
    for kw in (dict(n_q_heads=8), dict(block_size=1, top_k=4096)):  # G = 2; tokens
        assert call("msa_workspace_bytes", P(prob(**kw)), 3, ctypes.byref(need))[0] == 0
        assert need.value == 0, kw
        st, msg = call("msa_sparse_attn_prefill_status_offset", P(prob(**kw)), ctypes.byref(off))
        assert st == 2 and "bounded" in msg, msg
    assert call("msa_sparse_attn_prefill_status_offset", P(p), NULL)[0] == 1


@pytest.mark.parametrize("scale", [0.0, -0.088, float("-inf"), float("nan")])
def test_softmax_scale_must_be_positive(scale):
    """A scale <= 0 is rejected before launch by every entry point (the tiled
    kernels take the running max on unscaled scores); non-finite is invalid."""
    p = prob(softmax_scale=scale)
    code = 2 if scale == scale and abs(scale) != float("inf") else 1
    st, msg = call("msa_sparse_attn_prefill", P(p), A, A, A, A4, A, NULL, A, 1 << 40, NULL)
    assert st == code and "softmax_scale" in msg, (st, msg)
    d = prob(DECODE_32x256K, softmax_scale=scale)
    st, msg = call("msa_sparse_attn_decode", P(d), A, A, A, A4, A4, A, NULL, A, 1 << 40, NULL)
    assert st == code and "softmax_scale" in msg, (st, msg)


def test_static_decode_rules():
    """The allocation-free decode validates like msa_sparse_attn_decode and
    refuses, before touching the GPU, problems whose partials exceed its 16 MiB."""
    d = prob(DECODE_32x256K)
    assert call("msa_sparse_attn_decode_static", P(d), NULL, A, A, A4, A4, A, NULL, NULL)[0] == 1
    assert call("msa_sparse_attn_decode_static", P(d), A, A, A, A4, NULL, A, NULL, NULL)[0] == 1
    big = prob(DECODE_32x256K, batch=4096)
    st, msg = call("msa_sparse_attn_decode_static", P(big), A, A, A, A4, A4, A, NULL, NULL)
    assert st == 3 and "scratch" in msg, msg
    st, msg = call("msa_sparse_attn_decode_static", P(prob()), A, A, A, A4, A4, A, NULL, NULL)
    assert st == 1 and "seq_q" in msg, msg  # a prefill problem


def test_wait_limit_knob_is_host_only():
    L = binding.lib()
    L.msa_set_wait_limit(5)
    L.msa_set_wait_limit(0)  # back to the default


def test_token_level_rules():
    """Block size 1 (token-level selection): accepted by the index scores, the
    top-k and the sparse prefill at prefill positions, with top_k up to 65536
    tokens; every other entry point and decode positions reject it."""
    p = prob(PREFILL_32K, block_size=1, top_k=2048)
    need = ctypes.c_size_t(7)
    for op in (0, 1, 3):
        assert call("msa_workspace_bytes", P(p), op, ctypes.byref(need))[0] == 0 and need.value == 0
    for op in (2, 5, 7):
        st, msg = call("msa_workspace_bytes", P(p), op, ctypes.byref(need))
        assert st == 2 and "block_size 1" in msg, (op, msg)
    st, msg = call("msa_index_topk_fused", P(p), A, A, NULL, A4, A, 1 << 40, NULL)
    assert st == 2 and "block_size 1" in msg, msg
    # decode positions
    d = prob(DECODE_32x256K, block_size=1, top_k=4096)
    st, msg = call("msa_index_block_scores", P(d), A, A, A4, A4, NULL)
    assert st == 2 and "prefill" in msg, msg
    st, msg = call("msa_sparse_attn_decode", P(d), A, A, A, A4, A4, A, NULL, A, 1 << 40, NULL)
    assert st == 2, msg
    # k limits: tokens up to 65536, blocks up to 256
    assert call("msa_topk_blocks", P(prob(PREFILL_32K, block_size=1, top_k=65537)), A4, NULL, A4,
                NULL)[0] == 2
    assert call("msa_workspace_bytes", P(prob(PREFILL_32K, block_size=1, top_k=65536)), 1,
                ctypes.byref(need))[0] == 0
    assert call("msa_workspace_bytes", P(prob(PREFILL_32K, top_k=2048)), 1,
                ctypes.byref(need))[0] == 2
    # pointers are still checked
    assert call("msa_topk_blocks", P(p), NULL, NULL, A4, NULL)[0] == 1
    assert call("msa_sparse_attn_prefill", P(p), A, A, A, NULL, A, NULL, NULL, 0, NULL)[0] == 1


def test_index_kl_rules():
    """Host-side checks of the index KL gradient entry: workspace size, missing
    or misaligned pointers, the supported group sizes, caches too long for the
    LDS block mask, rows past the cache."""
    p = prob()
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(p), 9, ctypes.byref(need))[0] == 0
    # the index log-sum-exp (B * 4 * Sq fp32) plus the inverse row lists
    assert need.value >= 4 * 4 * 131072 + 4 * 131072 * 64 * 4
    args = [A, A, A, A, A4, A4, A4, A, A]
    st, msg = call("msa_index_kl_backward", P(p), *args, A, need.value - 1, NULL)
    assert st == 3, msg
    st, msg = call("msa_index_kl_backward", P(p), *args, NULL, need.value, NULL)
    assert st == 1, msg
    for i in range(len(args)):
        a = list(args)
        a[i] = NULL
        assert call("msa_index_kl_backward", P(p), *a, A, need.value, NULL)[0] == 1, i
    # diq must be 16-byte aligned (vector stores)
    a = list(args)
    a[7] = A4
    assert call("msa_index_kl_backward", P(p), *a, A, need.value, NULL)[0] == 1
    # G = 2 (8 query heads over 4 KV heads) is not implemented
    st, msg = call("msa_index_kl_backward", P(prob(n_q_heads=8)), *args, A, 1 << 40, NULL)
    assert st == 2 and "index KL" in msg, msg
    # G = 4 with one KV head (four index heads per KV head), G = 4 over 2 KV
    # heads, and G = 16 are accepted
    assert call("msa_workspace_bytes", P(prob(n_q_heads=4, n_kv_heads=1)), 9,
                ctypes.byref(need))[0] == 0
    assert call("msa_workspace_bytes", P(prob(n_q_heads=8, n_kv_heads=2)), 9,
                ctypes.byref(need))[0] == 0
    assert call("msa_workspace_bytes", P(prob(n_q_heads=16, n_kv_heads=1)), 9,
                ctypes.byref(need))[0] == 0
    # the block mask of 2M cached tokens does not fit LDS
    big = prob(CHUNK_1M, seq_kv=2 * 1048576)
    assert call("msa_workspace_bytes", P(big), 9, ctypes.byref(need))[0] == 2
    # rows past the cache; decode positions are not accepted
    assert call("msa_workspace_bytes", P(prob(q_start=1)), 9, ctypes.byref(need))[0] == 1


def test_binding_raises_with_detail():
    p = msa.Problem.from_workload(PREFILL_128K, head_dim=64)
    with pytest.raises(msa.MsaError, match="UNSUPPORTED"):
        msa.msa_workspace_bytes(p, "sparse_attn_prefill")


def test_backward_rules():
    """Host-side checks of the main-branch gradient entry: workspace size,
    group sizes that do not divide 64, caches too long for the LDS bitmap,
    missing pointers, rows past the cache."""
    p = prob()
    need = ctypes.c_size_t()
    assert call("msa_workspace_bytes", P(p), 7, ctypes.byref(need))[0] == 0
    assert need.value > 0
    args = [A, A, A, A4, A, A4, A, A, A, A]
    st, msg = call("msa_sparse_attn_prefill_backward", P(p), *args, A, need.value - 1, NULL)
    assert st == 3, msg
    st, msg = call("msa_sparse_attn_prefill_backward", P(p), *args, NULL, need.value, NULL)
    assert st == 1, msg
    for i in range(len(args)):
        a = list(args)
        a[i] = NULL
        assert call("msa_sparse_attn_prefill_backward", P(p), *a, A, need.value, NULL)[0] == 1, i
    # 12 query heads over 4 KV heads: G = 3 does not divide 64
    st, msg = call("msa_sparse_attn_prefill_backward", P(prob(n_q_heads=12)), *args, A,
                   1 << 40, NULL)
    assert st == 2 and "divide 64" in msg, msg
    # the block bitmap of 2M cached tokens does not fit LDS
    big = prob(CHUNK_1M, seq_kv=2 * 1048576)
    assert call("msa_workspace_bytes", P(big), 7, ctypes.byref(need))[0] == 2
    # rows past the cache
    bad = prob(q_start=1)
    assert call("msa_workspace_bytes", P(bad), 7, ctypes.byref(need))[0] == 1
