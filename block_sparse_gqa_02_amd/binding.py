"""Thin ctypes binding of libmsa.so: the C entry points under the same names.

Argument marshalling only: every step of the hot path runs in the HIP kernels
of the library.  Tensors are torch tensors on the GPU (torch provides device
memory and the stream); outputs and workspaces are caller-provided, or
allocated here with torch when passed as None.  If the library is missing the
import of any entry point fails loudly; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")

MSA_OK = 0
STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARGUMENT", 2: "MSA_ERR_UNSUPPORTED",
          3: "MSA_ERR_WORKSPACE_TOO_SMALL", 4: "MSA_ERR_HIP"}
OPS = {"index_block_scores": 0, "topk_blocks": 1, "index_topk_fused": 2,
       "sparse_attn_prefill": 3, "sparse_attn_decode": 4, "dense_attn_prefill": 5,
       "dense_attn_decode": 6, "sparse_attn_prefill_backward": 7, "index_topk_fused_decode": 8,
       "index_kl_backward": 9}


class MsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class _CProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq_q", "seq_kv", "q_start", "n_q_heads", "n_kv_heads", "head_dim",
        "n_idx_heads", "idx_head_dim", "block_size", "top_k")] + [("softmax_scale", ctypes.c_float)]


@dataclass
class Problem:
    """Mirror of msa_problem."""
    batch: int
    seq_q: int
    seq_kv: int
    q_start: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_idx_heads: int
    idx_head_dim: int
    block_size: int
    top_k: int
    softmax_scale: float

    @classmethod
    def from_workload(cls, w, **override) -> "Problem":
        kw = {f.name: getattr(w, f.name) for f in fields(cls) if f.name != "softmax_scale"}
        kw["softmax_scale"] = w.softmax_scale
        kw.update(override)
        return cls(**kw)

    def c(self) -> _CProblem:
        return _CProblem(*(int(getattr(self, f.name)) for f in fields(self)
                           if f.name != "softmax_scale"), float(self.softmax_scale))

    @property
    def nblk(self) -> int:
        return (self.seq_kv + self.block_size - 1) // self.block_size


_lib = None


def lib():
    """Load libmsa.so (built by block_sparse_gqa_02_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_gqa_02_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, vp, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
        pr = P(_CProblem)
        sig = {
            "msa_index_block_scores": [pr, vp, vp, vp, vp, vp],
            "msa_topk_blocks": [pr, vp, vp, vp, vp],
            "msa_index_topk_fused": [pr, vp, vp, vp, vp, vp, sz, vp],
            "msa_sparse_attn_prefill": [pr, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_sparse_attn_decode": [pr, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_dense_attn_prefill": [pr, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_dense_attn_decode": [pr, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_workspace_bytes": [pr, ctypes.c_int, P(sz)],
            "msa_index_block_scores_paged": [pr, vp, vp, vp, ctypes.c_int32, vp, vp, vp],
            "msa_sparse_attn_decode_paged": [pr, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp,
                                             vp, sz, vp],
            "msa_sparse_attn_prefill_backward": [pr, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                 sz, vp],
            "msa_index_kl_backward": [pr, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_sparse_attn_prefill_status_offset": [pr, P(sz)],
            "msa_index_topk_fused_paged": [pr, vp, vp, vp, ctypes.c_int32, vp, vp, vp, sz, vp],
            "msa_sparse_attn_decode_static": [pr, vp, vp, vp, vp, vp, vp, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_abi_version.argtypes = []
        L.msa_abi_version.restype = ctypes.c_int
        L.msa_set_wait_limit.argtypes = [ctypes.c_int32]
        L.msa_set_wait_limit.restype = None
        _lib = L
    return _lib


def _check(status: int):
    if status != MSA_OK:
        raise MsaError(status, lib().msa_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def abi_version() -> int:
    return lib().msa_abi_version()


def msa_workspace_bytes(p: Problem, op: str) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().msa_workspace_bytes(ctypes.byref(p.c()), OPS[op], ctypes.byref(out)))
    return out.value


# Operations whose workspace starts with arrival counters that must be zero
# before the first call (each call leaves them zero).
_ZEROED = {"index_topk_fused_decode"}


def _workspace(p: Problem, op: str, ws, device):
    need = msa_workspace_bytes(p, op)
    if ws is None:
        alloc = torch.zeros if op in _ZEROED else torch.empty
        ws = alloc(max(need, 16), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def decode_workspace(p: Problem, dense: bool = False, device="cuda", op=None):
    """A reusable workspace for msa_sparse_attn_decode (dense=False),
    msa_dense_attn_decode (dense=True) or another op named by `op`, zero-filled
    (the decode form of msa_index_topk_fused needs its counter region zero)."""
    if op is None:
        op = "dense_attn_decode" if dense else "sparse_attn_decode"
    return torch.zeros(max(msa_workspace_bytes(p, op), 16), dtype=torch.uint8, device=device)


def msa_sparse_attn_prefill_status_offset(p: Problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().msa_sparse_attn_prefill_status_offset(ctypes.byref(p.c()), ctypes.byref(out)))
    return out.value


def msa_set_wait_limit(polls: int) -> None:
    lib().msa_set_wait_limit(int(polls))


def msa_index_block_scores(p: Problem, iq, ik, seq_lens=None, block_scores=None, stream=None):
    if block_scores is None:
        block_scores = torch.empty((p.batch, p.n_kv_heads, p.seq_q, p.nblk), dtype=torch.float32,
                                   device=iq.device)
    _check(lib().msa_index_block_scores(ctypes.byref(p.c()), _ptr(iq, torch.bfloat16),
                                        _ptr(ik, torch.bfloat16), _ptr(seq_lens, torch.int32),
                                        _ptr(block_scores, torch.float32), _stream(stream)))
    return block_scores


def msa_topk_blocks(p: Problem, block_scores, seq_lens=None, sel=None, stream=None):
    if sel is None:
        sel = torch.empty((p.batch, p.n_kv_heads, p.seq_q, p.top_k), dtype=torch.int32,
                          device=block_scores.device)
    _check(lib().msa_topk_blocks(ctypes.byref(p.c()), _ptr(block_scores, torch.float32),
                                 _ptr(seq_lens, torch.int32), _ptr(sel, torch.int32),
                                 _stream(stream)))
    return sel


def msa_index_topk_fused(p: Problem, iq, ik, seq_lens=None, sel=None, workspace=None,
                         stream=None):
    if sel is None:
        sel = torch.empty((p.batch, p.n_kv_heads, p.seq_q, p.top_k), dtype=torch.int32,
                          device=iq.device)
    op = "index_topk_fused" if seq_lens is None else "index_topk_fused_decode"
    ws, nbytes = _workspace(p, op, workspace, iq.device)
    _check(lib().msa_index_topk_fused(ctypes.byref(p.c()), _ptr(iq, torch.bfloat16),
                                      _ptr(ik, torch.bfloat16), _ptr(seq_lens, torch.int32),
                                      _ptr(sel, torch.int32), _ptr(ws), nbytes, _stream(stream)))
    return sel


def msa_sparse_attn_prefill(p: Problem, q, k, v, sel, out=None, lse=None, workspace=None,
                            stream=None):
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(p, "sparse_attn_prefill", workspace, q.device)
    _check(lib().msa_sparse_attn_prefill(ctypes.byref(p.c()), _ptr(q, torch.bfloat16),
                                         _ptr(k, torch.bfloat16), _ptr(v, torch.bfloat16),
                                         _ptr(sel, torch.int32), _ptr(out, torch.bfloat16),
                                         _ptr(lse, torch.float32), _ptr(ws), nbytes,
                                         _stream(stream)))
    return out


def msa_sparse_attn_prefill_backward(p: Problem, q, k, v, sel, out, lse, dout, dq=None, dk=None,
                                     dv=None, workspace=None, stream=None):
    """Gradients (dq [B][Sq][Hq][128], dk, dv [B][Hkv][Skv][128], fp32) of
    sum(dout * out) for msa_sparse_attn_prefill's out and lse on these inputs."""
    f32 = dict(dtype=torch.float32, device=q.device)
    if dq is None:
        dq = torch.empty(q.shape, **f32)
    if dk is None:
        dk = torch.empty(k.shape, **f32)
    if dv is None:
        dv = torch.empty(v.shape, **f32)
    ws, nbytes = _workspace(p, "sparse_attn_prefill_backward", workspace, q.device)
    _check(lib().msa_sparse_attn_prefill_backward(
        ctypes.byref(p.c()), _ptr(q, torch.bfloat16), _ptr(k, torch.bfloat16),
        _ptr(v, torch.bfloat16), _ptr(sel, torch.int32), _ptr(out, torch.bfloat16),
        _ptr(lse, torch.float32), _ptr(dout, torch.bfloat16), _ptr(dq, torch.float32),
        _ptr(dk, torch.float32), _ptr(dv, torch.float32), _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv


def msa_index_kl_backward(p: Problem, q, k, iq, ik, sel, lse, loss=None, diq=None, dik=None,
                          workspace=None, stream=None):
    """The index branch's KL loss (loss [B][Sq][4]) and its gradients (diq
    [B][Sq][4][64], dik [B][Skv][64]), fp32, over the selection sel, with the
    main branch's weights taken from msa_sparse_attn_prefill's lse."""
    f32 = dict(dtype=torch.float32, device=q.device)
    if loss is None:
        loss = torch.empty(iq.shape[:3], **f32)
    if diq is None:
        diq = torch.empty(iq.shape, **f32)
    if dik is None:
        dik = torch.empty(ik.shape, **f32)
    ws, nbytes = _workspace(p, "index_kl_backward", workspace, q.device)
    _check(lib().msa_index_kl_backward(
        ctypes.byref(p.c()), _ptr(q, torch.bfloat16), _ptr(k, torch.bfloat16),
        _ptr(iq, torch.bfloat16), _ptr(ik, torch.bfloat16), _ptr(sel, torch.int32),
        _ptr(lse, torch.float32), _ptr(loss, torch.float32), _ptr(diq, torch.float32),
        _ptr(dik, torch.float32), _ptr(ws), nbytes, _stream(stream)))
    return loss, diq, dik


def msa_sparse_attn_decode(p: Problem, q, k_cache, v_cache, seq_lens, sel, out=None, lse=None,
                           workspace=None, stream=None):
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(p, "sparse_attn_decode", workspace, q.device)
    _check(lib().msa_sparse_attn_decode(ctypes.byref(p.c()), _ptr(q, torch.bfloat16),
                                        _ptr(k_cache, torch.bfloat16),
                                        _ptr(v_cache, torch.bfloat16), _ptr(seq_lens, torch.int32),
                                        _ptr(sel, torch.int32), _ptr(out, torch.bfloat16),
                                        _ptr(lse, torch.float32), _ptr(ws), nbytes,
                                        _stream(stream)))
    return out


def msa_sparse_attn_decode_static(p: Problem, q, k_cache, v_cache, seq_lens, sel, out=None,
                                  lse=None, stream=None):
    """msa_sparse_attn_decode with the library's own scratch (no workspace)."""
    if out is None:
        out = torch.empty_like(q)
    _check(lib().msa_sparse_attn_decode_static(
        ctypes.byref(p.c()), _ptr(q, torch.bfloat16), _ptr(k_cache, torch.bfloat16),
        _ptr(v_cache, torch.bfloat16), _ptr(seq_lens, torch.int32), _ptr(sel, torch.int32),
        _ptr(out, torch.bfloat16), _ptr(lse, torch.float32), _stream(stream)))
    return out


def msa_index_block_scores_paged(p: Problem, iq, ik_pages, page_table, num_pages: int, seq_lens,
                                 block_scores=None, stream=None):
    """Decode block scores with the index-K cache in pages [num_pages][64][64]."""
    if block_scores is None:
        block_scores = torch.empty((p.batch, p.n_kv_heads, 1, p.nblk), dtype=torch.float32,
                                   device=iq.device)
    _check(lib().msa_index_block_scores_paged(
        ctypes.byref(p.c()), _ptr(iq, torch.bfloat16), _ptr(ik_pages, torch.bfloat16),
        _ptr(page_table, torch.int32), int(num_pages), _ptr(seq_lens, torch.int32),
        _ptr(block_scores, torch.float32), _stream(stream)))
    return block_scores


def msa_index_topk_fused_paged(p: Problem, iq, ik_pages, page_table, num_pages: int, seq_lens,
                               sel=None, workspace=None, stream=None):
    """Decode index scoring + top-k in one launch, index-K cache in pages."""
    if sel is None:
        sel = torch.empty((p.batch, p.n_kv_heads, 1, p.top_k), dtype=torch.int32, device=iq.device)
    ws, nbytes = _workspace(p, "index_topk_fused_decode", workspace, iq.device)
    _check(lib().msa_index_topk_fused_paged(
        ctypes.byref(p.c()), _ptr(iq, torch.bfloat16), _ptr(ik_pages, torch.bfloat16),
        _ptr(page_table, torch.int32), int(num_pages), _ptr(seq_lens, torch.int32),
        _ptr(sel, torch.int32), _ptr(ws), nbytes, _stream(stream)))
    return sel


def msa_sparse_attn_decode_paged(p: Problem, q, k_pages, v_pages, page_table, num_pages: int,
                                 seq_lens, sel, out=None, lse=None, workspace=None, stream=None):
    """Sparse decode with K and V in pages [num_pages][Hkv][64][128]."""
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(p, "sparse_attn_decode", workspace, q.device)
    _check(lib().msa_sparse_attn_decode_paged(
        ctypes.byref(p.c()), _ptr(q, torch.bfloat16), _ptr(k_pages, torch.bfloat16),
        _ptr(v_pages, torch.bfloat16), _ptr(page_table, torch.int32), int(num_pages),
        _ptr(seq_lens, torch.int32), _ptr(sel, torch.int32), _ptr(out, torch.bfloat16),
        _ptr(lse, torch.float32), _ptr(ws), nbytes, _stream(stream)))
    return out


def msa_dense_attn_prefill(p: Problem, q, k, v, out=None, lse=None, workspace=None, stream=None):
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(p, "dense_attn_prefill", workspace, q.device)
    _check(lib().msa_dense_attn_prefill(ctypes.byref(p.c()), _ptr(q, torch.bfloat16),
                                        _ptr(k, torch.bfloat16), _ptr(v, torch.bfloat16),
                                        _ptr(out, torch.bfloat16), _ptr(lse, torch.float32),
                                        _ptr(ws), nbytes, _stream(stream)))
    return out


def msa_dense_attn_decode(p: Problem, q, k_cache, v_cache, seq_lens, out=None, lse=None,
                          workspace=None, stream=None):
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(p, "dense_attn_decode", workspace, q.device)
    _check(lib().msa_dense_attn_decode(ctypes.byref(p.c()), _ptr(q, torch.bfloat16),
                                       _ptr(k_cache, torch.bfloat16),
                                       _ptr(v_cache, torch.bfloat16), _ptr(seq_lens, torch.int32),
                                       _ptr(out, torch.bfloat16), _ptr(lse, torch.float32),
                                       _ptr(ws), nbytes, _stream(stream)))
    return out
