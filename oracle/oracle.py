"""ctypes wrapper over the CPU oracle (msa_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never imports it.  It shares
no code with the HIP library.  Inputs are numpy arrays: bf16 tensors are passed
as their raw uint16 bit patterns (the exact bytes the GPU consumed).

The oracle itself is single-threaded; `forward_rows_parallel` only runs
independent row shards of it on several host threads (ctypes releases the GIL
while a C call runs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
           _SRC, "-o", _LIB, "-lm"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11, IEEE double, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq_q", "seq_kv", "q_start", "n_q_heads", "n_kv_heads", "head_dim",
        "n_idx_heads", "idx_head_dim", "block_size", "top_k", "decode")] + [
        ("softmax_scale", ctypes.c_double)]


@dataclass
class Problem:
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
    decode: bool
    softmax_scale: float

    def c(self) -> _Problem:
        return _Problem(self.batch, self.seq_q, self.seq_kv, self.q_start, self.n_q_heads,
                        self.n_kv_heads, self.head_dim, self.n_idx_heads, self.idx_head_dim,
                        self.block_size, self.top_k, int(bool(self.decode)),
                        float(self.softmax_scale))

    @property
    def nblk(self) -> int:
        return (self.seq_kv + self.block_size - 1) // self.block_size


_lib = None


def lib(path: str | None = None):
    global _lib
    if path is not None:  # an explicitly named build (used by the mutation pins)
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(L):
    P = ctypes.POINTER
    u16, i32, i64, f32, f64 = (P(ctypes.c_uint16), P(ctypes.c_int32), P(ctypes.c_int64),
                               P(ctypes.c_float), P(ctypes.c_double))
    prob = P(_Problem)
    L.oracle_num_blocks.argtypes = [prob]
    L.oracle_num_blocks.restype = ctypes.c_int32
    L.oracle_position.argtypes = [prob, i32, ctypes.c_int32, ctypes.c_int32]
    L.oracle_position.restype = ctypes.c_int32
    L.oracle_block_scores_row.argtypes = [prob, u16, u16, i32, ctypes.c_int32, ctypes.c_int32, f32]
    L.oracle_select_row.argtypes = [prob, f32, ctypes.c_int32, i32]
    L.oracle_attend_row.argtypes = [prob, u16, u16, u16, i32, i32, ctypes.c_int32,
                                    ctypes.c_int32, f64, f64]
    L.oracle_dense_row.argtypes = [prob, u16, u16, u16, i32, ctypes.c_int32, ctypes.c_int32,
                                   f64, f64]
    L.oracle_forward_rows.argtypes = [prob, u16, u16, u16, u16, u16, i32, ctypes.c_int64, i64,
                                      i32, f64, f64, f32]
    L.oracle_attend_row_f64.argtypes = [prob, f64, f64, f64, i32, i32, ctypes.c_int32,
                                        ctypes.c_int32, f64, f64]
    L.oracle_attend_backward.argtypes = [prob, f64, f64, f64, f64, i32, i32, f64, f64, f64]
    L.oracle_index_kl.argtypes = [prob, f64, f64, f64, f64, i32, i32, f64, f64, f64]
    for name in ("oracle_block_scores_row", "oracle_select_row", "oracle_attend_row",
                 "oracle_dense_row", "oracle_forward_rows", "oracle_attend_row_f64", "oracle_index_kl",
                 "oracle_attend_backward"):
        getattr(L, name).restype = ctypes.c_int
    return L


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.POINTER(ctype)()
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 tensors are passed as uint16 bit patterns"
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def position(p: Problem, seq_lens, b: int, t: int, L=None) -> int:
    L = L or lib()
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    return int(L.oracle_position(ctypes.byref(p.c()), _ptr(sl, ctypes.c_int32), b, t))


def block_scores_row(p: Problem, iq, ik, seq_lens, b: int, t: int, L=None) -> np.ndarray:
    L = L or lib()
    out = np.empty((p.n_kv_heads, p.nblk), dtype=np.float32)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    iq, ik = _u16(iq), _u16(ik)
    _check(L.oracle_block_scores_row(ctypes.byref(p.c()), _ptr(iq, ctypes.c_uint16),
                                     _ptr(ik, ctypes.c_uint16), _ptr(sl, ctypes.c_int32), b, t,
                                     _ptr(out, ctypes.c_float)), "block_scores_row")
    return out


def select_row(p: Problem, scores, cur: int, L=None) -> np.ndarray:
    L = L or lib()
    s = np.ascontiguousarray(scores, dtype=np.float32)
    assert s.shape[0] >= cur + 1
    sel = np.empty((p.top_k,), dtype=np.int32)
    _check(L.oracle_select_row(ctypes.byref(p.c()), _ptr(s, ctypes.c_float), cur,
                               _ptr(sel, ctypes.c_int32)), "select_row")
    return sel


def attend_row(p: Problem, q, k, v, seq_lens, sel, b: int, t: int, L=None):
    L = L or lib()
    q, k, v = _u16(q), _u16(k), _u16(v)
    s = np.ascontiguousarray(sel, dtype=np.int32).reshape(p.n_kv_heads, p.top_k)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((p.n_q_heads, p.head_dim), dtype=np.float64)
    lse = np.empty((p.n_q_heads,), dtype=np.float64)
    _check(L.oracle_attend_row(ctypes.byref(p.c()), _ptr(q, ctypes.c_uint16),
                               _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                               _ptr(sl, ctypes.c_int32), _ptr(s, ctypes.c_int32), b, t,
                               _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double)),
           "attend_row")
    return out, lse


def dense_row(p: Problem, q, k, v, seq_lens, b: int, t: int, L=None):
    L = L or lib()
    q, k, v = _u16(q), _u16(k), _u16(v)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((p.n_q_heads, p.head_dim), dtype=np.float64)
    lse = np.empty((p.n_q_heads,), dtype=np.float64)
    _check(L.oracle_dense_row(ctypes.byref(p.c()), _ptr(q, ctypes.c_uint16),
                              _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                              _ptr(sl, ctypes.c_int32), b, t, _ptr(out, ctypes.c_double),
                              _ptr(lse, ctypes.c_double)), "dense_row")
    return out, lse


def forward_rows(p: Problem, q, k, v, iq, ik, seq_lens, rows, want_scores=False, L=None):
    """Block scores -> selection -> attention for the given row ids (b*seq_q+t).

    Returns (sel [n][Hkv][k] int32, out [n][Hq][D] f64, lse [n][Hq] f64,
    scores [n][Hkv][nblk] f32 or None)."""
    L = L or lib()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    q, k, v, iq, ik = (_u16(x) for x in (q, k, v, iq, ik))
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    sel = np.empty((n, p.n_kv_heads, p.top_k), dtype=np.int32)
    out = np.empty((n, p.n_q_heads, p.head_dim), dtype=np.float64)
    lse = np.empty((n, p.n_q_heads), dtype=np.float64)
    scores = np.empty((n, p.n_kv_heads, p.nblk), dtype=np.float32) if want_scores else None
    _check(L.oracle_forward_rows(ctypes.byref(p.c()), _ptr(q, ctypes.c_uint16),
                                 _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                                 _ptr(iq, ctypes.c_uint16), _ptr(ik, ctypes.c_uint16),
                                 _ptr(sl, ctypes.c_int32), n, _ptr(rows, ctypes.c_int64),
                                 _ptr(sel, ctypes.c_int32), _ptr(out, ctypes.c_double),
                                 _ptr(lse, ctypes.c_double), _ptr(scores, ctypes.c_float)),
           "forward_rows")
    return sel, out, lse, scores


def forward_rows_parallel(p: Problem, q, k, v, iq, ik, seq_lens, rows, threads: int,
                          want_scores=False):
    """forward_rows over `threads` independent, interleaved row shards."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    threads = max(1, min(threads, len(rows)))
    shards = [rows[i::threads] for i in range(threads)]
    L = lib()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda r: forward_rows(p, q, k, v, iq, ik, seq_lens, r,
                                                   want_scores, L), shards))
    n = len(rows)
    sel = np.empty((n, p.n_kv_heads, p.top_k), dtype=np.int32)
    out = np.empty((n, p.n_q_heads, p.head_dim), dtype=np.float64)
    lse = np.empty((n, p.n_q_heads), dtype=np.float64)
    scores = np.empty((n, p.n_kv_heads, p.nblk), dtype=np.float32) if want_scores else None
    for i, (s, o, l, sc) in enumerate(parts):
        sel[i::threads], out[i::threads], lse[i::threads] = s, o, l
        if want_scores:
            scores[i::threads] = sc
    return sel, out, lse, scores


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def attend_row_f64(p: Problem, q, k, v, seq_lens, sel, b: int, t: int, L=None):
    """oracle_attend_row on fp64 inputs (q [B][Sq][Hq][D], k, v [B][Hkv][Skv][D])."""
    L = L or lib()
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = np.ascontiguousarray(sel, dtype=np.int32).reshape(p.n_kv_heads, p.top_k)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((p.n_q_heads, p.head_dim), dtype=np.float64)
    lse = np.empty((p.n_q_heads,), dtype=np.float64)
    _check(L.oracle_attend_row_f64(ctypes.byref(p.c()), _ptr(q, ctypes.c_double),
                                   _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                                   _ptr(sl, ctypes.c_int32), _ptr(s, ctypes.c_int32), b, t,
                                   _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double)),
           "attend_row_f64")
    return out, lse


def attend_backward(p: Problem, q, k, v, dout, seq_lens, sel_all, L=None):
    """Gradients (dq [B][Sq][Hq][D], dk, dv [B][Hkv][Skv][D], fp64) of
    sum(dout * out) for the sparse attention of every row over the selection
    sel_all [B][Sq][Hkv][top_k]; inputs are fp64 arrays (or anything numpy
    converts: pass bf16 values as exact doubles)."""
    L = L or lib()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    s = np.ascontiguousarray(sel_all, dtype=np.int32)
    assert s.shape == (p.batch, p.seq_q, p.n_kv_heads, p.top_k)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    dq = np.empty((p.batch, p.seq_q, p.n_q_heads, p.head_dim), dtype=np.float64)
    dk = np.empty((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim), dtype=np.float64)
    dv = np.empty_like(dk)
    _check(L.oracle_attend_backward(ctypes.byref(p.c()), _ptr(q, ctypes.c_double),
                                    _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                                    _ptr(g, ctypes.c_double), _ptr(sl, ctypes.c_int32),
                                    _ptr(s, ctypes.c_int32), _ptr(dq, ctypes.c_double),
                                    _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double)),
           "attend_backward")
    return dq, dk, dv


def index_kl(p: Problem, q, k, iq, ik, seq_lens, sel_all, L=None):
    """The index branch's KL training signal (oracle_index_kl): loss
    [B][Sq][Hi], diq [B][Sq][Hi][Di], dik [B][Skv][Di], all fp64, over the
    selection sel_all [B][Sq][Hkv][top_k]; inputs fp64 (bf16 values as exact
    doubles)."""
    L = L or lib()
    q, k, iq, ik = _f64(q), _f64(k), _f64(iq), _f64(ik)
    s = np.ascontiguousarray(sel_all, dtype=np.int32)
    assert s.shape == (p.batch, p.seq_q, p.n_kv_heads, p.top_k)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    loss = np.empty((p.batch, p.seq_q, p.n_idx_heads), dtype=np.float64)
    diq = np.empty((p.batch, p.seq_q, p.n_idx_heads, p.idx_head_dim), dtype=np.float64)
    dik = np.empty((p.batch, p.seq_kv, p.idx_head_dim), dtype=np.float64)
    _check(L.oracle_index_kl(ctypes.byref(p.c()), _ptr(q, ctypes.c_double),
                             _ptr(k, ctypes.c_double), _ptr(iq, ctypes.c_double),
                             _ptr(ik, ctypes.c_double), _ptr(sl, ctypes.c_int32),
                             _ptr(s, ctypes.c_int32), _ptr(loss, ctypes.c_double),
                             _ptr(diq, ctypes.c_double), _ptr(dik, ctypes.c_double)),
           "index_kl")
    return loss, diq, dik
