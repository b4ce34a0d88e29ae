"""Seeded synthetic inputs, shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method itself: it only draws tensors.
Both the HIP path and the CPU oracle consume the exact bytes drawn here (the
oracle receives them as uint16 bit patterns after a device-to-host copy).

Recipe: every tensor is drawn in fp32 from one seeded torch.Generator on the
target device, in the order Q, K, V, iQ, iK, and rounded to bf16
(round-to-nearest-even).  With a block offset (std > 0), one vector per
(sequence, head, 64-token block) is drawn right before the tensor it offsets
(keys K and index keys iK) and added in fp32 before the rounding.  Large
tensors are drawn in fixed-size chunks so that generation needs little scratch
memory; the result depends only on the seed, the device type and the shapes.
Integer mode draws every entry uniformly from {-2, ..., 2} instead, so that
every index score is an integer that fp32 represents exactly.  With
iq_shared_rows = r > 1 (diagnostic workloads), iQ is drawn for ceil(Sq / r)
rows and each draw is repeated for r consecutive rows.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from .configs import Workload

_CHUNK = 1 << 26  # elements per randn call


@dataclass
class Inputs:
    q: torch.Tensor         # [B, Sq, Hq, D] bf16
    k: torch.Tensor         # [B, Hkv, Skv, D] bf16
    v: torch.Tensor         # [B, Hkv, Skv, D] bf16
    iq: torch.Tensor        # [B, Sq, Hi, Di] bf16
    ik: torch.Tensor        # [B, Skv, Di] bf16
    seq_lens: Optional[torch.Tensor]  # [B] int32 (decode), else None


def _draw(n: int, gen: torch.Generator, device, integer: bool) -> torch.Tensor:
    if integer:
        return torch.randint(-2, 3, (n,), generator=gen, device=device).to(torch.float32)
    return torch.randn(n, generator=gen, device=device, dtype=torch.float32)


def _fill(dst: torch.Tensor, gen, integer: bool) -> None:
    flat = dst.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        flat[s:e] = _draw(e - s, gen, dst.device, integer).to(torch.bfloat16)


def _fill_with_block_offset(dst: torch.Tensor, gen, std: float, block: int) -> None:
    """dst is [..., S, D]: one N(0, std^2) vector per 64-token block of every
    leading slice, added in fp32 to N(0, 1) draws before rounding."""
    S, D = dst.shape[-2], dst.shape[-1]
    nblk = (S + block - 1) // block
    slabs = dst.reshape(-1, S, D)
    tok_block = torch.arange(S, device=dst.device) // block
    for i in range(slabs.shape[0]):
        off = _draw(nblk * D, gen, dst.device, False).view(nblk, D) * std
        base = _draw(S * D, gen, dst.device, False).view(S, D)
        slabs[i].copy_((base + off[tok_block]).to(torch.bfloat16))


def generate(w: Workload, device, *, seed: Optional[int] = None, integer: bool = False,
             seq_lens: Optional[list] = None) -> Inputs:
    """Draw the inputs of workload `w` on `device`.

    seq_lens (decode only): per-sequence cache lengths; default all = seq_kv.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    B, Sq, Skv = w.batch, w.seq_q, w.seq_kv
    bf = dict(dtype=torch.bfloat16, device=device)
    q = torch.empty((B, Sq, w.n_q_heads, w.head_dim), **bf)
    k = torch.empty((B, w.n_kv_heads, Skv, w.head_dim), **bf)
    v = torch.empty_like(k)
    iq = torch.empty((B, Sq, w.n_idx_heads, w.idx_head_dim), **bf)
    ik = torch.empty((B, Skv, w.idx_head_dim), **bf)
    offset = w.block_offset_std > 0 and not integer
    _fill(q, gen, integer)
    if offset:
        _fill_with_block_offset(k, gen, w.block_offset_std, w.block_size)
    else:
        _fill(k, gen, integer)
    _fill(v, gen, integer)
    r = w.iq_shared_rows
    if r > 1:
        runs = torch.empty((B, (Sq + r - 1) // r, w.n_idx_heads, w.idx_head_dim), **bf)
        _fill(runs, gen, integer)
        iq.copy_(runs.repeat_interleave(r, dim=1)[:, :Sq])
        del runs
    else:
        _fill(iq, gen, integer)
    if offset:
        _fill_with_block_offset(ik, gen, w.block_offset_std, w.block_size)
    else:
        _fill(ik, gen, integer)
    lens = None
    if w.decode:
        if seq_lens is None:
            seq_lens = [Skv] * B
        assert len(seq_lens) == B and all(1 <= L <= Skv for L in seq_lens)
        lens = torch.tensor(seq_lens, dtype=torch.int32, device=device)
    return Inputs(q, k, v, iq, ik, lens)


def cotangent(like: torch.Tensor, seed: int) -> torch.Tensor:
    """Seeded N(0, 1) bf16 tensor shaped like `like` (the output gradient fed
    to the main branch's backward), drawn on like's device."""
    gen = torch.Generator(device=like.device)
    gen.manual_seed(seed)
    out = torch.empty(like.shape, dtype=torch.bfloat16, device=like.device)
    _fill(out, gen, False)
    return out


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bytes (for the oracle)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
