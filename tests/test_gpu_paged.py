"""Paged decode caches (one page per 64-token block, random page table): the
paged entry points must give the contiguous path's results bit for bit, and
page ids outside the pool must be skipped (never read)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import block_sparse_gqa_02_amd as msa
from block_sparse_gqa_02_amd.configs import DECODE_32x256K
from block_sparse_gqa_02_amd.inputs import bf16_bits, generate
import oracle.oracle as O
import parity as PAR

pytestmark = pytest.mark.gpu
DEV = "cuda"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_pages(w, inp, seed, extra=5):
    """Scatters the contiguous caches into page pools under a random table;
    unused pages hold a constant no cache page holds."""
    B, Hkv, nblk = w.batch, w.n_kv_heads, w.nblk
    pad = nblk * 64 - w.seq_kv
    k = F.pad(inp.k, (0, 0, 0, pad))
    v = F.pad(inp.v, (0, 0, 0, pad))
    ik = F.pad(inp.ik, (0, 0, 0, pad))
    npages = B * nblk + extra
    g = torch.Generator().manual_seed(seed)
    ids = torch.randperm(npages, generator=g)[: B * nblk].to(DEV)
    kp = torch.full((npages, Hkv, 64, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    vp = torch.full_like(kp, -3.0)
    ikp = torch.full((npages, 64, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    kp[ids] = k.view(B, Hkv, nblk, 64, 128).permute(0, 2, 1, 3, 4).reshape(B * nblk, Hkv, 64, 128)
    vp[ids] = v.view(B, Hkv, nblk, 64, 128).permute(0, 2, 1, 3, 4).reshape(B * nblk, Hkv, 64, 128)
    ikp[ids] = ik.view(B, nblk, 64, 64).reshape(B * nblk, 64, 64)
    table = ids.view(B, nblk).to(torch.int32).contiguous()
    return kp, vp, ikp, table, npages


W = DECODE_32x256K.shrink(batch=4, seq_kv=3000, top_k=11)
LENS = [3000, 65, 1, 2048]


def contiguous(p, inp, sel=None):
    bs = msa.msa_index_block_scores(p, inp.iq, inp.ik, inp.seq_lens)
    if sel is None:
        sel = msa.msa_topk_blocks(p, bs, inp.seq_lens)
    lse = torch.empty((W.batch, W.n_q_heads, 1), dtype=torch.float32, device=DEV)
    out = msa.msa_sparse_attn_decode(p, inp.q, inp.k, inp.v, inp.seq_lens, sel, lse=lse)
    return bs, sel, out, lse


def test_paged_decode_equals_contiguous_and_oracle():
    need_gpu()
    inp = generate(W, DEV, seed=41, seq_lens=LENS)
    p = msa.Problem.from_workload(W)
    kp, vp, ikp, table, npages = to_pages(W, inp, seed=3)
    bs, sel, out, lse = contiguous(p, inp)
    bs_p = msa.msa_index_block_scores_paged(p, inp.iq, ikp, table, npages, inp.seq_lens)
    sel_p = msa.msa_topk_blocks(p, bs_p, inp.seq_lens)
    lse_p = torch.empty_like(lse)
    out_p = msa.msa_sparse_attn_decode_paged(p, inp.q, kp, vp, table, npages, inp.seq_lens,
                                             sel_p, lse=lse_p)
    torch.cuda.synchronize()
    for b, L in enumerate(LENS):
        cur = (L - 1) // 64
        assert torch.equal(bs_p[b, :, 0, : cur + 1], bs[b, :, 0, : cur + 1]), b
    assert torch.equal(sel_p, sel)
    assert torch.equal(out_p, out)
    assert torch.equal(lse_p, lse)
    # and against the oracle on the contiguous caches
    po = O.Problem(W.batch, W.seq_q, W.seq_kv, W.q_start, W.n_q_heads, W.n_kv_heads, W.head_dim,
                   W.n_idx_heads, W.idx_head_dim, W.block_size, W.top_k, W.decode, W.softmax_scale)
    h = {n: bf16_bits(getattr(inp, n)) for n in ("q", "k", "v")}
    lens = inp.seq_lens.cpu().numpy()
    sel_h, out_h = sel_p.cpu().numpy(), out_p.float().cpu().numpy()
    for b in range(W.batch):
        o, _ = O.attend_row(po, h["q"], h["k"], h["v"], lens, sel_h[b, :, 0], b, 0)
        PAR.assert_attention_close(out_h[b, 0], o, f"paged seq {b}")


def test_paged_out_of_pool_ids_are_skipped():
    need_gpu()
    inp = generate(W, DEV, seed=42, seq_lens=LENS)
    p = msa.Problem.from_workload(W)
    kp, vp, ikp, table, npages = to_pages(W, inp, seed=4)
    bs, sel, _, _ = contiguous(p, inp)
    sel_h = sel.cpu().numpy()
    bad = table.clone()
    sel_mod = sel.clone()
    hits = []
    for b, L in enumerate(LENS):
        cur = (L - 1) // 64
        # the first selected block of KV head 0 that is not the own block
        c = next((int(x) for x in sel_h[b, 0, 0] if 0 <= x < cur), None)
        if c is None:
            continue
        bad[b, c] = -1 if b % 2 == 0 else npages + 3
        hits.append((b, c))
        for hh in range(W.n_kv_heads):  # the page holds every KV head of the block
            row = sel_mod[b, hh, 0]
            row[row == c] = -1
    assert hits
    bs_p = msa.msa_index_block_scores_paged(p, inp.iq, ikp, bad, npages, inp.seq_lens)
    out_p = msa.msa_sparse_attn_decode_paged(p, inp.q, kp, vp, bad, npages, inp.seq_lens, sel)
    _, _, out_ref, _ = contiguous(p, inp, sel=sel_mod)
    torch.cuda.synchronize()
    for b, c in hits:
        assert torch.all(bs_p[b, :, 0, c] == -np.inf), (b, c)
        cur = (LENS[b] - 1) // 64
        keep = torch.ones(cur + 1, dtype=torch.bool, device=DEV)
        keep[c] = False
        assert torch.equal(bs_p[b, :, 0, : cur + 1][:, keep], bs[b, :, 0, : cur + 1][:, keep])
    assert torch.equal(out_p, out_ref)
