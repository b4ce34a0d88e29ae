"""Full-path GPU-vs-oracle check of one workload at its real size, in the launch
configuration bench.py times (used by the GPU workload tests)."""
from __future__ import annotations

import time

import numpy as np
import torch

import block_sparse_gqa_02_amd as msa
from block_sparse_gqa_02_amd.inputs import bf16_bits, generate
import oracle.oracle as O
import parity as PAR


def oprob(w):
    return O.Problem(w.batch, w.seq_q, w.seq_kv, w.q_start, w.n_q_heads, w.n_kv_heads,
                     w.head_dim, w.n_idx_heads, w.idx_head_dim, w.block_size, w.top_k, w.decode,
                     w.softmax_scale)


def gpu_forward(w, inp, fused: bool):
    """The hot path as the library runs it; returns (sel, out, lse)."""
    p = msa.Problem.from_workload(w)
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_q), dtype=torch.float32, device="cuda")
    if fused:
        sel = msa.msa_index_topk_fused(p, inp.iq, inp.ik)
    else:
        bs = msa.msa_index_block_scores(p, inp.iq, inp.ik, inp.seq_lens)
        sel = msa.msa_topk_blocks(p, bs, inp.seq_lens)
        del bs
    if w.decode:
        out = msa.msa_sparse_attn_decode(p, inp.q, inp.k, inp.v, inp.seq_lens, sel, lse=lse)
    else:
        out = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse)
    torch.cuda.synchronize()
    return sel, out, lse


def check(w, fused: bool, rows=None, seed=None, log=print):
    """Runs the workload on the GPU and checks `rows` (row ids b*Sq+t; None =
    all) against the oracle.  Returns a dict of statistics."""
    t0 = time.time()
    inp = generate(w, "cuda", seed=seed)
    sel, out, lse = gpu_forward(w, inp, fused)
    if rows is None:
        rows = np.arange(w.batch * w.seq_q)
    rows = np.asarray(rows, dtype=np.int64)
    h = {n: bf16_bits(getattr(inp, n)) for n in ("q", "k", "v", "iq", "ik")}
    lens = None if inp.seq_lens is None else inp.seq_lens.cpu().numpy()
    rb, rt = rows // w.seq_q, rows % w.seq_q
    ib, it = torch.as_tensor(rb, device="cuda"), torch.as_tensor(rt, device="cuda")
    sel_h = sel[ib, :, it].cpu().numpy()                  # [n][Hkv][k]
    out_h = out[ib, it].float().cpu().numpy()             # [n][Hq][D]
    lse_h = lse[ib, :, it].cpu().numpy()                  # [n][Hq]
    del out, lse
    log(f"[{w.name}] gpu done, {len(rows)} rows to check ({time.time() - t0:.1f}s)")
    p = oprob(w)
    o_sel, o_out, o_lse, o_sc = O.forward_rows_parallel(p, h["q"], h["k"], h["v"], h["iq"],
                                                        h["ik"], lens, rows, PAR.host_threads(),
                                                        want_scores=True)
    log(f"[{w.name}] oracle done ({time.time() - t0:.1f}s)")
    ties = 0
    ref_out, ref_lse = o_out.copy(), o_lse.copy()
    for i, r in enumerate(rows):
        b, t = int(rb[i]), int(rt[i])
        pos = int(lens[b]) - 1 if w.decode else w.q_start + t
        cur = pos // w.block_size
        tie_row = False
        for hh in range(w.n_kv_heads):
            tie_row |= PAR.check_selection_row(sel_h[i, hh], o_sc[i, hh], cur, w.top_k, False,
                                               f"{w.name} row {r} head {hh}")
        if tie_row:  # attention is compared on the GPU's own selection
            ties += 1
            ref_out[i], ref_lse[i] = O.attend_row(p, h["q"], h["k"], h["v"], lens, sel_h[i], b, t)
    mx, mean = PAR.assert_attention_close(out_h, ref_out, w.name)
    lse_err = float(np.max(np.abs(lse_h - ref_lse)))
    assert lse_err < 1e-2, f"{w.name}: lse error {lse_err}"
    stats = dict(workload=w.name, fused=fused, rows=len(rows), tie_rows=ties, max_abs=mx,
                 mean_abs=mean, lse_max_abs=lse_err, seconds=time.time() - t0)
    log(f"[{w.name}] {stats}")
    return stats
