"""Main-branch gradient (msa_sparse_attn_prefill_backward) against the CPU
oracle's gradient (oracle_attend_backward) on the GPU's own selection and the
same bf16 inputs, every element compared.  Sizes span several 64-row batches
and 64-key blocks with ragged tails, rows that precede k blocks (short, padded
lists), a chunk whose rows start past 0 with a cache longer than the rows
(blocks no row reads: their dk, dv must be exactly zero), query groups of
2, 4, 8 and 16 heads (4 and 8 take the ring dq kernel, the others the
per-row one), and row lists of hundreds of 64-column chunks.

Tolerance, per tensor, from the arithmetic: the kernels round P and dS to
bf16 (as the forward rounds P) and take Dsum from the bf16 forward output, so
each term carries a few bf16 roundings (unit roundoff 2^-9) while sums stay in
fp32.  Errors are measured against the reference's scale: max |gpu - ref| <=
2e-2 * max |ref| and mean |gpu - ref| <= 4e-3 * mean |ref|."""
import numpy as np
import pytest
import torch

import block_sparse_gqa_02_amd as msa
from block_sparse_gqa_02_amd.configs import PREFILL_32K, TINY_PREFILL_2K
from block_sparse_gqa_02_amd.inputs import cotangent, generate
import oracle.oracle as O

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
MEAN_REL = 4e-3

CASES = {
    # G = 4, k = 8, 1000 rows (ragged last batch and block), rows < 448 hold short lists
    "g4_ragged": TINY_PREFILL_2K.shrink(name="bwd_g4", seq_q=1000, seq_kv=1000),
    # G = 8, two sequences, rows 650..1349 of a 1500-token cache (blocks past the rows)
    "g8_chunk": TINY_PREFILL_2K.shrink(name="bwd_g8", batch=2, seq_q=700, seq_kv=1500,
                                       q_start=650, n_q_heads=16, n_kv_heads=2, top_k=6),
    # G = 8 over 4 KV heads, k larger than the causal block count of most rows
    "g8_hkv4": TINY_PREFILL_2K.shrink(name="bwd_hkv4", seq_q=520, seq_kv=520, n_q_heads=32,
                                      n_kv_heads=4, top_k=12),
    # group sizes outside 4 and 8 take the per-row dq kernel
    "g2_rowwise": TINY_PREFILL_2K.shrink(name="bwd_g2", seq_q=300, seq_kv=300, n_q_heads=8,
                                         n_kv_heads=4, top_k=3),
    "g16_rowwise": TINY_PREFILL_2K.shrink(name="bwd_g16", seq_q=400, seq_kv=900, q_start=500,
                                          n_q_heads=32, n_kv_heads=2, top_k=6),
    # 1536 rows of one KV head at G = 16 (4 rows per 64-column chunk): the
    # first blocks' row lists run to hundreds of chunks in the dK/dV pass
    "g16_long_lists": TINY_PREFILL_2K.shrink(name="bwd_g16s", seq_q=1536, seq_kv=1536, n_q_heads=16,
                                        n_kv_heads=1, top_k=8),
}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def oprob(w):
    return O.Problem(w.batch, w.seq_q, w.seq_kv, w.q_start, w.n_q_heads, w.n_kv_heads,
                     w.head_dim, w.n_idx_heads, w.idx_head_dim, w.block_size, w.top_k, False,
                     w.softmax_scale)


def rel_errors(gpu, ref):
    d = np.abs(gpu - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-30)), float(d.mean() / max(np.abs(ref).mean(), 1e-30))


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(case):
    need_gpu()
    w = CASES[case]
    print(f"[backward] {case}: B={w.batch} Sq={w.seq_q} Skv={w.seq_kv} q_start={w.q_start} "
          f"Hq={w.n_q_heads} Hkv={w.n_kv_heads} k={w.top_k}", flush=True)
    inp = generate(w, "cuda")
    p = msa.Problem.from_workload(w)
    bs = msa.msa_index_block_scores(p, inp.iq, inp.ik)
    sel = msa.msa_topk_blocks(p, bs)
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_q), dtype=torch.float32, device="cuda")
    out = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse)
    dout = cotangent(out, w.seed + 7)
    dq, dk, dv = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse, dout)
    dq2, dk2, dv2 = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse,
                                                         dout)
    torch.cuda.synchronize()
    for a, b, n in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(a, b), f"{n} differs between two identical calls"
    sel_rows = sel.permute(0, 2, 1, 3).contiguous().cpu().numpy()  # [B][Sq][Hkv][k]
    rq, rk, rv = O.attend_backward(oprob(w), f64(inp.q), f64(inp.k), f64(inp.v), f64(dout), None,
                                   sel_rows)
    # keys past the last row's position are read by no row: exactly zero
    last = w.q_start + w.seq_q
    if last < w.seq_kv:
        assert not torch.any(dk[:, :, last:]) and not torch.any(dv[:, :, last:])
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        mx, mn = rel_errors(f64(g), r)
        print(f"  {name}: max {mx:.2e} mean {mn:.2e} (of the reference's max / mean magnitude)",
              flush=True)
        assert mx <= MAX_REL and mn <= MEAN_REL, (name, mx, mn)


def test_backward_bounded_wait_failure_gives_nan():
    """The tile-union dq pass waits on its ring's tags with the library's
    bound.  Forced down to one poll from the host, waves give up early: every
    kernel still exits normally and rows of the affected tiles get NaN dq, while
    dk and dv (a pass with no waits) are unchanged.  With the default bound
    restored the call equals one made before the knob was touched."""
    need_gpu()
    w = PREFILL_32K.shrink(seq_q=4096, seq_kv=4096)
    inp = generate(w, "cuda")
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, msa.msa_index_block_scores(p, inp.iq, inp.ik))
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_q), dtype=torch.float32, device="cuda")
    out = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse)
    dout = cotangent(out, w.seed + 7)
    ref = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse, dout)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(t).all()) for t in ref)
    try:
        msa.msa_set_wait_limit(1)
        bad = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse, dout)
        torch.cuda.synchronize()
        nan_rows = int(torch.isnan(bad[0]).any(dim=3).any(dim=2).sum().item())  # [B][Sq]
        print(f"forced give-up: rows with NaN dq {nan_rows} of {w.seq_q}", flush=True)
        assert nan_rows > 0
        assert torch.equal(bad[1], ref[1]) and torch.equal(bad[2], ref[2])
    finally:
        msa.msa_set_wait_limit(0)
    again = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse, dout)
    torch.cuda.synchronize()
    for a, b in zip(again, ref):
        assert torch.equal(a, b)


def _row_oracle_dq(w, inp, sel, dout, t):
    """The oracle's dq of row t alone: a compact problem holding only the
    row's selected blocks (ascending, own block last) with the row at the same
    offset inside its own block attends exactly the row's tokens."""
    pos = w.q_start + t
    cur = pos // w.block_size
    m = min(w.top_k, cur + 1)
    blocks = sel[0, :, t, :m].long()                                   # [Hkv][m], own last
    tok = (blocks.unsqueeze(-1) * w.block_size +
           torch.arange(w.block_size, device=blocks.device)).reshape(w.n_kv_heads, -1)
    kk = torch.stack([inp.k[0, h].index_select(0, tok[h].clamp(max=w.seq_kv - 1))
                      for h in range(w.n_kv_heads)]).unsqueeze(0)       # [1][Hkv][m*64][D]
    vv = torch.stack([inp.v[0, h].index_select(0, tok[h].clamp(max=w.seq_kv - 1))
                      for h in range(w.n_kv_heads)]).unsqueeze(0)
    p = O.Problem(1, 1, m * w.block_size, (m - 1) * w.block_size + pos % w.block_size,
                  w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_idx_heads, w.idx_head_dim,
                  w.block_size, m, False, w.softmax_scale)
    s = np.tile(np.arange(m, dtype=np.int32), (1, 1, w.n_kv_heads, 1))  # [1][1][Hkv][m]
    dq, _, _ = O.attend_backward(p, f64(inp.q[:, t:t + 1]), f64(kk), f64(vv),
                                 f64(dout[:, t:t + 1]), None, s)
    return dq[0, 0]


def test_backward_128k_sampled_rows_and_sum_rules():
    """The 128K workload at full size, as the bench runs it.  dq of a
    stratified row sample against the oracle (compact per-row problems); dk
    and dv of every key through the sum rules: per (KV head, dim) the sum of
    dk over keys vanishes and the sum of dv equals the sum of dout over the
    rows and query heads reading that KV head.  The residuals are rounding:
    the kernels round P and dS to bf16, so a row's weights sum to one and its
    dS to zero only up to that rounding, and a gradient entry with a dropped
    or wrong term would leave a residual of order one; bound 5e-4 of the sum
    of magnitudes."""
    need_gpu()
    from block_sparse_gqa_02_amd.configs import PREFILL_128K as w
    import parity as PAR
    print(f"[backward] {w.name} full size", flush=True)
    inp = generate(w, "cuda")
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, msa.msa_index_block_scores(p, inp.iq, inp.ik))
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_q), dtype=torch.float32, device="cuda")
    out = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse)
    dout = cotangent(out, w.seed + 7)
    dq, dk, dv = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse, dout)
    torch.cuda.synchronize()
    G = w.group
    sk = dk.double().sum(dim=2)                                  # [B][Hkv][D]
    ak = dk.double().abs().sum(dim=2)
    want = dout.double().reshape(w.batch, w.seq_q, w.n_kv_heads, G, w.head_dim).sum(dim=(1, 3))
    sv = dv.double().sum(dim=2)
    av = dv.double().abs().sum(dim=2)
    rk = float((sk.abs() / ak).max())
    rv = float(((sv - want).abs() / av).max())
    print(f"  sum rules: |sum dk| / sum |dk| <= {rk:.2e}, |sum dv - sum dout| / sum |dv| <= {rv:.2e}",
          flush=True)
    assert rk <= 5e-4 and rv <= 5e-4, (rk, rv)
    rows = PAR.sample_rows(w.seq_q, w.q_start, w.block_size, seed=7, n_uniform=48, n_log=8)
    rows = rows[np.random.default_rng(7).permutation(len(rows))[:96]]
    gq = f64(dq[0, torch.as_tensor(rows, device="cuda")])             # [n][Hq][D]
    ref = np.stack([_row_oracle_dq(w, inp, sel, dout, int(t)) for t in rows])
    mx, mn = rel_errors(gq, ref)
    print(f"  dq on {len(rows)} rows: max {mx:.2e} mean {mn:.2e}", flush=True)
    assert mx <= MAX_REL and mn <= MEAN_REL, (mx, mn)


def test_backward_g4_rows_past_one_union_window():
    """Groups of 4 (64-row tiles in the ring dq kernel) over rows whose causal
    range spans two 512-block union windows: 1500 rows at q_start 38000 of a
    40000-token cache, k = 24.  dk and dv through the sum rules, dq of a row
    sample on both sides of the window boundary against the oracle (compact
    per-row problems)."""
    need_gpu()
    import parity as PAR
    w = TINY_PREFILL_2K.shrink(name="bwd_g4_roll", seq_q=1500, seq_kv=40000, q_start=38000,
                               n_q_heads=16, n_kv_heads=4, top_k=24)
    print(f"[backward] {w.name}: Sq={w.seq_q} Skv={w.seq_kv} q_start={w.q_start} G={w.group}",
          flush=True)
    inp = generate(w, "cuda")
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, msa.msa_index_block_scores(p, inp.iq, inp.ik))
    assert int(sel.max()) >= 512 and int(sel[sel >= 0].min()) < 512  # both windows are read
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_q), dtype=torch.float32, device="cuda")
    out = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse)
    dout = cotangent(out, w.seed + 7)
    dq, dk, dv = msa.msa_sparse_attn_prefill_backward(p, inp.q, inp.k, inp.v, sel, out, lse, dout)
    torch.cuda.synchronize()
    G = w.group
    sk = dk.double().sum(dim=2)
    ak = dk.double().abs().sum(dim=2)
    want = dout.double().reshape(w.batch, w.seq_q, w.n_kv_heads, G, w.head_dim).sum(dim=(1, 3))
    sv = dv.double().sum(dim=2)
    av = dv.double().abs().sum(dim=2)
    rk = float((sk.abs() / ak).max())
    rv = float(((sv - want).abs() / av).max())
    print(f"  sum rules: {rk:.2e} {rv:.2e}", flush=True)
    assert rk <= 5e-4 and rv <= 5e-4, (rk, rv)
    rows = PAR.sample_rows(w.seq_q, w.q_start, w.block_size, seed=11, n_uniform=96, n_log=8)
    gq = f64(dq[0, torch.as_tensor(rows, device="cuda")])
    ref = np.stack([_row_oracle_dq(w, inp, sel, dout, int(t)) for t in rows])
    mx, mn = rel_errors(gq, ref)
    print(f"  dq on {len(rows)} rows: max {mx:.2e} mean {mn:.2e}", flush=True)
    assert mx <= MAX_REL and mn <= MEAN_REL, (mx, mn)
