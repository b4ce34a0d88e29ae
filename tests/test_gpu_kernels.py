"""Per-kernel parity of the HIP path against the CPU oracle at small sizes that
still span several tiles and ragged tails (every row checked)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_02_amd as msa
from block_sparse_gqa_02_amd.configs import TINY_PREFILL_2K, DECODE_32x256K, PREFILL_32K
from block_sparse_gqa_02_amd.inputs import bf16_bits, generate
import oracle.oracle as O
import parity as PAR

pytestmark = pytest.mark.gpu

DEV = "cuda"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oprob(w):
    return O.Problem(w.batch, w.seq_q, w.seq_kv, w.q_start, w.n_q_heads, w.n_kv_heads,
                     w.head_dim, w.n_idx_heads, w.idx_head_dim, w.block_size, w.top_k, w.decode,
                     w.softmax_scale)


def host(inp):
    return dict(q=bf16_bits(inp.q), k=bf16_bits(inp.k), v=bf16_bits(inp.v),
                iq=bf16_bits(inp.iq), ik=bf16_bits(inp.ik),
                seq_lens=None if inp.seq_lens is None else inp.seq_lens.cpu().numpy())


def positions(w, seq_lens):
    if w.decode:
        return np.array(seq_lens) - 1
    return w.q_start + np.arange(w.seq_q)


def oracle_all(w, h, rows=None):
    p = oprob(w)
    if rows is None:
        rows = np.arange(w.batch * w.seq_q)
    return O.forward_rows_parallel(p, h["q"], h["k"], h["v"], h["iq"], h["ik"], h["seq_lens"],
                                   rows, PAR.host_threads(), want_scores=True)


PREFILL_SMALL = [
    # name, overrides (seq_q, seq_kv, q_start, heads, k)
    ("g4_hkv2_ragged", dict(seq_q=1000, seq_kv=1000, q_start=0, n_q_heads=8, n_kv_heads=2, top_k=5)),
    ("g8_hkv4_offset", dict(seq_q=333, seq_kv=1500, q_start=1100, n_q_heads=32, n_kv_heads=4, top_k=7)),
    ("g4_hkv1", dict(seq_q=700, seq_kv=700, q_start=0, n_q_heads=4, n_kv_heads=1, top_k=3)),
    ("batch2_k_all", dict(batch=2, seq_q=300, seq_kv=300, q_start=0, n_q_heads=8, n_kv_heads=2, top_k=64)),
    ("g16_rowwise", dict(seq_q=400, seq_kv=900, q_start=500, n_q_heads=32, n_kv_heads=2, top_k=6)),
    ("g2_rowwise", dict(seq_q=300, seq_kv=300, q_start=0, n_q_heads=8, n_kv_heads=4, top_k=3)),
    ("g8_many_tiles", dict(seq_q=1500, seq_kv=4000, q_start=2500, n_q_heads=16, n_kv_heads=2, top_k=20)),
    # rows past 512 causal blocks: the tile-union kernel's block windows roll over
    ("g4_two_windows", dict(seq_q=300, seq_kv=40000, q_start=39700, n_q_heads=8, n_kv_heads=2, top_k=24)),
    ("g8_two_windows", dict(seq_q=200, seq_kv=36000, q_start=35800, n_q_heads=16, n_kv_heads=2, top_k=24)),
    # a tile's rows select fewer blocks than the context holds (48 k < 625 for
    # groups of 8, 96 k < 625 for groups of 4): the KV-block-stationary schedule
    ("g8_kvs", dict(seq_q=310, seq_kv=40000, q_start=39690, n_q_heads=16, n_kv_heads=2, top_k=8)),
    ("g4_kvs", dict(seq_q=250, seq_kv=40000, q_start=39750, n_q_heads=8, n_kv_heads=2, top_k=5)),
    ("g8_kvs_batch2_k1", dict(batch=2, seq_q=130, seq_kv=20000, q_start=19870, n_q_heads=32,
                              n_kv_heads=4, top_k=1)),
    ("g8_kvs_batch2", dict(batch=2, seq_q=200, seq_kv=20000, q_start=19800, n_q_heads=32,
                           n_kv_heads=4, top_k=6)),
]


@pytest.mark.parametrize("integer", [True, False], ids=["integer", "normal"])
@pytest.mark.parametrize("name,ov", PREFILL_SMALL, ids=[x[0] for x in PREFILL_SMALL])
def test_prefill_pipeline_small(name, ov, integer):
    need_gpu()
    w = TINY_PREFILL_2K.shrink(**ov)
    inp = generate(w, DEV, seed=1234, integer=integer)
    p = msa.Problem.from_workload(w)
    bs = msa.msa_index_block_scores(p, inp.iq, inp.ik)
    sel = msa.msa_topk_blocks(p, bs)
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_q), dtype=torch.float32, device=DEV)
    out = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse)
    torch.cuda.synchronize()
    h = host(inp)
    o_sel, o_out, o_lse, o_sc = oracle_all(w, h)
    bs_h, sel_h = bs.cpu().numpy(), sel.cpu().numpy()
    out_h = out.float().cpu().numpy()
    lse_h = lse.cpu().numpy()
    pos = positions(w, None)
    ties = 0
    for b in range(w.batch):
        for t in range(w.seq_q):
            r = b * w.seq_q + t
            cur = int(pos[t]) // 64
            for hh in range(w.n_kv_heads):
                ref = o_sc[r, hh, : cur + 1]
                got = bs_h[b, hh, t, : cur + 1]
                assert got[cur] == np.inf
                if integer:
                    assert np.array_equal(got[:cur], ref[:cur]), (b, t, hh)
                else:
                    err = np.abs(got[:cur].astype(np.float64) - ref[:cur])
                    assert np.all(err <= 1e-5 * np.maximum(1.0, np.abs(ref[:cur]))), (b, t, hh)
                ties += PAR.check_selection_row(sel_h[b, hh, t], ref, cur, w.top_k, integer,
                                                f"row {t} head {hh}")
    # attention on the GPU's own selection
    p_o = oprob(w)
    ref_out = np.empty_like(out_h, dtype=np.float64)
    ref_lse = np.empty_like(lse_h, dtype=np.float64)
    for b in range(w.batch):
        for t in range(w.seq_q):
            o, l = O.attend_row(p_o, h["q"], h["k"], h["v"], None, sel_h[b, :, t], b, t)
            ref_out[b, t] = o
            ref_lse[b, :, t] = l
    PAR.assert_attention_close(out_h, ref_out, name)
    assert np.allclose(lse_h, ref_lse, atol=1e-3, rtol=1e-4)
    print(f"{name}: tie-band mismatches {ties}")


@pytest.mark.parametrize("k,nblk,seed", [(1, 40, 0), (5, 130, 1), (64, 700, 2), (200, 513, 3),
                                         (256, 256, 4), (8, 32, 5), (64, 1100, 6), (200, 1500, 7),
                                         (1, 1024, 8), (3, 4096, 9), (64, 5000, 10),
                                         (128, 9000, 11), (256, 16384, 12),
                                         # past 16384 candidates: the wide-row kernel
                                         (64, 20000, 13), (128, 17000, 14), (200, 18000, 15),
                                         (256, 16500, 16),
                                         # k of 129..192: the 320-entry list instances
                                         (150, 700, 17), (150, 17500, 18)])
def test_topk_exact_against_oracle_on_same_scores(k, nblk, seed):
    """Top-k alone on synthetic scores full of exact ties (integers, -0/+0):
    the decision is taken on identical fp32 values, so it must be bit-exact."""
    need_gpu()
    g = torch.Generator().manual_seed(seed)
    Sq, Hkv = 2 * 64 * 3 + 17, 2
    seq_kv = nblk * 64
    q_start = seq_kv - Sq
    sc = torch.randint(-3, 4, (1, Hkv, Sq, nblk), generator=g).float()
    sc[sc == 0] = torch.where(torch.rand(sc[sc == 0].shape, generator=g) < 0.5,
                              torch.tensor(-0.0), torch.tensor(0.0))
    sc[0, 1] = torch.randn((Sq, nblk), generator=g)  # one head without ties
    w = TINY_PREFILL_2K.shrink(seq_q=Sq, seq_kv=seq_kv, q_start=q_start, n_kv_heads=Hkv,
                               n_q_heads=8, top_k=k)
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, sc.to(DEV)).cpu().numpy()
    po = oprob(w)
    for hh in range(Hkv):
        for t in range(Sq):
            cur = (q_start + t) // 64
            row = sc[0, hh, t].numpy().copy()
            row[cur] = np.inf  # the oracle's scores carry the own block at +inf
            ref = O.select_row(po, row, cur)
            assert np.array_equal(sel[0, hh, t], ref), (hh, t, sel[0, hh, t], ref)


@pytest.mark.parametrize("k", [1, 9, 64])
def test_topk_radix_rows_shorter_than_k(k):
    """Few long rows (the work-group radix select): sequences whose causal
    blocks number fewer than, equal to or more than k, on scores full of exact
    ties; the selection must follow the (score desc, block asc) rule exactly."""
    need_gpu()
    nblk = 1100
    lens = [nblk * 64, 1, 64, 65, 129, 4100, 64 * 9, 64 * 9 + 1]
    w = DECODE_32x256K.shrink(batch=len(lens), seq_kv=nblk * 64, top_k=k)
    g = torch.Generator().manual_seed(40 + k)
    sc = torch.randint(-3, 4, (w.batch, w.n_kv_heads, 1, nblk), generator=g).float()
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, sc.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV))
    sel = sel.cpu().numpy()
    po = oprob(w)
    for b, L in enumerate(lens):
        cur = (L - 1) // 64
        for hh in range(w.n_kv_heads):
            row = sc[b, hh, 0].numpy().copy()
            row[cur] = np.inf
            ref = O.select_row(po, row, cur)
            assert np.array_equal(sel[b, hh, 0], ref), (b, hh, sel[b, hh, 0], ref)


@pytest.mark.parametrize("hkv", [4, 2, 1], ids=["hkv4", "hkv2", "hkv1"])
def test_index_scores_decode_and_topk_ragged(hkv):
    # with fewer KV heads than index heads, a KV head's block score is the max
    # over the index heads i = h (mod Hkv): the decode kernel folds them across lanes
    need_gpu()
    w = DECODE_32x256K.shrink(batch=5, seq_kv=5000, top_k=9, n_kv_heads=hkv, n_q_heads=8 * hkv)
    lens = [5000, 1, 4097, 64, 65]
    inp = generate(w, DEV, seed=77, seq_lens=lens)
    p = msa.Problem.from_workload(w)
    bs = msa.msa_index_block_scores(p, inp.iq, inp.ik, inp.seq_lens)
    sel = msa.msa_topk_blocks(p, bs, inp.seq_lens)
    torch.cuda.synchronize()
    h = host(inp)
    o_sel, _, _, o_sc = oracle_all(w, h)
    bs_h, sel_h = bs.cpu().numpy(), sel.cpu().numpy()
    for b, L in enumerate(lens):
        cur = (L - 1) // 64
        for hh in range(w.n_kv_heads):
            got = bs_h[b, hh, 0, : cur + 1]
            ref = o_sc[b, hh, : cur + 1]
            assert got[cur] == np.inf
            assert np.all(np.abs(got[:cur] - ref[:cur]) <= 1e-5 * np.maximum(1, np.abs(ref[:cur])))
            PAR.check_selection_row(sel_h[b, hh, 0], ref, cur, w.top_k, False, f"seq {b}")


@pytest.mark.parametrize("heads", [(32, 4), (8, 2)], ids=["g8", "g4_hkv2"])
@pytest.mark.parametrize("dense", [False, True], ids=["sparse", "dense"])
def test_decode_attention_ragged(dense, heads):
    need_gpu()
    w = DECODE_32x256K.shrink(batch=4, seq_kv=3000, top_k=11, n_q_heads=heads[0], n_kv_heads=heads[1])
    lens = [3000, 65, 1, 2048]
    inp = generate(w, DEV, seed=5, seq_lens=lens)
    p = msa.Problem.from_workload(w)
    lse = torch.empty((w.batch, w.n_q_heads, 1), dtype=torch.float32, device=DEV)
    if dense:
        out = msa.msa_dense_attn_decode(p, inp.q, inp.k, inp.v, inp.seq_lens, lse=lse)
    else:
        bs = msa.msa_index_block_scores(p, inp.iq, inp.ik, inp.seq_lens)
        sel = msa.msa_topk_blocks(p, bs, inp.seq_lens)
        out = msa.msa_sparse_attn_decode(p, inp.q, inp.k, inp.v, inp.seq_lens, sel, lse=lse)
        sel_h = sel.cpu().numpy()
    torch.cuda.synchronize()
    h = host(inp)
    po = oprob(w)
    out_h, lse_h = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        if dense:
            o, l = O.dense_row(po, h["q"], h["k"], h["v"], h["seq_lens"], b, 0)
        else:
            o, l = O.attend_row(po, h["q"], h["k"], h["v"], h["seq_lens"], sel_h[b, :, 0], b, 0)
        PAR.assert_attention_close(out_h[b, 0], o, f"seq {b}")
        assert np.allclose(lse_h[b, :, 0], l, atol=1e-3, rtol=1e-4)


def test_dense_prefill_small():
    need_gpu()
    w = PREFILL_32K.shrink(seq_q=300, seq_kv=400, q_start=100, top_k=1, block_offset_std=0.0)
    inp = generate(w, DEV, seed=9)
    p = msa.Problem.from_workload(w)
    lse = torch.empty((1, w.n_q_heads, w.seq_q), dtype=torch.float32, device=DEV)
    out = msa.msa_dense_attn_prefill(p, inp.q, inp.k, inp.v, lse=lse)
    torch.cuda.synchronize()
    h = host(inp)
    po = oprob(w)
    out_h, lse_h = out.float().cpu().numpy(), lse.cpu().numpy()
    ref = np.empty_like(out_h, dtype=np.float64)
    for t in range(w.seq_q):
        o, l = O.dense_row(po, h["q"], h["k"], h["v"], None, 0, t)
        ref[0, t] = o
        assert np.allclose(lse_h[0, :, t], l, atol=1e-3, rtol=1e-4)
    PAR.assert_attention_close(out_h, ref, "dense prefill")


def test_sparse_equals_dense_when_every_block_is_kept():
    """k >= nblk: the sparse kernels attend every causal block, so they must
    reproduce the dense kernel (both in the library)."""
    need_gpu()
    w = PREFILL_32K.shrink(seq_q=520, seq_kv=520, q_start=0, top_k=9, block_offset_std=0.0)
    inp = generate(w, DEV, seed=3)
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, msa.msa_index_block_scores(p, inp.iq, inp.ik))
    a = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel).float()
    d = msa.msa_dense_attn_prefill(p, inp.q, inp.k, inp.v).float()
    assert torch.max(torch.abs(a - d)).item() <= 1e-2


FUSED_CASES = [
    # seq_q, seq_kv, q_start, Hq, Hkv, k
    ("multi_split_k128", dict(seq_q=256, seq_kv=16384, q_start=16128, n_q_heads=32, n_kv_heads=4, top_k=128)),
    ("multi_split_unaligned", dict(seq_q=300, seq_kv=12000, q_start=11650, n_q_heads=8, n_kv_heads=2, top_k=37)),
    ("k1", dict(seq_q=200, seq_kv=9000, q_start=8700, n_q_heads=4, n_kv_heads=1, top_k=1)),
    ("k256", dict(seq_q=130, seq_kv=20000, q_start=19800, n_q_heads=8, n_kv_heads=2, top_k=256)),
    ("k150", dict(seq_q=150, seq_kv=14000, q_start=13850, n_q_heads=8, n_kv_heads=2, top_k=150)),
    ("short_rows", dict(seq_q=700, seq_kv=700, q_start=0, n_q_heads=8, n_kv_heads=2, top_k=6)),
]


@pytest.mark.parametrize("integer", [True, False], ids=["integer", "normal"])
@pytest.mark.parametrize("name,ov", FUSED_CASES, ids=[x[0] for x in FUSED_CASES])
def test_fused_equals_separate_and_oracle(name, ov, integer):
    """The fused kernel computes the same fp32 block maxima as the block-score
    kernel, so its selection must equal block scores + top-k exactly; both are
    also held to the oracle protocol on every row."""
    need_gpu()
    w = TINY_PREFILL_2K.shrink(**ov)
    inp = generate(w, DEV, seed=4321, integer=integer)
    p = msa.Problem.from_workload(w)
    sel_f = msa.msa_index_topk_fused(p, inp.iq, inp.ik)
    bs = msa.msa_index_block_scores(p, inp.iq, inp.ik)
    sel_s = msa.msa_topk_blocks(p, bs)
    torch.cuda.synchronize()
    assert torch.equal(sel_f, sel_s), "fused selection differs from block scores + top-k"
    h = host(inp)
    rows = np.arange(w.seq_q)
    _, _, _, o_sc = O.forward_rows_parallel(oprob(w), h["q"], h["k"], h["v"], h["iq"], h["ik"],
                                            None, rows, PAR.host_threads(), want_scores=True)
    sel_h = sel_f.cpu().numpy()
    for t in rows:
        cur = (w.q_start + t) // 64
        for hh in range(w.n_kv_heads):
            PAR.check_selection_row(sel_h[0, hh, t], o_sc[t, hh], cur, w.top_k, integer,
                                    f"{name} row {t} head {hh}")


@pytest.mark.parametrize("heads", [(32, 4), (8, 2), (8, 4)], ids=["g8_tiled", "g4_tiled", "g2_rowwise"])
def test_prefill_ignores_cache_rows_past_the_context(heads):
    """Rows of K and V at or past q_start + seq_q belong to no query's context:
    filling them with NaN must leave the output and LSE bit-identical (the
    tiled kernel's transposed V tiles repeat the last context row there, the
    diagonal K fetch re-reads the last used row, the row-wise kernel stops at
    the query)."""
    need_gpu()
    hq, hkv = heads
    w = TINY_PREFILL_2K.shrink(seq_q=300, seq_kv=1000, q_start=610, n_q_heads=hq, n_kv_heads=hkv,
                               top_k=6)
    inp = generate(w, DEV, seed=77)
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, msa.msa_index_block_scores(p, inp.iq, inp.ik))
    lse_a = torch.empty((1, w.n_q_heads, w.seq_q), dtype=torch.float32, device=DEV)
    lse_b = torch.empty_like(lse_a)
    a = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, lse=lse_a)
    ctx = w.q_start + w.seq_q
    k2, v2 = inp.k.clone(), inp.v.clone()
    k2[:, :, ctx:] = float("nan")
    v2[:, :, ctx:] = float("nan")
    b = msa.msa_sparse_attn_prefill(p, inp.q, k2, v2, sel, lse=lse_b)
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse_a, lse_b)


def test_sparse_prefill_bounded_wait_failure_is_reported():
    """The tile-union kernel's ring waits are bounded.  With the bound forced
    down to one poll from the host, waves give up early: every kernel still
    exits normally, the affected rows hold NaN and the workspace's status word
    reads 1.  With the default bound restored the same call is complete (word
    0) and equals a call made before the knob was touched."""
    need_gpu()
    w = PREFILL_32K.shrink(seq_q=4096, seq_kv=4096)
    inp = generate(w, DEV)
    p = msa.Problem.from_workload(w)
    sel = msa.msa_topk_blocks(p, msa.msa_index_block_scores(p, inp.iq, inp.ik))
    off = msa.msa_sparse_attn_prefill_status_offset(p)
    ws = torch.full((msa.msa_workspace_bytes(p, "sparse_attn_prefill"),), 7, dtype=torch.uint8,
                    device=DEV)
    word = lambda: int(ws[off:off + 4].view(torch.int32).item())
    ref = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, workspace=ws)
    torch.cuda.synchronize()
    assert word() == 0 and bool(torch.isfinite(ref.float()).all())
    try:
        msa.msa_set_wait_limit(1)
        bad = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, workspace=ws)
        torch.cuda.synchronize()
        nan_rows = int(torch.isnan(bad.float()).any(dim=3).any(dim=2).sum().item())  # [B][Sq]
        print(f"forced give-up: status word {word()}, rows with NaN {nan_rows} of {w.seq_q}",
              flush=True)
        assert word() == 1 and nan_rows > 0
    finally:
        msa.msa_set_wait_limit(0)
    again = msa.msa_sparse_attn_prefill(p, inp.q, inp.k, inp.v, sel, workspace=ws)
    torch.cuda.synchronize()
    assert word() == 0 and torch.equal(again, ref)
