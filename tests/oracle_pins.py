"""Pins of the CPU oracle to facts other than itself.

Each check takes a bound oracle library `L` (see oracle.lib) so that the same
checks also run against deliberately broken builds of the oracle
(test_oracle_mutants.py): every plausible mistake must fail at least one check.
A check raises AssertionError on failure.

What pins what:
  * dense attention   -> torch's scaled_dot_product_attention in float64
                         (a library routine), causal, grouped query heads;
  * sparse attention  -> the same library routine under an explicit boolean
                         mask built from the selection, and the closed forms
                         V == const -> O == const, Q == 0 -> O == mean of V over
                         the attended tokens and LSE == log |T|, pos 0 -> V[0];
  * all blocks kept   -> sparse forward == dense attention (the identity the
                         method must satisfy when nothing is pruned);
  * block scores      -> integer closed forms (one-hot index queries read one
                         index-key column, so a block score is a plain max of
                         integers), exact rational brute force on tiny inputs,
                         causality and index-head attribution;
  * selection         -> exhaustive subset enumeration (the k-subset with the
                         largest score sum, ties to the lexicographically
                         smallest ascending list) and the rank-count formula;
  * golden            -> a hand-derived worked example (tests/golden);
  * block size 1      -> exact rational token scores, a lexicographic sort for
                         the selection, library attention under a token mask
                         (token-level selection, the pages' contrast case);
  * gradient          -> central differences of the fp64 forward, torch
                         autograd of dense causal attention (all blocks kept),
                         and the sum rules over keys (sum of dk = 0, sum of
                         dv = sum of dout over the rows reading the head);
  * index KL          -> central differences of the loss, torch autograd of
                         the definition written with library softmaxes, zero
                         loss and gradient when the distributions agree (and
                         at one attended token), the key sum rule and the
                         invariance of the loss under a shift of every key.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

import oracle.oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


def int_bf16(shape, gen, lo=-2, hi=2):
    return torch.randint(lo, hi + 1, shape, generator=gen).to(torch.bfloat16)


def problem(B=1, Sq=8, Skv=8, q_start=0, Hq=4, Hkv=2, D=16, Hi=4, Di=8, bs=4, k=2,
            decode=False, scale=None):
    return O.Problem(B, Sq, Skv, q_start, Hq, Hkv, D, Hi, Di, bs, k, decode,
                     scale if scale is not None else 1.0 / math.sqrt(D))


def make(p: O.Problem, seed=0, integer=False):
    g = torch.Generator().manual_seed(seed)
    mk = (lambda s: int_bf16(s, g)) if integer else (lambda s: rand_bf16(s, g))
    q = mk((p.batch, p.seq_q, p.n_q_heads, p.head_dim))
    k = mk((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    v = mk((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    iq = mk((p.batch, p.seq_q, p.n_idx_heads, p.idx_head_dim))
    ik = mk((p.batch, p.seq_kv, p.idx_head_dim))
    return q, k, v, iq, ik


def sdpa_row(p, q, k, v, b, t, pos, allowed=None):
    """Library attention (float64) of one row; allowed[hq, j] bool or None."""
    qq = q[b, t].to(torch.float64).view(1, p.n_q_heads, 1, p.head_dim)
    kk = k[b, :, : pos + 1].to(torch.float64).unsqueeze(0)
    vv = v[b, :, : pos + 1].to(torch.float64).unsqueeze(0)
    if allowed is None:
        o = F.scaled_dot_product_attention(qq, kk, vv, scale=p.softmax_scale, enable_gqa=True)
    else:
        m = torch.as_tensor(allowed[:, : pos + 1]).view(1, p.n_q_heads, 1, pos + 1)
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=p.softmax_scale,
                                           enable_gqa=True)
    return o.view(p.n_q_heads, p.head_dim).numpy()


def close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------- dense / attention
def check_dense_vs_library(L):
    for (Hq, Hkv, D, S, seed) in [(4, 1, 16, 37, 1), (8, 2, 128, 130, 2), (2, 2, 8, 5, 3)]:
        p = problem(Sq=S, Skv=S, Hq=Hq, Hkv=Hkv, D=D, Hi=Hkv, bs=8, k=1)
        q, k, v, _, _ = make(p, seed)
        for t in range(S):
            out, _ = O.dense_row(p, bits(q), bits(k), bits(v), None, 0, t, L=L)
            close(out, sdpa_row(p, q, k, v, 0, t, t), 1e-12, f"dense row {t}")


def check_attend_vs_masked_library(L):
    """Arbitrary (random, possibly non-causal-looking) selections; the oracle
    must equal library attention under the mask 'token in a selected block of
    this query head's KV head, and j <= pos'."""
    p = problem(Sq=40, Skv=40, Hq=6, Hkv=3, D=32, Hi=3, bs=4, k=3)
    q, k, v, _, _ = make(p, 11)
    rng = np.random.default_rng(5)
    G = p.n_q_heads // p.n_kv_heads
    for t in range(p.seq_q):
        pos, cur = t, t // p.block_size
        sel = np.full((p.n_kv_heads, p.top_k), -1, np.int32)
        for h in range(p.n_kv_heads):
            others = [c for c in range(cur)]
            pick = sorted(set(rng.choice(others, size=min(len(others), p.top_k - 1),
                                         replace=False).tolist()) | {cur}) if others else [cur]
            sel[h, : len(pick)] = pick
        allowed = np.zeros((p.n_q_heads, p.seq_kv), bool)
        for hq in range(p.n_q_heads):
            for c in sel[hq // G]:
                if c >= 0:
                    allowed[hq, c * p.block_size:(c + 1) * p.block_size] = True
        out, _ = O.attend_row(p, bits(q), bits(k), bits(v), None, sel, 0, t, L=L)
        close(out, sdpa_row(p, q, k, v, 0, t, pos, allowed), 1e-12, f"attend row {t}")


def check_all_blocks_equals_dense(L):
    for (Hq, Hkv, Hi, S, bs, seed, qs) in [(8, 2, 4, 70, 8, 4, 0), (4, 4, 4, 64, 16, 5, 0),
                                           (4, 1, 4, 50, 4, 6, 13)]:
        Skv = S + qs
        p = problem(Sq=S, Skv=Skv, q_start=qs, Hq=Hq, Hkv=Hkv, D=32, Hi=Hi, Di=16, bs=bs,
                    k=(Skv + bs - 1) // bs + 3)
        q, k, v, iq, ik = make(p, seed)
        rows = np.arange(S)
        sel, out, lse, _ = O.forward_rows(p, bits(q), bits(k), bits(v), bits(iq), bits(ik),
                                          None, rows, L=L)
        for t in range(S):
            d, dl = O.dense_row(p, bits(q), bits(k), bits(v), None, 0, t, L=L)
            close(out[t], d, 1e-12, f"all-blocks row {t}")
            close(lse[t], dl, 1e-12, f"all-blocks lse row {t}")


def check_softmax_closed_forms(L):
    p = problem(Sq=24, Skv=24, Hq=4, Hkv=2, D=8, Hi=2, bs=4, k=3)
    q, k, v, iq, ik = make(p, 7)
    rows = np.arange(p.seq_q)
    # V == per-dimension constant: every softmax row sums to 1 so O == that constant
    const = torch.arange(1, p.head_dim + 1, dtype=torch.float32).to(torch.bfloat16)
    vc = const.view(1, 1, 1, -1).expand_as(v).contiguous()
    _, out, _, _ = O.forward_rows(p, bits(q), bits(k), bits(vc), bits(iq), bits(ik), None, rows,
                                  L=L)
    close(out, np.broadcast_to(const.to(torch.float64).numpy(), out.shape), 1e-12, "V==const")
    # Q == 0: uniform weights -> O = mean of V over T, LSE = log |T|
    qz = torch.zeros_like(q)
    sel, out, lse, _ = O.forward_rows(p, bits(qz), bits(k), bits(v), bits(iq), bits(ik), None,
                                      rows, L=L)
    G = p.n_q_heads // p.n_kv_heads
    for t in rows:
        for hq in range(p.n_q_heads):
            toks = [j for c in sel[t, hq // G] if c >= 0
                    for j in range(c * p.block_size, (c + 1) * p.block_size) if j <= t]
            exp = v[0, hq // G, toks].to(torch.float64).mean(0).numpy()
            close(out[t, hq], exp, 1e-12, f"Q==0 mean row {t}")
            close(lse[t, hq], math.log(len(toks)), 1e-12, f"Q==0 lse row {t}")
    # position 0 attends to itself only: O == V[0]
    close(out[0], v[0, np.arange(p.n_q_heads) // G, 0].to(torch.float64).numpy(), 1e-12,
          "pos0 -> V[0]")


def check_decode_is_last_prefill_row(L):
    """Decode semantics: the query of a sequence of length L sits at L-1 and
    sees the whole cache; it equals a one-row prefill at q_start = L-1."""
    B, Skv = 3, 48
    lens = [48, 17, 1]
    pd = problem(B=B, Sq=1, Skv=Skv, Hq=4, Hkv=2, D=16, Hi=4, Di=8, bs=8, k=3, decode=True)
    q, k, v, iq, ik = make(pd, 9)
    sel, out, lse, sc = O.forward_rows(pd, bits(q), bits(k), bits(v), bits(iq), bits(ik),
                                       np.array(lens, np.int32), np.arange(B), want_scores=True,
                                       L=L)
    for b, Lb in enumerate(lens):
        assert O.position(pd, np.array(lens, np.int32), b, 0, L=L) == Lb - 1
        pp = problem(B=1, Sq=1, Skv=Skv, q_start=Lb - 1, Hq=4, Hkv=2, D=16, Hi=4, Di=8, bs=8,
                     k=3)
        s2, o2, l2, sc2 = O.forward_rows(pp, bits(q[b:b + 1]), bits(k[b:b + 1]), bits(v[b:b + 1]),
                                         bits(iq[b:b + 1]), bits(ik[b:b + 1]), None,
                                         np.array([0]), want_scores=True, L=L)
        assert np.array_equal(sel[b], s2[0]), "decode selection != prefill at L-1"
        close(out[b], o2[0], 0.0, "decode out")
        d, _ = O.dense_row(pd, bits(q), bits(k), bits(v), np.array(lens, np.int32), b, 0, L=L)
        if Lb <= pd.block_size * pd.top_k:
            close(out[b], d, 1e-12, "short decode == dense")


# ----------------------------------------------------------------- block scores
def check_block_scores_integer_closed_form(L):
    """One-hot index queries: head i reads column d_i of index-K, so a block
    score is max over the attributed heads and the block's tokens of an integer
    table entry.  The table is a formula of (j, d), not an oracle output."""
    Hi, Hkv, Di, bs, S = 4, 2, 8, 4, 29
    p = problem(Sq=S, Skv=S, Hq=4, Hkv=Hkv, D=8, Hi=Hi, Di=Di, bs=bs, k=2)
    col = [5, 2, 7, 0]  # head i is one-hot at dim col[i]
    iq = torch.zeros((1, S, Hi, Di))
    for i in range(Hi):
        iq[0, :, i, col[i]] = 1.0
    table = lambda j, d: ((j * 37 + d * 11) % 17) - 8  # noqa: E731
    ik = torch.tensor([[table(j, d) for d in range(Di)] for j in range(S)],
                      dtype=torch.float32).view(1, S, Di)
    iqb, ikb = bits(iq.to(torch.bfloat16)), bits(ik.to(torch.bfloat16))
    for t in range(S):
        got = O.block_scores_row(p, iqb, ikb, None, 0, t, L=L)
        cur = t // bs
        for h in range(Hkv):
            for c in range(p.nblk):
                if c < cur:
                    exp = max(table(j, col[i]) for i in range(Hi) if i % Hkv == h
                              for j in range(c * bs, (c + 1) * bs))
                elif c == cur:
                    exp = math.inf
                else:
                    exp = -math.inf
                assert got[h, c] == exp, f"row {t} head {h} block {c}: {got[h, c]} != {exp}"


def check_block_scores_rational_brute_force(L):
    """Exact rational recomputation of every token score on a tiny problem,
    then the fp32 rounding of the block max."""
    p = problem(Sq=12, Skv=12, Hq=2, Hkv=1, D=4, Hi=4, Di=6, bs=3, k=2)
    g = torch.Generator().manual_seed(21)
    iq, ik = rand_bf16((1, 12, 4, 6), g), rand_bf16((1, 12, 6), g)
    iqf = [[[Fraction(float(x)) for x in iq[0, t, i]] for i in range(4)] for t in range(12)]
    ikf = [[Fraction(float(x)) for x in ik[0, j]] for j in range(12)]
    for t in range(12):
        got = O.block_scores_row(p, bits(iq), bits(ik), None, 0, t, L=L)
        for c in range(t // 3):
            best = max(sum(a * b for a, b in zip(iqf[t][i], ikf[j]))
                       for i in range(4) for j in range(3 * c, 3 * c + 3))
            assert got[0, c] == np.float32(float(best)), f"row {t} block {c}"


def check_block_scores_causal_and_attribution(L):
    p = problem(Sq=20, Skv=20, Hq=4, Hkv=2, D=8, Hi=4, Di=8, bs=4, k=2)
    g = torch.Generator().manual_seed(8)
    iq, ik = rand_bf16((1, 20, 4, 8), g), rand_bf16((1, 20, 8), g)
    for t in [0, 5, 11, 19]:
        base = O.block_scores_row(p, bits(iq), bits(ik), None, 0, t, L=L)
        cur = t // 4
        ik2 = ik.clone()
        ik2[0, cur * 4:] = rand_bf16((20 - cur * 4, 8), g, 9.0)  # own + future blocks
        assert np.array_equal(base, O.block_scores_row(p, bits(iq), bits(ik2), None, 0, t, L=L)), \
            "block scores depend on own/future tokens"
    # only index head 3 active: KV head 1 (= 3 mod 2) sees its scores, KV head 0 sees 0
    iq3 = torch.zeros_like(iq)
    iq3[:, :, 3] = iq[:, :, 3]
    t = 19
    got = O.block_scores_row(p, bits(iq3), bits(ik), None, 0, t, L=L)
    for c in range(t // 4):
        s = [float((iq[0, t, 3].double() * ik[0, j].double()).sum()) for j in range(4 * c, 4 * c + 4)]
        assert got[1, c] == np.float32(max(s)), "index head 3 must drive KV head 1"
        assert got[0, c] == 0.0, "KV head 0 must only see index heads 0 and 2"
    # permuting tokens inside a block keeps scores; swapping two blocks swaps them
    perm = ik.clone()
    perm[0, 4:8] = ik[0, [6, 4, 7, 5]]
    perm[0, 8:12], perm[0, 12:16] = ik[0, 12:16], ik[0, 8:12]
    a = O.block_scores_row(p, bits(iq), bits(ik), None, 0, 19, L=L)
    b2 = O.block_scores_row(p, bits(iq), bits(perm), None, 0, 19, L=L)
    assert np.array_equal(a[:, 1], b2[:, 1]) and np.array_equal(a[:, 2], b2[:, 3]) \
        and np.array_equal(a[:, 3], b2[:, 2]), "block/token mapping"


def check_planted_winners_per_kv_head(L):
    """Each KV head is steered to a different block by its index heads; the
    selections must differ per KV head (no cross-head merging)."""
    S, bs = 64, 8
    p = problem(Sq=S, Skv=S, Hq=4, Hkv=2, D=8, Hi=4, Di=8, bs=bs, k=2)
    q, k, v, iq, ik = make(p, 12)
    iq = iq * 0.1
    ik = ik * 0.1
    ik[0, 8:16, 0] = 40.0   # block 1 lights up dim 0
    ik[0, 32:40, 1] = 40.0  # block 4 lights up dim 1
    iq[0, :, 0, 0] = 1.0    # index head 0 (KV head 0) looks at dim 0
    iq[0, :, 2, 0] = 1.0
    iq[0, :, 1, 1] = 1.0    # index heads 1, 3 (KV head 1) look at dim 1
    iq[0, :, 3, 1] = 1.0
    t = 63
    sel, _, _, _ = O.forward_rows(p, bits(q), bits(k), bits(v), bits(iq.to(torch.bfloat16)),
                                  bits(ik.to(torch.bfloat16)), None, np.array([t]), L=L)
    assert sel[0, 0].tolist() == [1, 7], sel[0, 0]
    assert sel[0, 1].tolist() == [4, 7], sel[0, 1]


# ----------------------------------------------------------------- selection
def _brute_select(scores, cur, k):
    """Exhaustive: among k-subsets of [0, cur] containing the own block, the
    largest finite score sum wins; ties -> lexicographically smallest list."""
    m = min(k, cur + 1)
    best, best_key = None, None
    for sub in itertools.combinations(range(cur + 1), m):
        if cur not in sub:
            continue
        total = sum(Fraction(float(scores[c])) for c in sub if c != cur)
        key = (-total, sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return list(best) + [-1] * (k - m)


def check_select_brute_force(L):
    rng = np.random.default_rng(3)
    for trial in range(300):
        cur = int(rng.integers(0, 10))
        k = int(rng.integers(1, 7))
        s = rng.integers(-3, 4, size=cur + 1).astype(np.float32)  # many exact ties
        if trial % 3 == 0:
            s = rng.standard_normal(cur + 1).astype(np.float32)
        if trial % 7 == 0 and cur >= 2:
            s[1] = -0.0
            s[0] = 0.0  # -0 == +0: the lower index (0) must win the tie
        s[cur] = np.inf
        p = problem(k=k)
        got = O.select_row(p, s, cur, L=L)
        assert got.tolist() == _brute_select(s, cur, k), (s, cur, k, got)
        # rank-count characterisation of the same rule
        m = min(k, cur + 1)
        chosen = [c for c in range(cur + 1)
                  if sum(1 for c2 in range(cur + 1)
                         if s[c2] > s[c] or (s[c2] == s[c] and c2 < c)) < m]
        assert got[:m].tolist() == chosen


def check_select_edge_cases(L):
    s = np.array([5, 4, 3, 2, np.inf], np.float32)
    assert O.select_row(problem(k=1), s, 4, L=L).tolist() == [4]
    assert O.select_row(problem(k=7), s, 4, L=L).tolist() == [0, 1, 2, 3, 4, -1, -1]
    assert O.select_row(problem(k=3), s, 4, L=L).tolist() == [0, 1, 4]
    assert O.select_row(problem(k=3), np.array([np.inf], np.float32), 0, L=L).tolist() == [0, -1, -1]


# ----------------------------------------------------------------- golden
def check_golden_hand_example(L):
    with open(os.path.join(GOLDEN, "hand_example_bs2.json")) as f:
        ex = json.load(f)
    pr = ex["problem"]
    p = O.Problem(**pr)
    f16 = lambda a, shape: bits(torch.tensor(a, dtype=torch.float32).view(shape).to(torch.bfloat16))  # noqa: E731
    q = f16(ex["q"], (1, 1, p.n_q_heads, p.head_dim))
    k = f16(ex["k"], (1, p.n_kv_heads, p.seq_kv, p.head_dim))
    v = f16(ex["v"], (1, p.n_kv_heads, p.seq_kv, p.head_dim))
    iq = f16(ex["iq"], (1, 1, p.n_idx_heads, p.idx_head_dim))
    ik = f16(ex["ik"], (1, p.seq_kv, p.idx_head_dim))
    sel, out, lse, sc = O.forward_rows(p, q, k, v, iq, ik, None, np.array([0]), want_scores=True,
                                       L=L)
    exp = ex["expected"]
    want_scores = [math.inf if x == "inf" else x for x in exp["block_scores"]]
    assert sc[0, 0].tolist() == want_scores, sc
    assert sel[0, 0].tolist() == exp["selection"], sel
    e = math.e
    want_out = [[3.5, 6.5], [(3 + 4 * e) / (1 + e), (7 + 6 * e) / (1 + e)]]
    want_lse = [math.log(4.0), math.log(2 + 2 * e)]
    close(out[0], want_out, 1e-12, "golden out")
    close(lse[0], want_lse, 1e-12, "golden lse")
    assert exp["out_formula"] and exp["lse_formula"]


# ----------------------------------------------------------------- main-branch gradient
def _random_selection(p, rng):
    """[B][Sq][Hkv][k]: own block plus random earlier blocks, ascending, -1 padded."""
    sel = np.full((p.batch, p.seq_q, p.n_kv_heads, p.top_k), -1, np.int32)
    for b in range(p.batch):
        for t in range(p.seq_q):
            cur = (p.q_start + t) // p.block_size
            for h in range(p.n_kv_heads):
                others = list(range(cur))
                m = min(len(others), p.top_k - 1)
                pick = sorted(set(rng.choice(others, size=m, replace=False).tolist()) | {cur}) \
                    if m > 0 else [cur]
                sel[b, t, h, : len(pick)] = pick
    return sel


def _loss_f64(p, q, k, v, dout, sel, L):
    tot = 0.0
    for b in range(p.batch):
        for t in range(p.seq_q):
            o, _ = O.attend_row_f64(p, q, k, v, None, sel[b, t], b, t, L=L)
            tot += float(np.sum(dout[b, t] * o))
    return tot


def check_backward_finite_differences(L):
    """Gradient of sum(dout * out) against central differences of the fp64
    forward, on sampled coordinates of q, k and v (random selections, a ragged
    last block, two sequences)."""
    p = problem(B=2, Sq=11, Skv=11, Hq=4, Hkv=2, D=8, Hi=2, bs=4, k=2)
    rng = np.random.default_rng(21)
    q = rng.standard_normal((p.batch, p.seq_q, p.n_q_heads, p.head_dim))
    k = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    v = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    g = rng.standard_normal(q.shape)
    sel = _random_selection(p, rng)
    dq, dk, dv = O.attend_backward(p, q, k, v, g, None, sel, L=L)
    h = 1e-6
    for name, x, gx in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss_f64(p, q, k, v, g, sel, L)
            x[idx] = x0 - h
            lm = _loss_f64(p, q, k, v, g, sel, L)
            x[idx] = x0
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gx[idx]) <= 1e-6 * (1.0 + abs(fd)), \
                f"d{name}{idx}: analytic {gx[idx]:.9e} vs central difference {fd:.9e}"


def check_backward_dense_vs_autograd(L):
    """Every causal block selected: the gradient is that of dense causal GQA
    attention, taken by torch autograd in float64 (a library routine)."""
    p = problem(B=1, Sq=19, Skv=23, q_start=4, Hq=6, Hkv=2, D=16, Hi=2, bs=4, k=8)
    rng = np.random.default_rng(22)
    q = rng.standard_normal((p.batch, p.seq_q, p.n_q_heads, p.head_dim))
    k = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    v = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    g = rng.standard_normal(q.shape)
    sel = np.full((p.batch, p.seq_q, p.n_kv_heads, p.top_k), -1, np.int32)
    for t in range(p.seq_q):
        cur = (p.q_start + t) // p.block_size
        sel[0, t, :, : cur + 1] = np.arange(cur + 1)
    dq, dk, dv = O.attend_backward(p, q, k, v, g, None, sel, L=L)
    tq = torch.tensor(q[0].transpose(1, 0, 2)).unsqueeze(0).requires_grad_()  # [1,Hq,Sq,D]
    tk = torch.tensor(k).requires_grad_()                                      # [1,Hkv,Skv,D]
    tv = torch.tensor(v).requires_grad_()
    pos = torch.arange(p.seq_q) + p.q_start
    mask = pos[:, None] >= torch.arange(p.seq_kv)[None, :]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=p.softmax_scale,
                                       enable_gqa=True)
    (o * torch.tensor(g[0].transpose(1, 0, 2)).unsqueeze(0)).sum().backward()
    close(dq[0], tq.grad[0].transpose(0, 1).numpy(), 1e-10, "dense dq")
    close(dk, tk.grad.numpy(), 1e-10, "dense dk")
    close(dv, tv.grad.numpy(), 1e-10, "dense dv")


def check_backward_invariants(L):
    """Sparse selections: the softmax weights of a row sum to one, so the
    key gradient summed over all keys of a KV head vanishes and the value
    gradient summed over all keys equals the sum of dout over the rows and
    query heads that read that KV head."""
    p = problem(B=2, Sq=30, Skv=34, q_start=4, Hq=8, Hkv=2, D=16, Hi=2, bs=4, k=3)
    rng = np.random.default_rng(23)
    q = rng.standard_normal((p.batch, p.seq_q, p.n_q_heads, p.head_dim))
    k = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    v = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    g = rng.standard_normal(q.shape)
    sel = _random_selection(p, rng)
    dq, dk, dv = O.attend_backward(p, q, k, v, g, None, sel, L=L)
    G = p.n_q_heads // p.n_kv_heads
    close(dk.sum(axis=2), np.zeros((p.batch, p.n_kv_heads, p.head_dim)), 1e-10, "sum of dk")
    want = g.reshape(p.batch, p.seq_q, p.n_kv_heads, G, p.head_dim).sum(axis=(1, 3))
    close(dv.sum(axis=2), want, 1e-10, "sum of dv")
    # a cotangent of zero gives zero gradients
    z = O.attend_backward(p, q, k, v, np.zeros_like(g), None, sel, L=L)
    for a in z:
        assert not np.any(a), "zero cotangent, nonzero gradient"


# ----------------------------------------------------------------- index KL
def _kl_inputs(p, rng):
    q = rng.standard_normal((p.batch, p.seq_q, p.n_q_heads, p.head_dim))
    k = rng.standard_normal((p.batch, p.n_kv_heads, p.seq_kv, p.head_dim))
    iq = rng.standard_normal((p.batch, p.seq_q, p.n_idx_heads, p.idx_head_dim))
    ik = rng.standard_normal((p.batch, p.seq_kv, p.idx_head_dim))
    return q, k, iq, ik


def check_index_kl_finite_differences(L):
    """Gradients of the summed KL loss against central differences of the
    loss itself, on sampled coordinates of iq and ik (two index heads per KV
    head, a ragged last block, two sequences, random selections)."""
    p = problem(B=2, Sq=11, Skv=13, q_start=2, Hq=4, Hkv=2, D=8, Hi=4, Di=6, bs=4, k=2)
    rng = np.random.default_rng(31)
    q, k, iq, ik = _kl_inputs(p, rng)
    sel = _random_selection(p, rng)
    loss, diq, dik = O.index_kl(p, q, k, iq, ik, None, sel, L=L)
    h = 1e-6
    for name, x, gx in (("iq", iq, diq), ("ik", ik, dik)):
        for _ in range(16):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            x0 = x[idx]
            x[idx] = x0 + h
            lp = O.index_kl(p, q, k, iq, ik, None, sel, L=L)[0].sum()
            x[idx] = x0 - h
            lm = O.index_kl(p, q, k, iq, ik, None, sel, L=L)[0].sum()
            x[idx] = x0
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gx[idx]) <= 1e-6 * (1.0 + abs(fd)), \
                f"d{name}{idx}: analytic {gx[idx]:.9e} vs central difference {fd:.9e}"


def check_index_kl_vs_autograd(L):
    """The loss and both gradients against the definition written with torch
    operations in float64 (masked softmaxes over the attended tokens, the
    group-averaged main-branch distribution as a constant target, KL through
    log_softmax) and differentiated by torch autograd."""
    p = problem(B=1, Sq=14, Skv=18, q_start=4, Hq=6, Hkv=2, D=8, Hi=4, Di=5, bs=4, k=2)
    rng = np.random.default_rng(32)
    q, k, iq, ik = _kl_inputs(p, rng)
    sel = _random_selection(p, rng)
    loss, diq, dik = O.index_kl(p, q, k, iq, ik, None, sel, L=L)
    G = p.n_q_heads // p.n_kv_heads
    tiq = torch.tensor(iq).requires_grad_()
    tik = torch.tensor(ik).requires_grad_()
    total = torch.zeros((), dtype=torch.float64)
    want_loss = np.zeros_like(loss)
    for t in range(p.seq_q):
        pos = p.q_start + t
        for i in range(p.n_idx_heads):
            h = i % p.n_kv_heads
            allowed = torch.zeros(p.seq_kv, dtype=torch.bool)
            for c in sel[0, t, h]:
                if c >= 0:
                    allowed[c * p.block_size: min((c + 1) * p.block_size, pos + 1)] = True
            z = torch.tensor(q[0, t, h * G:(h + 1) * G]) @ torch.tensor(k[0, h]).T  # [G][Skv]
            z = (z * p.softmax_scale).masked_fill(~allowed, float("-inf"))
            P = torch.softmax(z, dim=-1).mean(dim=0)
            s = (tik[0] @ tiq[0, t, i]).masked_fill(~allowed, float("-inf"))
            logq = torch.log_softmax(s, dim=-1)
            m = allowed & (P > 0)
            kl = (P[m] * (torch.log(P[m]) - logq[m])).sum()
            want_loss[0, t, i] = kl.item()
            total = total + kl
    total.backward()
    close(loss, want_loss, 1e-12, "kl loss")
    close(diq, tiq.grad.numpy(), 1e-12, "kl diq")
    close(dik, tik.grad.numpy(), 1e-12, "kl dik")


def check_index_kl_zero_when_distributions_agree(L):
    """When the index scores are exactly the main branch's scaled scores and
    the group's query heads agree, Q == P: the loss and every gradient vanish
    (up to rounding).  Rows at position 0 (one attended token) have Q == P == 1
    whatever the inputs."""
    p = problem(B=1, Sq=12, Skv=12, Hq=4, Hkv=2, D=8, Hi=2, Di=8, bs=4, k=2)
    rng = np.random.default_rng(33)
    G = p.n_q_heads // p.n_kv_heads
    iq = rng.standard_normal((p.batch, p.seq_q, p.n_idx_heads, p.idx_head_dim))
    ik = rng.standard_normal((p.batch, p.seq_kv, p.idx_head_dim))
    q = np.repeat(iq, G, axis=2) / p.softmax_scale  # head hq = h G + g reads index head h
    k = np.repeat(ik[:, None], p.n_kv_heads, axis=1)
    sel = _random_selection(p, rng)
    loss, diq, dik = O.index_kl(p, q, k, iq, ik, None, sel, L=L)
    close(loss, np.zeros_like(loss), 1e-12, "agreeing loss")
    close(diq, np.zeros_like(diq), 1e-10, "agreeing diq")
    close(dik, np.zeros_like(dik), 1e-10, "agreeing dik")
    # position 0: a single attended token
    q2, k2, iq2, ik2 = _kl_inputs(p, rng)
    loss2, diq2, _ = O.index_kl(p, q2, k2, iq2, ik2, None, sel, L=L)
    close(loss2[0, 0], np.zeros(p.n_idx_heads), 1e-14, "single-token loss")
    close(diq2[0, 0], np.zeros((p.n_idx_heads, p.idx_head_dim)), 1e-14, "single-token diq")
    assert np.all(loss2 >= -1e-12) and loss2[0, 5:].max() > 1e-3, "KL must be >= 0 and not all 0"


def check_index_kl_invariants(L):
    """Q - P sums to zero over a row's tokens: the key gradient summed over all
    keys vanishes, and shifting every index key by one vector (every score of a
    row moves by the same amount) leaves the loss unchanged."""
    p = problem(B=2, Sq=20, Skv=25, q_start=5, Hq=8, Hkv=2, D=8, Hi=4, Di=6, bs=4, k=3)
    rng = np.random.default_rng(34)
    q, k, iq, ik = _kl_inputs(p, rng)
    sel = _random_selection(p, rng)
    loss, diq, dik = O.index_kl(p, q, k, iq, ik, None, sel, L=L)
    close(dik.sum(axis=1), np.zeros((p.batch, p.idx_head_dim)), 1e-10, "sum of dik")
    shift = rng.standard_normal(p.idx_head_dim)
    loss_s = O.index_kl(p, q, k, iq, ik + shift, None, sel, L=L)[0]
    close(loss_s, loss, 1e-10, "shifted index keys")


# ----------------------------------------------------------------- token level
def check_token_level_block_size_one(L):
    """Block size 1 (token-level selection, the ablation the pages contrast
    with blocks): a block score is the fp32 rounding of the exact token score
    (max over the attributed index heads), the selection is a plain lexicographic
    sort (score descending, token ascending) cut at k, and attention is library
    attention under the mask of the selected tokens; k >= pos + 1 keeps every
    causal token, i.e. dense attention."""
    S, Hi, Hkv, Di = 23, 4, 2, 6
    p = problem(Sq=S, Skv=S, Hq=4, Hkv=Hkv, D=16, Hi=Hi, Di=Di, bs=1, k=5)
    q, k, v, iq, ik = make(p, 31)
    iqf = [[[Fraction(float(x)) for x in iq[0, t, i]] for i in range(Hi)] for t in range(S)]
    ikf = [[Fraction(float(x)) for x in ik[0, j]] for j in range(S)]
    G = p.n_q_heads // Hkv
    for t in range(S):
        got = O.block_scores_row(p, bits(iq), bits(ik), None, 0, t, L=L)
        sel = np.full((Hkv, p.top_k), -1, np.int32)
        for h in range(Hkv):
            for j in range(S):
                if j < t:
                    exact = max(sum(a * b for a, b in zip(iqf[t][i], ikf[j]))
                                for i in range(Hi) if i % Hkv == h)
                    want = np.float32(float(exact))
                else:
                    want = np.float32(np.inf if j == t else -np.inf)
                assert got[h, j] == want, f"row {t} head {h} token {j}: {got[h, j]} != {want}"
            order = np.lexsort((np.arange(t + 1), -got[h, : t + 1].astype(np.float64)))
            m = min(p.top_k, t + 1)
            want_sel = sorted(order[:m].tolist()) + [-1] * (p.top_k - m)
            got_sel = O.select_row(p, got[h], t, L=L)
            assert got_sel.tolist() == want_sel, f"row {t} head {h}: {got_sel} != {want_sel}"
            sel[h] = got_sel
        allowed = np.zeros((p.n_q_heads, S), bool)
        for hq in range(p.n_q_heads):
            for j in sel[hq // G]:
                if j >= 0:
                    allowed[hq, j] = True
        out, _ = O.attend_row(p, bits(q), bits(k), bits(v), None, sel, 0, t, L=L)
        close(out, sdpa_row(p, q, k, v, 0, t, t, allowed), 1e-12, f"token attend row {t}")
        full = np.tile(np.arange(S, dtype=np.int32), (Hkv, 1))
        full[:, t + 1:] = -1
        pf = problem(Sq=S, Skv=S, Hq=4, Hkv=Hkv, D=16, Hi=Hi, Di=Di, bs=1, k=S)
        out, _ = O.attend_row(pf, bits(q), bits(k), bits(v), None, full, 0, t, L=L)
        close(out, sdpa_row(p, q, k, v, 0, t, t), 1e-12, f"token attend all row {t}")


ALL_CHECKS = [check_dense_vs_library, check_attend_vs_masked_library,
              check_all_blocks_equals_dense, check_softmax_closed_forms,
              check_decode_is_last_prefill_row, check_block_scores_integer_closed_form,
              check_block_scores_rational_brute_force, check_block_scores_causal_and_attribution,
              check_planted_winners_per_kv_head, check_select_brute_force,
              check_select_edge_cases, check_golden_hand_example,
              check_backward_finite_differences, check_backward_dense_vs_autograd,
              check_backward_invariants, check_token_level_block_size_one,
              check_index_kl_finite_differences, check_index_kl_vs_autograd,
              check_index_kl_zero_when_distributions_agree, check_index_kl_invariants]
