"""GPU-vs-oracle comparison protocol (shared by the GPU tests, smoke and bench).

Selection: the GPU's list for a (row, KV head) must equal the oracle's, except
in tie-affected rows, where the k-th and (k+1)-th best oracle block scores
differ by less than 1e-5 relative; there any list is accepted whose every kept
block scores at least as high as every dropped block, up to that same 1e-5
relative band (the only freedom near-ties leave).  Always required: the own
block is kept, the count is min(k, cur+1), the list is strictly ascending and
padded with -1.  With integer-valued inputs (exact scores) no mismatch at all
is allowed.

Attention: GPU output against the oracle's exact attention evaluated on the
GPU's own selection: max-abs <= 2e-2 and mean-abs <= 2e-3 over every checked
element.
"""
from __future__ import annotations

import os

import numpy as np

TIE_REL = 1e-5
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def check_selection_row(gpu: np.ndarray, scores: np.ndarray, cur: int, k: int, exact: bool,
                        what: str = "") -> bool:
    """Returns True if the row was an allowed tie mismatch, False if identical.
    Raises AssertionError on a violation."""
    m = min(k, cur + 1)
    g = [int(x) for x in gpu[:m]]
    assert all(int(x) == -1 for x in gpu[m:]), f"{what}: padding {gpu}"
    assert all(0 <= c <= cur for c in g), f"{what}: out of causal range {g} (cur {cur})"
    assert all(a < b for a, b in zip(g, g[1:])), f"{what}: not strictly ascending {g}"
    assert cur in g, f"{what}: own block {cur} missing from {g}"
    cand = np.asarray(scores[: cur + 1], dtype=np.float64).copy()
    cand[cur] = np.inf
    order = sorted(range(cur + 1), key=lambda c: (-cand[c], c))
    want = sorted(order[:m])
    if g == want:
        return False
    assert not exact, f"{what}: selection {g} != oracle {want} (exact inputs)"
    rk, rk1 = cand[order[m - 1]], cand[order[m]]
    tie = abs(rk - rk1) < TIE_REL * max(abs(rk), abs(rk1), 1e-30)
    assert tie, f"{what}: selection {g} != oracle {want}, not a near-tie ({rk} vs {rk1})"
    gs = set(g)
    sel_min = min(cand[c] for c in g)
    unsel_max = max(cand[c] for c in range(cur + 1) if c not in gs)
    tol = TIE_REL * max(abs(sel_min), abs(unsel_max), 1e-30)
    assert sel_min >= unsel_max - tol, \
        f"{what}: tie row but kept {sel_min} < dropped {unsel_max} beyond the band"
    return True


def attention_errors(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()), float(d.mean())


def assert_attention_close(gpu, ref, what=""):
    mx, mean = attention_errors(gpu, ref)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, \
        f"{what}: max-abs {mx:.3e} (<= {MAX_ABS}), mean-abs {mean:.3e} (<= {MEAN_ABS})"
    return mx, mean


def boundary_blocks(seq_q: int, q_start: int, block: int, n_log: int) -> list[int]:
    """At least n_log distinct query blocks (absolute block ids) past the
    first two blocks of the rows, log-spaced over the rest of the range (all
    of them when fewer exist).  Block ids are drawn directly, so rounding
    never collapses two positions into one block."""
    first = q_start // block
    last = (q_start + seq_q - 1) // block
    lo = first + 2
    n_cand = last - lo + 1
    if n_cand <= 0:
        return []
    if n_cand <= n_log:
        return list(range(lo, last + 1))
    n = n_log
    while True:
        xs = np.unique(np.round(np.geomspace(1, n_cand, n)).astype(np.int64))
        if len(xs) >= n_log:
            return [lo + int(x) - 1 for x in xs]
        n += 1


def sample_rows(seq_q: int, q_start: int, block: int, seed: int, n_uniform: int = 2048,
                n_log: int = 32) -> np.ndarray:
    """Stratified row sample: all rows of the first two blocks, the last 64
    rows, both boundary rows (pos % 64 in {0, 63}) of >= n_log distinct
    log-spaced blocks, and n_uniform uniform random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(seq_q, 2 * block - q_start % block)))
    rows |= set(range(max(0, seq_q - 64), seq_q))
    for c in boundary_blocks(seq_q, q_start, block, n_log):
        for t in (c * block - q_start, c * block + block - 1 - q_start):
            if 0 <= t < seq_q:
                rows.add(t)
    rows |= set(rng.choice(seq_q, size=min(n_uniform, seq_q), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
