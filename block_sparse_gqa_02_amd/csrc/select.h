// select.h — wave-cooperative exact top-m over (key, block index) candidates.
//
// The pages stress that top-k carries internal data dependencies that resist
// parallelisation, and that moving from tokens to blocks cuts the number of
// candidates and the cost of top-k and of merging results (talk analysis
// "How MiniMax M3 Was Built", key_points 3-4; news write-up "MiniMax
// Researcher Olive Song: Sparse Attention Cannot Be Directly Ported Across
// Architectures…", paragraph 6).  Here a selection is a running candidate list
// per (query row, KV head): candidates arrive in ascending block order, only
// those above the current threshold are appended, and when the list fills it
// is compacted to the m best.  Compaction finds the m-th largest key by bitwise
// bisection (each step is one compare and one ballot per register, so the whole
// wave counts 64 candidates per instruction), then keeps, in order, every
// entry above it plus the lowest-indexed entries equal to it.  Lists therefore
// stay sorted by block index, which makes "ties go to the lower block" exact and
// leaves the final list already in ascending order.
//
// Keys are score_key(score) (order-preserving uint32 of the fp32 block score);
// the own block uses 0xffffffff, above every real score.
#pragma once

#include "common.h"

namespace msa {

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Selection core on a wave's registers: entry e * 64 + lane (< n) is
// (kr[e], ir[e]), ascending idx order, n > m >= 1, n <= 64 * MAXE.  Calls
// put(d, key, idx) for the m entries with the largest (key, -idx), d = 0..m-1
// in their original order, and returns the m-th largest key: a later candidate
// (higher idx) can only enter the top m if its key is larger.  Must be called
// by all 64 lanes of a wave with uniform n, m.
template <int MAXE, typename Put>
__device__ __forceinline__ uint32_t wave_topm_regs(const uint32_t (&kr)[MAXE],
                                                   const int32_t (&ir)[MAXE], int n, int m,
                                                   Put&& put) {
  const int lane = lane_id();
  uint32_t mx = 0, mn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    if (e * kWave + lane < n) {
      mx = max(mx, kr[e]);
      mn = min(mn, kr[e]);
    }
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  uint32_t V = mx;
  if (mx != mn) {
    // every candidate shares the bits of mx above the highest differing bit
    const int top = 31 - __builtin_clz(mx ^ mn);
    const uint32_t low = (top == 31) ? 0xffffffffu : ((2u << top) - 1u);
    V = mx & ~low;
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t T = V | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < MAXE; ++e)
        if (e * kWave < n) cnt += __popcll(ballot(e * kWave + lane < n && kr[e] >= T));
      if (cnt >= m) V = T;
    }
  }
  int greater = 0;
#pragma unroll
  for (int e = 0; e < MAXE; ++e)
    if (e * kWave < n) greater += __popcll(ballot(e * kWave + lane < n && kr[e] > V));
  const int take_equal = m - greater;
  __builtin_amdgcn_wave_barrier();
  int out = 0, eq_seen = 0;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    if (e * kWave >= n) break;
    const bool ok = e * kWave + lane < n;
    const bool gt = ok && kr[e] > V;
    const bool eq = ok && kr[e] == V;
    const uint64_t eqm = ballot(eq);
    const bool keep = gt || (eq && eq_seen + prefix_count(eqm) < take_equal);
    const uint64_t km = ballot(keep);
    if (keep) put(out + prefix_count(km), kr[e], ir[e]);
    out += __popcll(km);
    eq_seen += __popcll(eqm);
  }
  __builtin_amdgcn_wave_barrier();
  return V;
}

// Compacts entries [0, n) of (keys, idxs) (any address space, ascending idx
// order, n > m >= 1, n <= 64 * MAXE) in place to the m entries with the
// largest (key, -idx), preserving order; returns the m-th largest key.
template <int MAXE, typename KP, typename IP>
__device__ __forceinline__ uint32_t wave_compact_topm(KP keys, IP idxs, int n, int m) {
  const int lane = lane_id();
  uint32_t kr[MAXE];
  int32_t ir[MAXE];
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = e * kWave + lane;
    const bool ok = i < n;
    kr[e] = ok ? keys[i] : 0u;
    ir[e] = ok ? idxs[i] : 0;
  }
  __builtin_amdgcn_wave_barrier();
  return wave_topm_regs<MAXE>(kr, ir, n, m, [&](int d, uint32_t k, int32_t i) {
    keys[d] = k;
    idxs[d] = i;
  });
}

// Packed candidate: the key in the high word, the block index in the low word.
__device__ __forceinline__ uint64_t pack_cand(uint32_t key, int32_t idx) {
  return ((uint64_t)key << 32) | (uint32_t)idx;
}

// wave_compact_topm over a packed list (pack_cand entries) in global memory.
template <int MAXE>
__device__ __forceinline__ uint32_t wave_compact_topm_packed(uint64_t* ents, int n, int m) {
  const int lane = lane_id();
  uint32_t kr[MAXE];
  int32_t ir[MAXE];
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = e * kWave + lane;
    const uint64_t v = i < n ? ents[i] : 0ull;
    kr[e] = (uint32_t)(v >> 32);
    ir[e] = (int32_t)(uint32_t)v;
  }
  return wave_topm_regs<MAXE>(kr, ir, n, m, [&](int d, uint32_t k, int32_t i) {
    ents[d] = pack_cand(k, i);
  });
}

// Appends this lane's candidate (if `pass`) at the end of a list of length
// cnt, in lane order.  Returns the new length.
template <typename KP, typename IP>
__device__ __forceinline__ int wave_append(KP keys, IP idxs, int cnt, bool pass, uint32_t key,
                                           int32_t idx) {
  const uint64_t mask = ballot(pass);
  if (pass) {
    const int d = cnt + prefix_count(mask);
    keys[d] = key;
    idxs[d] = idx;
  }
  __builtin_amdgcn_wave_barrier();
  return cnt + (int)__popcll(mask);
}

}  // namespace msa
