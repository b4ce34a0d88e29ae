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

// Wave-wide max / min of a uint32, returned as a wave-uniform (scalar) value:
// DPP steps within each 16-lane row (swap neighbours, swap pairs, mirror within
// 8 and within 16 lanes), then v_permlane16_swap and v_permlane32_swap across
// rows.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_uniform(uint32_t v) {
  auto op = [](uint32_t x, uint32_t y) { return MAX ? max(x, y) : min(x, y); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(r[0], r[1]);
  return __builtin_amdgcn_readfirstlane(v);
}

// Selection core on a wave's registers: entry e * 64 + lane (< n) is
// (kr[e], ir[e]), ascending idx order, n > m >= 1, n <= 64 * MAXE; real keys
// are nonzero (score_key of a non-NaN score, or the own block's all-ones key)
// and slots at or beyond n hold key 0.  Calls put(d, key, idx) for the m
// entries with the largest (key, -idx), d = 0..m-1 in their original order,
// and returns the m-th largest key: a later candidate (higher idx) can only
// enter the top m if its key is larger.  Must be called by all 64 lanes of a
// wave with uniform n, m.
template <int MAXE, typename Put>
__device__ __forceinline__ uint32_t wave_topm_regs(const uint32_t (&kr)[MAXE],
                                                   const int32_t (&ir)[MAXE], int n, int m,
                                                   Put&& put) {
  const int lane = lane_id();
  uint32_t mx = 0, mn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    mx = max(mx, kr[e]);
    if (e * kWave + lane < n) mn = min(mn, kr[e]);
  }
  mx = wave_reduce_uniform<true>(mx);
  mn = wave_reduce_uniform<false>(mn);
  uint32_t V = mx;
  if (mx != mn) {
    // every candidate shares the bits of mx above the highest differing bit;
    // the zero padding never reaches a threshold T >= 1
    const int top = 31 - __builtin_clz(mx ^ mn);
    const uint32_t low = (top == 31) ? 0xffffffffu : ((2u << top) - 1u);
    V = mx & ~low;
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t T = V | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < MAXE; ++e) cnt += __popcll(ballot(kr[e] >= T));
      if (cnt >= m) V = T;
    }
  }
  // V is a real key, so the padding is neither above nor equal to it
  int greater = 0;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) greater += __popcll(ballot(kr[e] > V));
  const int take_equal = m - greater;
  __builtin_amdgcn_wave_barrier();
  int out = 0, eq_seen = 0;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    if (e * kWave < n) {  // (a guard, not a break: the loop must unroll fully)
      const bool gt = kr[e] > V;
      const bool eq = kr[e] == V;
      const uint64_t eqm = ballot(eq);
      const bool keep = gt || (eq && eq_seen + prefix_count(eqm) < take_equal);
      const uint64_t km = ballot(keep);
      if (keep) put(out + prefix_count(km), kr[e], ir[e]);
      out += __popcll(km);
      eq_seen += __popcll(eqm);
    }
  }
  __builtin_amdgcn_wave_barrier();
  return V;
}

// The m-th largest of the 128 keys held in (a, b) over the wave (zeros pad),
// or 0 when fewer than m of them are nonzero: the bitwise bisection of
// wave_topm_regs over two registers.  Wave-uniform.  Must be called by all 64
// lanes with uniform m.
__device__ __forceinline__ uint32_t wave_mth_key2(uint32_t a, uint32_t b, int m) {
  const uint32_t mx = wave_reduce_uniform<true>(max(a, b));
  const uint32_t mn = wave_reduce_uniform<false>(min(a, b));
  if (mx == mn) return m <= 2 * kWave && mx != 0 ? mx : 0u;
  const int top = 31 - __builtin_clz(mx ^ mn);
  const uint32_t low = (top == 31) ? 0xffffffffu : ((2u << top) - 1u);
  uint32_t V = mx & ~low;
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t T = V | (1u << bit);
    if (__popcll(ballot(a >= T)) + __popcll(ballot(b >= T)) >= m) V = T;
  }
  return V;
}

// A lower bound on the m-th largest of the 128 keys held in (a, b) over the
// wave (zeros pad), or 0 when fewer than m of them are nonzero: the bisection
// of wave_mth_key2 stopped at bit 16, so the bound has its low 16 bits clear
// and at least m keys reach it.  Half the steps of the exact form; as a
// filter threshold it admits only the keys sharing the m-th largest's top 16
// bits (sign, exponent, 7 mantissa bits) in addition.  Wave-uniform.
__device__ __forceinline__ uint32_t wave_mth_key2_lb(uint32_t a, uint32_t b, int m) {
  const uint32_t mx = wave_reduce_uniform<true>(max(a, b));
  const uint32_t mn = wave_reduce_uniform<false>(min(a, b));
  if (mx == mn) return m <= 2 * kWave && mx != 0 ? mx : 0u;
  const int top = 31 - __builtin_clz(mx ^ mn);
  const uint32_t low = (top == 31) ? 0xffffffffu : ((2u << top) - 1u);
  uint32_t V = mx & ~low;  // every key is >= V
  for (int bit = top; bit >= 16; --bit) {
    const uint32_t T = V | (1u << bit);
    if (__popcll(ballot(a >= T)) + __popcll(ballot(b >= T)) >= m) V = T;
  }
  return __popcll(ballot(a >= V)) + __popcll(ballot(b >= V)) >= m ? V : 0u;
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

constexpr int kStreamBatch = 16;  // 64-candidate chunks loaded together

// Streams block scores [c_beg, c_end) of one row (src[c] is block c's score)
// through a wave's running top-m list in LDS (keys, idxs; cnt entries, the
// threshold thr: only keys above it are taken), with the own block `cur`
// forced to the top key.  Up to kStreamBatch chunks are loaded at once, so a
// row costs one memory latency per batch, not per chunk.  For m <= 64 each
// batch first raises the threshold to just below the m-th largest of its
// lanes' two largest keys: at least m candidates of the batch reach that key,
// so the row's m-th largest does too, and only the candidates at or above it
// can be selected (about 70 of 1024 random scores at m = 64, against about
// 240 past a running threshold).  The list keeps room for a full chunk after
// every compaction (64 MAXE >= m + 64).
template <int MAXE, bool AgentLoads = false>
__device__ __forceinline__ void stream_candidates(const float* src, int c_beg, int c_end, int cur,
                                                  int m, uint32_t* keys, int32_t* idxs, int& cnt,
                                                  uint32_t& thr) {
  constexpr int CAP = MAXE * kWave;
  constexpr int NB = kStreamBatch;  // (a larger batch is no longer unrolled: its registers spill)
  const int lane = lane_id();
  for (int c0 = c_beg; c0 < c_end; c0 += NB * kWave) {
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = c0 + i * kWave + lane;
      if (AgentLoads) {
        // unconditional (clamped) loads: a load under a branch gets its own wait
        const float x = load_agent(src + min(c, c_end - 1));
        v[i] = c < c_end ? x : 0.f;
      } else {
        v[i] = c < c_end ? src[c] : 0.f;
      }
    }
    uint32_t kk[NB];  // keys; 0 past the end
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = c0 + i * kWave + lane;
      kk[i] = c < c_end ? ((c == cur) ? 0xffffffffu : score_key(v[i])) : 0u;
    }
    if (m <= kWave && c_end - c0 >= 2 * m) {
      uint32_t k1 = 0, k2 = 0;  // the lane's two largest keys
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        k2 = max(k2, min(k1, kk[i]));
        k1 = max(k1, kk[i]);
      }
      const uint32_t T = wave_mth_key2_lb(k1, k2, m);
      if (T > thr) thr = T - 1u;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (c0 + i * kWave >= c_end) break;
      const int c = c0 + i * kWave + lane;
      const uint32_t key = kk[i];
      cnt = wave_append(keys, idxs, cnt, key > thr, key, c);
      if (cnt > CAP - kWave) {
        thr = wave_compact_topm<MAXE>(keys, idxs, cnt, m);
        cnt = m;
      }
    }
  }
}

// One row's whole selection into dst[0 .. k): the first min(k, cur+1) blocks
// of [0, cur] by (score descending, block ascending), ascending, -1 padded.
// AgentLoads: the scores were written by other work-groups of the launch.
template <int MAXE, bool AgentLoads = false>
__device__ __forceinline__ void select_row(const float* src, int cur, int k, uint32_t* keys,
                                           int32_t* idxs, int32_t* dst) {
  const int lane = lane_id();
  const int m = min(k, cur + 1);
  int cnt = 0;
  uint32_t thr = 0;
  stream_candidates<MAXE, AgentLoads>(src, 0, cur + 1, cur, m, keys, idxs, cnt, thr);
  // (past the pre-threshold a list usually ends well under 128 entries)
  if (cnt > m) {
    if (MAXE > 2 && cnt <= 2 * kWave) wave_compact_topm<2>(keys, idxs, cnt, m);
    else wave_compact_topm<MAXE>(keys, idxs, cnt, m);
  }
  for (int i = lane; i < k; i += kWave) dst[i] = i < m ? idxs[i] : -1;
  __builtin_amdgcn_wave_barrier();
}

}  // namespace msa
