// token.hip — token-level selection (block size 1), the alternative the pages
// weigh MSA's blocks against: every KV head keeps its k highest-scoring single
// tokens and attends only to them.  The pages argue that blocks cut the
// number of top-k candidates and so the cost of selecting and merging them
// (news write-up "MiniMax Researcher Olive Song: Sparse Attention Cannot Be
// Directly Ported Across Architectures…", paragraph 6), and that block
// retrieval restores the contiguous reads that per-token gathers lose (talk
// summary "How MiniMax M3 Was Built", section "Block-level retrieval makes
// sparse attention easier to run on GPUs").  These kernels make that
// comparison measurable with the same inputs, the same index arithmetic and
// the same attention arithmetic as the block path.
//
//   token scores  S[b][h][t][j], j < pos: max over the KV head's index heads of
//                 iq . ik_j (bf16 products, fp32 accumulation on
//                 v_mfma_f32_16x16x32_bf16); j == pos: +inf; j > pos: not
//                 written.  One wave owns 16 MFMA columns (16 / nh rows x the
//                 nh index heads of the KV head) and a 4096-token span.
//   top-k         one work-group per (b, h, t): an exact radix select over
//                 the 32-bit order-preserving score keys (digits of 11, 11 and
//                 10 bits, histograms in LDS) finds the k-th key; the keys
//                 above it and the lowest-index ties equal to it are written
//                 in ascending token order by a block-wide ordered scan.  The
//                 own token takes the top key.
//   attention     one wave per (b, h, t) gathers its selected tokens 64 at a
//                 time: K rows into MFMA registers, V rows into the wave's LDS
//                 tile with LDS-bound loads, then the same online-softmax step
//                 as the block kernels (WaveAttn).
#include "attn_block.h"
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTokSpan = 4096;   // tokens per score wave
constexpr int kScoreWaves = 4;   // waves per score work-group
constexpr int kSelThreads = 256; // threads per top-k work-group
constexpr int kSelE = 8;         // candidates per thread per top-k chunk
constexpr int kAttnWaves = 4;    // waves per attention work-group

// ----------------------------------------------------------------- scores
struct ScoreArgs {
  const uint16_t* iq;  // [B][Sq][4][64]
  const uint16_t* ik;  // [B][Skv][64]
  float* out;          // [B][Hkv][Sq][Skv]
  int Sq, Skv, q_start, Hkv, nh, ntiles, nspans;
  int vec;             // every row starts 16-byte aligned
  long long units;     // B * nspans * Hkv * ntiles
};

template <int NH>
__global__ void __launch_bounds__(kScoreWaves * kWave) token_scores_kernel(ScoreArgs a) {
  constexpr int R = 16 / NH;  // rows per wave
  const int lane = threadIdx.x % kWave, n = lane % 16, g = lane / 16;
  const long long u = (long long)blockIdx.x * kScoreWaves + threadIdx.x / kWave;
  if (u >= a.units) return;
  // tiles innermost: neighbouring waves read the same index-key span
  const int tile = (int)(u % a.ntiles);
  long long rest = u / a.ntiles;
  const int h = (int)(rest % a.Hkv);
  rest /= a.Hkv;
  const int span = (int)(rest % a.nspans);
  const int b = (int)(rest / a.nspans);
  const int r0 = tile * R;
  const int pos_last = a.q_start + min(r0 + R, a.Sq) - 1;
  const int j_beg = span * kTokSpan;
  const int j_end = min(j_beg + kTokSpan, pos_last + 1);
  if (j_beg >= j_end) return;

  // column n: row r0 + n / NH, index head h + Hkv * (n % NH)
  const int t = r0 + n / NH;
  const bool row_ok = t < a.Sq;
  const int pos = a.q_start + t;
  const int head = h + a.Hkv * (n % NH);
  bf16x8 qf[2];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.iq + (((size_t)b * a.Sq + (row_ok ? t : 0)) * kIdxHeads + head) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (row_ok) v = src[4 * ks + g];
      qf[ks] = as_bf16x8(v);
    }
  }
  const u32x4* ikb = reinterpret_cast<const u32x4*>(a.ik + (size_t)b * a.Skv * kIdxDim);
  float* dst = a.out + (((size_t)b * a.Hkv + h) * a.Sq + (row_ok ? t : 0)) * a.Skv;
  const bool writer = row_ok && (n % NH) == 0;

  for (int j0 = j_beg; j0 < j_end; j0 += kBlock) {
    // A = 16 tokens x 32 dims per (M-tile, K-step); rows past pos_last are
    // clamped (in range, never written)
    f32x4 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int tok = min(j0 + 16 * mt + n, pos_last);
      const u32x4 k0 = ikb[(size_t)tok * 8 + g];
      const u32x4 k1 = ikb[(size_t)tok * 8 + 4 + g];
      sc[mt] = mfma16(as_bf16x8(k0), qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
      sc[mt] = mfma16(as_bf16x8(k1), qf[1], sc[mt]);
    }
    // max over the KV head's index heads: the NH columns of one row are
    // neighbouring lanes
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[mt][r];
        if (NH >= 2) v = fmaxf(v, __shfl_xor(v, 1));
        if (NH >= 4) v = fmaxf(v, __shfl_xor(v, 2));
        sc[mt][r] = v;
      }
    if (!writer) continue;
    // reg r of M-tile mt is token j0 + 16mt + 4g + r of this lane's row
    if (a.vec && j0 + kBlock - 1 < pos) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<f32x4*>(dst + j0 + 16 * mt + 4 * g) = sc[mt];
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 16 * mt + 4 * g + r;
          if (j < pos) dst[j] = sc[mt][r];
          else if (j == pos) dst[j] = __builtin_huge_valf();
        }
    }
  }
}

// ----------------------------------------------------------------- top-k
struct SelArgs {
  const float* scores;  // [B][Hkv][Sq][Skv]
  int32_t* sel;         // [B][Hkv][Sq][k]
  int Sq, Skv, q_start, k;
};

// Sum of v over the work-group's threads above the caller (higher thread ids)
// and the total; part: LDS scratch of kSelThreads / 64 words.  Contains
// barriers: every thread of the work-group must call it.
__device__ __forceinline__ uint32_t sum_above(uint32_t v, uint32_t* part, uint32_t& total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t s = v;  // inclusive suffix sum over lanes >= lane
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_down(s, d);
    if (lane + d < kWave) s += o;
  }
  if (lane == 0) part[wave] = s;
  __syncthreads();
  uint32_t above = s - v;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / kWave; ++w) {
    total += part[w];
    if (w > wave) above += part[w];
  }
  __syncthreads();
  return above;
}

__global__ void __launch_bounds__(kSelThreads) token_topk_kernel(SelArgs a) {
  constexpr int W = kSelThreads / kWave;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t part[W];
  __shared__ uint32_t cnt_eq[kSelE][W], cnt_take[kSelE][W];
  __shared__ uint32_t found[2];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const long long row = blockIdx.x;  // (b * Hkv + h) * Sq + t
  const int t = (int)(row % a.Sq);
  const int pos = a.q_start + t;
  const int n = pos + 1;
  const float* src = a.scores + (size_t)row * a.Skv;
  int32_t* dst = a.sel + (size_t)row * a.k;
  const int m = min(a.k, n);

  if (m == n) {  // every causal token is kept
    for (int x = tid; x < a.k; x += kSelThreads) dst[x] = x < n ? x : -1;
    return;
  }
  // Keys of one chunk of kSelE * kSelThreads candidates: element e of this
  // thread is token j0 + e * kSelThreads + tid (every load is a contiguous
  // 1 KiB run across the work-group, and the kSelE loads are in flight
  // together).  Tokens past pos read pos's entry and are flagged invalid; the
  // own token takes the top key whatever the score row holds there.
  auto load = [&](int j0, uint32_t (&u)[kSelE]) {
    float f[kSelE];
#pragma unroll
    for (int e = 0; e < kSelE; ++e) f[e] = src[min(j0 + e * kSelThreads + tid, pos)];
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      const int j = j0 + e * kSelThreads + tid;
      u[e] = j == pos ? 0xffffffffu : score_key(f[e]);
    }
  };
  // radix select of the m-th largest key: after the three digits, `prefix`
  // is that key T and `rem` the number of keys equal to T still to take
  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)m;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int x = tid; x < 2048; x += kSelThreads) hist[x] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += kSelE * kSelThreads) {
      uint32_t u[kSelE];
      load(j0, u);
#pragma unroll
      for (int e = 0; e < kSelE; ++e)
        if (j0 + e * kSelThreads + tid < n && (u[e] & pmask) == prefix)
          atomicAdd(&hist[(u[e] >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    const int per = nb / kSelThreads;
    uint32_t local = 0;
    for (int x = 0; x < per; ++x) local += hist[tid * per + x];
    uint32_t total;
    const uint32_t above = sum_above(local, part, total);
    // exactly one thread holds the digit where the count from the top reaches rem
    if (above < rem && rem <= above + local) {
      uint32_t acc = above;
      for (int x = per - 1; x >= 0; --x) {
        const uint32_t c = hist[tid * per + x];
        if (acc + c >= rem) {
          found[0] = (uint32_t)(tid * per + x);
          found[1] = rem - acc;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    prefix |= found[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    rem = found[1];
    __syncthreads();  // found[] and hist[] are rewritten by the next pass
  }
  const uint32_t T = prefix;

  // ascending emission: keys above T, then the first `rem` keys equal to T.
  // Token order within a chunk is (e, wave, lane), so an element's rank is
  // the counts of the earlier sub-chunks, of the lower waves in its own, and
  // of the lower lanes of its wave.
  uint32_t base_eq = 0, base_out = 0;
  for (int j0 = 0; j0 < n; j0 += kSelE * kSelThreads) {
    uint32_t u[kSelE];
    load(j0, u);
    uint64_t eb[kSelE];
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      const bool ok = j0 + e * kSelThreads + tid < n;
      eb[e] = ballot(ok && u[e] == T);
    }
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < kSelE; ++e) cnt_eq[e][wave] = (uint32_t)__popcll(eb[e]);
    }
    __syncthreads();
    uint64_t tb[kSelE];
    uint32_t run = base_eq;
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      uint32_t before = run + (uint32_t)prefix_count(eb[e]);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if (w < wave) before += cnt_eq[e][w];
        run += cnt_eq[e][w];
      }
      const bool ok = j0 + e * kSelThreads + tid < n;
      const bool eq = (eb[e] >> lane) & 1ull;
      tb[e] = ballot((ok && u[e] > T) || (eq && before < rem));
    }
    base_eq = run;
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < kSelE; ++e) cnt_take[e][wave] = (uint32_t)__popcll(tb[e]);
    }
    __syncthreads();
    run = base_out;
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      uint32_t at = run + (uint32_t)prefix_count(tb[e]);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if (w < wave) at += cnt_take[e][w];
        run += cnt_take[e][w];
      }
      // at < m always; the bound keeps a write inside the row regardless
      if (((tb[e] >> lane) & 1ull) && at < (uint32_t)a.k) dst[at] = j0 + e * kSelThreads + tid;
    }
    base_out = run;
  }
  for (int x = m + tid; x < a.k; x += kSelThreads) dst[x] = -1;
}

// ----------------------------------------------------------------- attention
struct TokAttnArgs {
  const uint16_t* q;    // [B][Sq][Hq][128]
  const uint16_t* k;    // [B][Hkv][Skv][128]
  const uint16_t* v;
  const int32_t* sel;   // [B][Hkv][Sq][k] tokens
  uint16_t* out;        // [B][Sq][Hq][128]
  float* lse;           // [B][Hq][Sq] or null
  int Sq, q_start, Skv, Hq, Hkv, G, top_k;
  float scale_log2;
  long long units;      // B * Hkv * Sq
};

__device__ __forceinline__ void wait_all_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xf70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(kAttnWaves * kWave) token_attn_kernel(TokAttnArgs a) {
  __shared__ u32x4 vtile[kAttnWaves][kBlock * 16];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n = lane % 16, g = lane / 16;
  const long long u = (long long)blockIdx.x * kAttnWaves + wave;
  if (u >= a.units) return;
  const int t = (int)(u % a.Sq);
  const int bh = (int)(u / a.Sq);
  const int h = bh % a.Hkv, b = bh / a.Hkv;
  const int pos = a.q_start + t;
  const int hq0 = h * a.G;

  WaveAttn st;
  st.init();
  st.load_q(a.q + (((size_t)b * a.Sq + t) * a.Hq + hq0) * kHeadDim, a.G);
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const uint16_t* vh = a.v + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const int32_t* list = a.sel + u * a.top_k;
  u32x4* tile = vtile[wave];
  // The list is read up to its first entry outside [0, pos] (the -1 padding
  // of a top-k row); slot s of a chunk stands for list entry s0 + s, and the
  // softmax masks slots at or past that end exactly as the block kernels mask
  // keys past the query.
  for (int s0 = 0; s0 < a.top_k; s0 += kBlock) {
    const int e = s0 + lane < a.top_k ? list[s0 + lane] : -1;
    const uint64_t bad = ballot(e < 0 || e > pos);
    const int nv = bad ? __builtin_ctzll(bad) : kBlock;
    if (nv == 0) break;
    const int tok = lane < nv ? e : pos;  // masked slots read the own row
    // V rows of the 64 slots straight into the LDS tile (vtile_slot layout):
    // load i writes slots 64i .. 64i+63, slot = key * 16 + swizzled chunk
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int slot = i * kWave + lane;
      const int key = slot >> 4;
      const int ch = (slot & 15) ^ (((key >> 2) & 1) << 3);
      const int tk = __shfl(tok, key);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(reinterpret_cast<const u32x4*>(vh + (size_t)tk * kHeadDim) + ch),
          (__attribute__((address_space(3))) void*)(tile + i * kWave), 16, 0, 0);
    }
    // K rows of slots 16mt + n, dims 32ks + 8g .. +7 (the S^T A operand)
    u32x4 kr[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int tk = __shfl(tok, 16 * mt + n);
      const u32x4* kb = reinterpret_cast<const u32x4*>(kh + (size_t)tk * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[mt][ks] = kb[4 * ks + g];
    }
    st.attend(kr, s0 / kBlock, s0 + nv - 1, a.scale_log2, tile, [] {}, [] { wait_all_vm(); });
    if (nv < kBlock) break;
  }
  const float L = st.total_l();
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (n < a.G) {
    st.store_bf16(a.out + (((size_t)b * a.Sq + t) * a.Hq + hq0 + n) * kHeadDim, inv);
    if (a.lse && g == 0)
      a.lse[((size_t)b * a.Hq + hq0 + n) * a.Sq + t] =
          L > 0.f ? (st.m + __log2f(L)) * kLn2 : -__builtin_huge_valf();
  }
}

}  // namespace

hipError_t launch_token_scores(const Shape& s, const void* iq, const void* ik, float* scores,
                               hipStream_t st) {
  const int nh = kIdxHeads / s.Hkv;
  const int R = 16 / nh;
  ScoreArgs a{static_cast<const uint16_t*>(iq), static_cast<const uint16_t*>(ik), scores,
              s.Sq, s.Skv, s.q_start, s.Hkv, nh, ceil_div(s.Sq, R),
              ceil_div(s.q_start + s.Sq, kTokSpan),
              (s.Skv % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) ? 1 : 0, 0};
  a.units = (long long)s.B * a.nspans * s.Hkv * a.ntiles;
  const long long grid = (a.units + kScoreWaves - 1) / kScoreWaves;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 blk(kScoreWaves * kWave);
  if (nh == 1) token_scores_kernel<1><<<(unsigned)grid, blk, 0, st>>>(a);
  else if (nh == 2) token_scores_kernel<2><<<(unsigned)grid, blk, 0, st>>>(a);
  else if (nh == 4) token_scores_kernel<4><<<(unsigned)grid, blk, 0, st>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_token_topk(const Shape& s, const float* scores, int32_t* sel, hipStream_t st) {
  const long long rows = (long long)s.B * s.Hkv * s.Sq;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  SelArgs a{scores, sel, s.Sq, s.Skv, s.q_start, s.top_k};
  token_topk_kernel<<<(unsigned)rows, kSelThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_token_attn_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                     const int32_t* sel, void* out, float* lse, hipStream_t st) {
  TokAttnArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse,
                s.Sq, s.q_start, s.Skv, s.Hq, s.Hkv, s.G, s.top_k, s.scale * kLog2e,
                (long long)s.B * s.Hkv * s.Sq};
  const long long grid = (a.units + kAttnWaves - 1) / kAttnWaves;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  token_attn_kernel<<<(unsigned)grid, kAttnWaves * kWave, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
