// index_scores.hip — index branch of MSA: block scores on gfx950.
//
// The index branch is a lightweight attention of 4 index-query heads against
// one index-key head (talk summary "How MiniMax M3 Was Built: Sparse Attention
// and Native Multimodality", section "MSA uses a lightweight index branch
// before sparse attention"); its scores are reduced to one score per 64-token
// block (section "Block-level retrieval makes sparse attention easier to run
// on GPUs"), the max over the block's tokens and over the index heads
// attributed to a KV head.  The token-level score matrix never leaves
// registers.
//
// Prefill kernel: one work-group per (sequence, 64-row query tile), one wave
// per index head.  The tile's index queries sit in registers as the B operand
// of v_mfma_f32_32x32x16_bf16 for the whole sweep; each 64-key index-K block
// (8 KiB) is staged once in LDS for the four waves; keys are on the M side so
// that the per-block max is a register max plus one cross-half lane swap.  The
// sweep only visits blocks strictly before a row's own block, so no causal mask
// is applied per element.
//
// Decode kernel: one query per sequence; the index-K cache is streamed from
// HBM once, each wave taking a run of blocks, with v_mfma_f32_16x16x32_bf16
// (half-keys on M, half index heads on N, so that loads read whole cache rows).
// In its selecting form (the fused decode index + top-k) the work-groups of a
// sequence count themselves in after writing their block scores, and the last
// one to arrive selects that sequence's blocks, one wave per KV head: top-k
// depends on nothing but its own sequence's scores, so no second launch and
// no wait on another work-group is needed.
#include "common.h"
#include "index_sweep.h"
#include "kernels.h"
#include "select.h"

namespace msa {
namespace {

struct IndexArgs {
  const uint16_t* iq;  // [B][Sq][4][64]
  const uint16_t* ik;  // [B][Skv][64]
  const int32_t* seq_lens;
  float* scores;       // [B][Hkv][Sq][nblk]
  int Sq, Skv, q_start, nblk;
  const int32_t* pages;  // decode with a paged index-K cache: [B][nblk] page ids, else null
  int num_pages;
  int32_t* sel;          // selecting decode form: [B][Hkv][1][k], else null
  int32_t* counters;     // arrivals of a sequence's work-groups (two levels); zero between calls
  int top_k;
};

template <int HKV>
__global__ void __launch_bounds__(256)
index_scores_prefill_kernel(IndexArgs a) {
  __shared__ IndexLds<> lds;
  const int tile = gridDim.x - 1 - blockIdx.x;  // late (long) tiles first
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int t0 = tile * kTileRows;
  const int rows = min(kTileRows, a.Sq - t0);
  const int cur_last = (a.q_start + t0 + rows - 1) / kBlock;  // sweep blocks [0, cur_last)
  const IndexTile T{a.iq, a.ik, b, t0, rows, a.Sq, a.Skv};

  index_sweep(T, 0, cur_last, lds, [&](int c0, int len, u32x4*) {
    // list (h, row): max over index heads i = h (mod HKV); written row-contiguous.
    // thread: blocks 4(tid % 8) .. +3 of the stage, rows tid / 8 + 32r of every
    // head; whole runs of four go out as one 16-byte store
    const int e4 = 4 * (tid % 8), r0 = tid / 8;
    const int c = c0 + e4;
    const bool vec_ok = (a.nblk & 3) == 0;
    if (e4 < len) {
#pragma unroll
      for (int h = 0; h < HKV; ++h) {
#pragma unroll
        for (int rr = 0; rr < kTileRows / 32; ++rr) {
          const int row = r0 + 32 * rr;
          if (row >= rows) continue;
          const int cur = (a.q_start + t0 + row) / kBlock;
          if (c >= cur) continue;
          f32x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float x = lds.stage[h][row][e4 + k];
#pragma unroll
            for (int i = h + HKV; i < kIdxHeads; i += HKV) x = fmax_nn(x, lds.stage[i][row][e4 + k]);
            v[k] = x;
          }
          float* dst = a.scores + (((size_t)b * HKV + h) * a.Sq + t0 + row) * a.nblk + c;
          if (vec_ok && c + 3 < cur && e4 + 3 < len) {
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (c + k < cur && e4 + k < len) dst[k] = v[k];
          }
        }
      }
    }
  });
  // own block: +inf
  for (int list = tid; list < HKV * rows; list += 256) {
    const int h = list / rows, row = list % rows;
    const int cur = (a.q_start + t0 + row) / kBlock;
    a.scores[(((size_t)b * HKV + h) * a.Sq + t0 + row) * a.nblk + cur] = __builtin_huge_valf();
  }
}


constexpr int kDecodeBlocksPerWave = 8;   // block scores only
constexpr int kSelectBlocksPerWave = 8;   // the selecting form
constexpr int kArriveGroup = 16;  // work-groups per first-level arrival counter

// Block scores of blocks [cbeg, cend) of sequence b (one wave, at most BPW
// blocks); Agent: with agent-coherent stores, for another work-group of the
// launch to read.
template <int HKV, bool Agent, int BPW>
__device__ __forceinline__ void decode_block_scores(const IndexArgs& a, int b, int cbeg, int cend,
                                                    float* out) {
  const int lane = threadIdx.x % kWave;

  // One K-step per M-tile, with each 64-dim key split over two operand rows:
  // A-operand row v of M-tile mt is dims 32(v & 1) .. +31 of key 8mt + v/2, so
  // the eight lanes that hold one key read its whole 128-byte row and every
  // load instruction reads one contiguous KiB of the cache.  B-operand column
  // 2i + h holds dims 32h .. 32h+31 of index head i (columns 8..15 are zero);
  // the products of a half-row with the other half's column are never used.
  const int n = lane % 16, g = lane / 16;
  bf16x8 qf;
  {
    u32x4 v = {0, 0, 0, 0};
    if (n < 2 * kIdxHeads)
      v = reinterpret_cast<const u32x4*>(a.iq + ((size_t)b * kIdxHeads + (n >> 1)) * kIdxDim)[4 * (n & 1) + g];
    qf = as_bf16x8(v);
  }
  const u32x4* ikb = reinterpret_cast<const u32x4*>(a.ik + (size_t)b * a.Skv * kIdxDim);
  // index-K block c: contiguous cache, or its page (ids outside the pool read
  // page 0 and score -inf)
  auto block_base = [&](int c) -> const u32x4* {
    if (!a.pages) return ikb + (size_t)c * kBlock * 8;
    const int pg = a.pages[(size_t)b * a.nblk + c];
    const bool ok = pg >= 0 && pg < a.num_pages;
    return reinterpret_cast<const u32x4*>(a.ik) + (size_t)(ok ? pg : 0) * kBlock * 8;
  };
  auto page_ok = [&](int c) {
    if (!a.pages) return true;
    const int pg = a.pages[(size_t)b * a.nblk + c];
    return pg >= 0 && pg < a.num_pages;
  };
  // two blocks per step: 16 independent 16-byte loads in flight per lane.  The
  // cache is read once, so the loads are non-temporal.
  auto load = [&](int c, u32x4 (&kr)[8]) {
    const u32x4* base = block_base(c) + 8 * (n >> 1) + 4 * (n & 1) + g;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) kr[mt] = __builtin_nontemporal_load(base + 64 * mt);
  };
  auto score = [&](int c, const u32x4 (&kr)[8]) -> float {
    // result register r of lane (n, g) is row 4g + r of column n: key
    // 8mt + 2g + r/2, half r & 1.  On an even lane (column 2i, dims 0..31)
    // registers 0 and 2 hold the low halves of keys 8mt + 2g and 8mt + 2g + 1,
    // and the odd neighbour's registers 1 and 3 the matching high halves.
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16(as_bf16x8(kr[mt]), qf, acc);
      const float hi0 = swap_lane_pairs(acc[1]), hi1 = swap_lane_pairs(acc[3]);
      m = fmax_nn(m, fmax_nn(acc[0] + hi0, acc[2] + hi1));
    }
    m = wave_max_xor16_32(m);  // lane 2i: block max of index head i
    if (HKV <= 2) m = fmax_nn(m, __shfl_xor(m, 4));
    if (HKV == 1) m = fmax_nn(m, __shfl_xor(m, 2));
    if (!page_ok(c)) m = -__builtin_huge_valf();
    return m;
  };
  const bool writer = lane < 2 * HKV && (lane & 1) == 0;  // lane 2i: KV head i's score
  float* dst = out + (size_t)(lane >> 1) * a.nblk;
  if (!Agent) {
    for (int c = cbeg; c < cend; c += 2) {
      u32x4 k0[8], k1[8];
      load(c, k0);
      const bool two = c + 1 < cend;
      if (two) load(c + 1, k1);
      const float m0 = score(c, k0);
      if (writer) dst[c] = m0;
      if (two) {
        const float m1 = score(c + 1, k1);
        if (writer) dst[c + 1] = m1;
      }
    }
    return;
  }
  // Agent form: the run's block maxima stay in registers until the run is
  // done, so the write-through stores stay out of the streaming loop's load
  // waits (the loop is unrolled so that every maximum has a fixed register)
  float runmax[BPW];
#pragma unroll
  for (int it = 0; it < BPW / 2; ++it) {
    const int c = cbeg + 2 * it;
    if (c >= cend) break;
    u32x4 k0[8], k1[8];
    load(c, k0);
    const bool two = c + 1 < cend;
    if (two) load(c + 1, k1);
    runmax[2 * it] = score(c, k0);
    runmax[2 * it + 1] = two ? score(c + 1, k1) : 0.f;
  }
  if (writer) {
#pragma unroll
    for (int i = 0; i < BPW; ++i)
      if (cbeg + i < cend) store_agent(dst + cbeg + i, runmax[i]);
  }
}

// MAXE == 0: block scores only; otherwise also the selection, with running
// lists of 64 MAXE entries (>= k + 64).
template <int HKV, int MAXE>
__global__ void __launch_bounds__(256)
index_scores_decode_kernel(IndexArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  // lengths outside [1, Skv] are clamped, so no read leaves the cache
  const int pos = min(max(a.seq_lens[b], 1), a.Skv) - 1;
  const int cur = pos / kBlock;
  // (runs of 8 blocks measured best for the selecting form too: longer runs
  // leave fewer, longer work-groups and a thinly occupied last round)
  constexpr int BPW = MAXE > 0 ? kSelectBlocksPerWave : kDecodeBlocksPerWave;
  const int cbeg = (blockIdx.x * 4 + wave) * BPW;
  const int cend = min(cbeg + BPW, cur);
  float* out = a.scores + (size_t)b * HKV * a.nblk;  // Sq == 1
  if (blockIdx.x == 0 && wave == 0 && lane < HKV) {
    if (MAXE > 0) store_agent(out + (size_t)lane * a.nblk + cur, __builtin_huge_valf());
    else out[(size_t)lane * a.nblk + cur] = __builtin_huge_valf();
  }
  if (cbeg < cend) decode_block_scores<HKV, (MAXE > 0), BPW>(a, b, cbeg, cend, out);
  if constexpr (MAXE > 0) {
    __shared__ uint32_t skeys[4][MAXE * kWave];
    __shared__ int32_t sidx[4][MAXE * kWave];
    __shared__ int is_last;
    // The last work-group of this sequence to finish selects for it.  Arrivals
    // are counted in two levels (groups of kArriveGroup work-groups, then the
    // groups of the sequence) so that no counter takes more than a few dozen
    // near-simultaneous atomics: same-address atomics at device scope
    // serialise.
    const int ngroups = ceil_div((int)gridDim.x, kArriveGroup);
    const int grp = blockIdx.x / kArriveGroup;
    const int in_grp = min(kArriveGroup, (int)gridDim.x - grp * kArriveGroup);
    int32_t* cnt = a.counters + (size_t)b * (1 + ngroups);
    if (!arrive_last(cnt + 1 + grp, in_grp, &is_last)) return;
    if (!arrive_last(cnt, ngroups, &is_last)) return;
    if (wave < HKV)
      select_row<MAXE, true>(out + (size_t)wave * a.nblk, cur, a.top_k, skeys[wave], sidx[wave],
                             a.sel + ((size_t)b * HKV + wave) * a.top_k);
  }
}

}  // namespace

hipError_t launch_index_block_scores(const Shape& s, const void* iq, const void* ik,
                                     const int32_t* seq_lens, float* scores, hipStream_t st,
                                     const Paging* pg) {
  if (pg && !seq_lens) return hipErrorInvalidValue;  // paged caches are decode caches
  IndexArgs a{static_cast<const uint16_t*>(iq), static_cast<const uint16_t*>(ik), seq_lens, scores,
              s.Sq, s.Skv, s.q_start, s.nblk, pg ? pg->table : nullptr, pg ? pg->num_pages : 0,
              nullptr, nullptr, 0};
  const bool dec = seq_lens != nullptr;
  const int per_wg = 4 * kDecodeBlocksPerWave;
  dim3 grid = dec ? dim3(ceil_div(s.nblk, per_wg), s.B) : dim3(ceil_div(s.Sq, kTileRows), s.B);
  switch (s.Hkv) {
    case 1:
      if (dec) index_scores_decode_kernel<1, 0><<<grid, 256, 0, st>>>(a);
      else index_scores_prefill_kernel<1><<<grid, 256, 0, st>>>(a);
      break;
    case 2:
      if (dec) index_scores_decode_kernel<2, 0><<<grid, 256, 0, st>>>(a);
      else index_scores_prefill_kernel<2><<<grid, 256, 0, st>>>(a);
      break;
    case 4:
      if (dec) index_scores_decode_kernel<4, 0><<<grid, 256, 0, st>>>(a);
      else index_scores_prefill_kernel<4><<<grid, 256, 0, st>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Selecting decode: the arrival counters in the fixed counter region (per
// sequence: one for the sequence, one per group of kArriveGroup work-groups),
// then the block scores [B][Hkv][nblk] fp32.
static long long decode_counters_per_seq(const Shape& s) {
  const int wgs = ceil_div(s.nblk, 4 * kSelectBlocksPerWave);
  return 1 + (long long)ceil_div(wgs, kArriveGroup);
}

bool index_topk_decode_counters_fit(const Shape& s) {
  return (long long)s.B * decode_counters_per_seq(s) <= kMaxCounters;
}

size_t index_topk_decode_workspace_bytes(const Shape& s) {
  return kCounterBytes + (size_t)s.B * s.Hkv * s.nblk * sizeof(float);
}

template <int HKV>
static void launch_selecting(const Shape& s, dim3 grid, const IndexArgs& a, hipStream_t st) {
  // running lists of 64 MAXE >= k + 64 entries (room for a full chunk after a
  // compaction); roomier lists for small k compact less often
  if (s.top_k <= 32) index_scores_decode_kernel<HKV, 3><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 128) index_scores_decode_kernel<HKV, 4><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 192) index_scores_decode_kernel<HKV, 5><<<grid, 256, 0, st>>>(a);
  else index_scores_decode_kernel<HKV, 6><<<grid, 256, 0, st>>>(a);
}

hipError_t launch_index_topk_decode(const Shape& s, const void* iq, const void* ik,
                                    const int32_t* seq_lens, int32_t* sel, void* ws,
                                    size_t ws_bytes, hipStream_t st, const Paging* pg) {
  if (!seq_lens || ws_bytes < index_topk_decode_workspace_bytes(s) || s.top_k > kMaxTopK ||
      !index_topk_decode_counters_fit(s))
    return hipErrorInvalidValue;
  IndexArgs a{static_cast<const uint16_t*>(iq), static_cast<const uint16_t*>(ik), seq_lens,
              reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes), 1, s.Skv, 0, s.nblk,
              pg ? pg->table : nullptr, pg ? pg->num_pages : 0, sel, static_cast<int32_t*>(ws),
              s.top_k};
  const dim3 grid(ceil_div(s.nblk, 4 * kSelectBlocksPerWave), s.B);
  switch (s.Hkv) {
    case 1: launch_selecting<1>(s, grid, a, st); break;
    case 2: launch_selecting<2>(s, grid, a, st); break;
    case 4: launch_selecting<4>(s, grid, a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
