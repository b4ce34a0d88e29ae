// topk.hip — per-KV-head causal top-k over materialised block scores.
//
// Each KV head keeps its own selection; nothing is merged across heads (news
// write-up "MiniMax Researcher Olive Song: Sparse Attention Cannot Be Directly
// Ported Across Architectures…", paragraph 6).  One wave owns one
// (sequence, KV head, query row): it streams the row's causal candidates
// [0, cur] in 64-wide coalesced chunks, appends those above the running
// threshold to a wave-private LDS list, and compacts the list when it fills
// (select.h).  The own block is forced to the top key, so it is always kept.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace msa {
namespace {

struct TopkArgs {
  const float* scores;  // [B][Hkv][Sq][nblk]
  const int32_t* seq_lens;
  int32_t* sel;         // [B][Hkv][Sq][k]
  int Sq, Skv, q_start, Hkv, nblk, k;
  long long nrows;      // B * Hkv * Sq
};

constexpr int kWavesPerWG = 4;
template <int MAXE>
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs a) {
  constexpr int CAP = MAXE * kWave;
  __shared__ uint32_t skeys[kWavesPerWG][CAP];
  __shared__ int32_t sidx[kWavesPerWG][CAP];
  const int wave = threadIdx.x / kWave;
  uint32_t* keys = skeys[wave];
  int32_t* idxs = sidx[wave];
  const long long stride = (long long)gridDim.x * kWavesPerWG;
  for (long long row = (long long)blockIdx.x * kWavesPerWG + wave; row < a.nrows; row += stride) {
    const int t = (int)(row % a.Sq);
    const int b = (int)(row / ((long long)a.Sq * a.Hkv));
    const int pos = a.seq_lens ? min(max(a.seq_lens[b], 1), a.Skv) - 1 : a.q_start + t;
    const int cur = pos / kBlock;
    select_row<MAXE>(a.scores + row * a.nblk, cur, a.k, keys, idxs, a.sel + row * a.k);
  }
}

// Few long rows (decode): one work-group of eight waves per row.  Wave w
// keeps the running list of candidate segment w; wave 0 then streams the eight
// lists, which are ascending and cover ascending ranges, through the same
// compaction.
template <int MAXE>
__global__ void __launch_bounds__(512) topk_wide_kernel(TopkArgs a) {
  constexpr int CAP = MAXE * kWave;
  __shared__ uint32_t skeys[8][CAP];
  __shared__ int32_t sidx[8][CAP];
  __shared__ int32_t scnt[8];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  for (long long row = blockIdx.x; row < a.nrows; row += gridDim.x) {
    const int t = (int)(row % a.Sq);
    const int b = (int)(row / ((long long)a.Sq * a.Hkv));
    const int pos = a.seq_lens ? min(max(a.seq_lens[b], 1), a.Skv) - 1 : a.q_start + t;
    const int cur = pos / kBlock;
    const int m = min(a.k, cur + 1);
    const float* src = a.scores + row * a.nblk;
    // segment of wave w: whole 64-candidate chunks, ascending
    const int nchunk = cur / kWave + 1;
    const int c_beg = (int)((long long)nchunk * wave / 8) * kWave;
    const int c_end = min((int)((long long)nchunk * (wave + 1) / 8) * kWave, cur + 1);
    uint32_t* keys = skeys[wave];
    int32_t* idxs = sidx[wave];
    int cnt = 0;
    uint32_t thr = 0;
    stream_candidates<MAXE>(src, c_beg, c_end, cur, m, keys, idxs, cnt, thr);
    if (cnt > m) {
      wave_compact_topm<MAXE>(keys, idxs, cnt, m);
      cnt = m;
    }
    if (lane == 0) scnt[wave] = cnt;
    __syncthreads();
    if (wave == 0) {
      // merge: stream the other waves' lists after wave 0's own
      cnt = scnt[0];
      thr = 0;
      for (int w = 1; w < 8; ++w) {
        const int nw = scnt[w];
        for (int off = 0; off < nw; off += kWave) {
          const int i = off + lane;
          const bool ok = i < nw;
          const uint32_t key = ok ? skeys[w][i] : 0u;
          const int32_t idx = ok ? sidx[w][i] : 0;
          cnt = wave_append(keys, idxs, cnt, ok && key > thr, key, idx);
          if (cnt > CAP - kWave) {
            thr = wave_compact_topm<MAXE>(keys, idxs, cnt, m);
            cnt = m;
          }
        }
      }
      if (cnt > m) wave_compact_topm<MAXE>(keys, idxs, cnt, m);
      int32_t* dst = a.sel + row * a.k;
      for (int i = lane; i < a.k; i += kWave) dst[i] = i < m ? idxs[i] : -1;
    }
    __syncthreads();
  }
}

// Few long rows, second form: an exact radix select per row.  A work-group of
// 512 threads holds the row's candidate keys in registers (thread t owns
// candidates [E t, E t + E)); four 8-bit passes over an LDS histogram find T,
// the m-th largest key, and how many keys equal to T are taken; two
// block-wide scans then place every key above T and the lowest-indexed keys
// equal to T at their ranks in ascending block order.  Same selection as the
// running-list kernels: score descending, ties to the lower block.
constexpr int kRadixThreads = 512;

// Exclusive prefix sum of v over the work-group (512 threads); total in *sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* sum) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kRadixThreads / kWave; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    total += x;
  }
  __syncthreads();
  *sum = total;
  return before + incl - v;
}

template <int E>
__global__ void __launch_bounds__(kRadixThreads) topk_radix_kernel(TopkArgs a) {
  __shared__ int hist[256];
  __shared__ int wsum[kRadixThreads / kWave];
  __shared__ uint32_t wand[kRadixThreads / kWave], wor[kRadixThreads / kWave];
  __shared__ int pick[2];  // digit, remaining count
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  for (long long row = blockIdx.x; row < a.nrows; row += gridDim.x) {
    const int t = (int)(row % a.Sq);
    const int b = (int)(row / ((long long)a.Sq * a.Hkv));
    const int pos = a.seq_lens ? min(max(a.seq_lens[b], 1), a.Skv) - 1 : a.q_start + t;
    const int cur = pos / kBlock;
    const int n = cur + 1;
    const int m = min(a.k, n);
    const float* src = a.scores + row * a.nblk;
    const int c0 = tid * E;
    // the own block is always kept; the other candidates compete for m - 1 places
    uint32_t key[E];
    uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = c0 + e;
      key[e] = c < cur ? score_key(src[c]) : 0u;  // 0: below every real key
      if (c < cur) {
        kand &= key[e];
        kor |= key[e];
      }
    }
    // Bits shared by every other candidate (block scores share their sign and
    // exponent): the radix passes start below them, so the first digit is not
    // one crowded histogram bin.
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      kand &= (uint32_t)__shfl_xor((int)kand, off);
      kor |= (uint32_t)__shfl_xor((int)kor, off);
    }
    if (lane == 0) {
      wand[wave] = kand;
      wor[wave] = kor;
    }
    __syncthreads();
    kand = 0xffffffffu;
    kor = 0u;
#pragma unroll
    for (int w = 0; w < kRadixThreads / kWave; ++w) {
      kand &= wand[w];
      kor |= wor[w];
    }
    int rem = m - 1;
    const int free_bits = kand == kor ? 0 : 32 - __clz((int)(kand ^ kor));
    uint32_t pmask = free_bits == 32 ? 0u : ~((1u << free_bits) - 1u);
    uint32_t prefix = kand & pmask;
    if (rem == 0) {
      prefix = 0xffffffffu;  // no other block is kept
      pmask = 0xffffffffu;
    }
    // radix select of the rem-th largest other key, most significant free digit first
#pragma unroll 1
    for (int shift = free_bits - 8; rem > 0 && shift > -8; shift -= 8) {
      const int sh = shift < 0 ? 0 : shift;  // the last digit may repeat decided bits
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (c0 + e < cur && (key[e] & pmask) == prefix) atomicAdd(&hist[(key[e] >> sh) & 255], 1);
      __syncthreads();
      if (wave == 0) {
        // lane l holds digits 4l..4l+3; count of matching keys with a higher digit
        int h[4], own = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          h[x] = hist[4 * lane + x];
          own += h[x];
        }
        int suffix = own;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int y = __shfl_down(suffix, off);
          if (lane + off < kWave) suffix += y;
        }
        int above = suffix - own;
#pragma unroll
        for (int x = 3; x >= 0; --x) {
          if (above < rem && above + h[x] >= rem) {
            pick[0] = 4 * lane + x;
            pick[1] = rem - above;
          }
          above += h[x];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)pick[0] << sh;
      pmask |= 0xffu << sh;
      rem = pick[1];
      __syncthreads();
    }
    // prefix is T; take the own block, every other key above T and the first
    // `rem` other keys equal to T
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = c0 + e;
      gt += (c < cur && key[e] > prefix) || c == cur;
      eq += c < cur && key[e] == prefix;
    }
    int ties_total;
    const int tie_rank = block_exclusive_scan(eq, wsum, &ties_total);
    const int take = min(max(rem - tie_rank, 0), eq);
    int selected;
    int at = block_exclusive_scan(gt + take, wsum, &selected);
    int32_t* dst = a.sel + row * a.k;
    int took = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = c0 + e;
      if (c > cur) continue;
      const bool tie = c < cur && key[e] == prefix;
      if (c == cur || (c < cur && key[e] > prefix) || (tie && took < take)) {
        dst[at++] = c;
        took += tie;
      }
    }
    for (int i = m + tid; i < a.k; i += kRadixThreads) dst[i] = -1;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk_blocks(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int32_t* sel, hipStream_t st) {
  TopkArgs a{scores, seq_lens, sel, s.Sq, s.Skv, s.q_start, s.Hkv, s.nblk, s.top_k,
             (long long)s.B * s.Hkv * s.Sq};
  // list capacity >= k + 128 so that a full chunk always fits after a compaction
  if (a.nrows < 2048 && s.nblk >= 1024 && s.nblk <= 32 * kRadixThreads) {
    // few long rows: a work-group per row, radix select
    const int grid = (int)a.nrows;
    if (s.nblk <= 8 * kRadixThreads) topk_radix_kernel<8><<<grid, kRadixThreads, 0, st>>>(a);
    else if (s.nblk <= 16 * kRadixThreads) topk_radix_kernel<16><<<grid, kRadixThreads, 0, st>>>(a);
    else topk_radix_kernel<32><<<grid, kRadixThreads, 0, st>>>(a);
    return hipGetLastError();
  }
  if (a.nrows < 2048 && s.nblk >= 1024) {
    // few longer rows: a work-group per row, eight running lists
    const int grid = (int)a.nrows;
    if (s.top_k <= 64) topk_wide_kernel<3><<<grid, 512, 0, st>>>(a);
    else if (s.top_k <= 128) topk_wide_kernel<4><<<grid, 512, 0, st>>>(a);
    else if (s.top_k <= 192) topk_wide_kernel<5><<<grid, 512, 0, st>>>(a);
    else topk_wide_kernel<6><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
  }
  const long long wgs_needed = (a.nrows + kWavesPerWG - 1) / kWavesPerWG;
  const int grid = (int)std::min<long long>(wgs_needed, 16384);
  // the smallest list that takes a full chunk after a compaction, except that
  // k of 33..64 gets 256 entries (fewer compactions: 1.20 -> 1.13 ms at 128K, k = 64)
  if (s.top_k <= 32) topk_kernel<3><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 128) topk_kernel<4><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 192) topk_kernel<5><<<grid, 256, 0, st>>>(a);
  else topk_kernel<6><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
