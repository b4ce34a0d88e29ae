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
constexpr int kBatch = 16;  // 64-candidate chunks loaded together

// Streams candidates [c_beg, c_end) of one row through the wave's running
// top-m list (own block `cur` forced to the top key).  Up to kBatch chunks are
// loaded at once, so a row costs one memory latency per batch, not per chunk.
template <int MAXE>
__device__ __forceinline__ void stream_candidates(const float* src, int c_beg, int c_end, int cur,
                                                  int m, uint32_t* keys, int32_t* idxs, int& cnt,
                                                  uint32_t& thr) {
  constexpr int CAP = MAXE * kWave;
  const int lane = lane_id();
  for (int c0 = c_beg; c0 < c_end; c0 += kBatch * kWave) {
    float v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + i * kWave + lane;
      v[i] = c < c_end ? src[c] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (c0 + i * kWave >= c_end) break;
      const int c = c0 + i * kWave + lane;
      const bool ok = c < c_end;
      uint32_t key = 0;
      if (ok) key = (c == cur) ? 0xffffffffu : score_key(v[i]);
      cnt = wave_append(keys, idxs, cnt, ok && key > thr, key, c);
      if (cnt > CAP - kWave) {
        thr = wave_compact_topm<MAXE>(keys, idxs, cnt, m);
        cnt = m;
      }
    }
  }
}

template <int MAXE>
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs a) {
  constexpr int CAP = MAXE * kWave;
  __shared__ uint32_t skeys[kWavesPerWG][CAP];
  __shared__ int32_t sidx[kWavesPerWG][CAP];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  uint32_t* keys = skeys[wave];
  int32_t* idxs = sidx[wave];
  const long long stride = (long long)gridDim.x * kWavesPerWG;
  for (long long row = (long long)blockIdx.x * kWavesPerWG + wave; row < a.nrows; row += stride) {
    const int t = (int)(row % a.Sq);
    const int b = (int)(row / ((long long)a.Sq * a.Hkv));
    const int pos = a.seq_lens ? min(max(a.seq_lens[b], 1), a.Skv) - 1 : a.q_start + t;
    const int cur = pos / kBlock;
    const int m = min(a.k, cur + 1);
    const float* src = a.scores + row * a.nblk;
    int cnt = 0;
    uint32_t thr = 0;
    stream_candidates<MAXE>(src, 0, cur + 1, cur, m, keys, idxs, cnt, thr);
    if (cnt > m) wave_compact_topm<MAXE>(keys, idxs, cnt, m);
    int32_t* dst = a.sel + row * a.k;
    for (int i = lane; i < a.k; i += kWave) dst[i] = i < m ? idxs[i] : -1;
    __builtin_amdgcn_wave_barrier();
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

}  // namespace

hipError_t launch_topk_blocks(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int32_t* sel, hipStream_t st) {
  TopkArgs a{scores, seq_lens, sel, s.Sq, s.Skv, s.q_start, s.Hkv, s.nblk, s.top_k,
             (long long)s.B * s.Hkv * s.Sq};
  // list capacity >= k + 128 so that a full chunk always fits after a compaction
  if (a.nrows < 2048 && s.nblk >= 1024) {
    // few long rows: a work-group per row
    const int grid = (int)a.nrows;
    if (s.top_k <= 64) topk_wide_kernel<3><<<grid, 512, 0, st>>>(a);
    else if (s.top_k <= 128) topk_wide_kernel<4><<<grid, 512, 0, st>>>(a);
    else if (s.top_k <= 192) topk_wide_kernel<5><<<grid, 512, 0, st>>>(a);
    else topk_wide_kernel<6><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
  }
  const long long wgs_needed = (a.nrows + kWavesPerWG - 1) / kWavesPerWG;
  const int grid = (int)std::min<long long>(wgs_needed, 16384);
  if (s.top_k <= 64) topk_kernel<3><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 128) topk_kernel<4><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 192) topk_kernel<5><<<grid, 256, 0, st>>>(a);
  else topk_kernel<6><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
