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
    for (int c0 = 0; c0 <= cur; c0 += kWave) {
      const int c = c0 + lane;
      const bool ok = c <= cur;
      uint32_t key = 0;
      if (ok) key = (c == cur) ? 0xffffffffu : score_key(src[c]);
      cnt = wave_append(keys, idxs, cnt, ok && key > thr, key, c);
      if (cnt > CAP - kWave) {
        thr = wave_compact_topm<MAXE>(keys, idxs, cnt, m);
        cnt = m;
      }
    }
    if (cnt > m) wave_compact_topm<MAXE>(keys, idxs, cnt, m);
    int32_t* dst = a.sel + row * a.k;
    for (int i = lane; i < a.k; i += kWave) dst[i] = i < m ? idxs[i] : -1;
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_topk_blocks(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int32_t* sel, hipStream_t st) {
  TopkArgs a{scores, seq_lens, sel, s.Sq, s.Skv, s.q_start, s.Hkv, s.nblk, s.top_k,
             (long long)s.B * s.Hkv * s.Sq};
  const long long wgs_needed = (a.nrows + kWavesPerWG - 1) / kWavesPerWG;
  const int grid = (int)std::min<long long>(wgs_needed, 16384);
  // list capacity >= k + 128 so that a full chunk always fits after a compaction
  if (s.top_k <= 64) topk_kernel<3><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 128) topk_kernel<4><<<grid, 256, 0, st>>>(a);
  else if (s.top_k <= 192) topk_kernel<5><<<grid, 256, 0, st>>>(a);
  else topk_kernel<6><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
