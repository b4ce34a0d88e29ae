// fused.hip — index scoring with a streaming per-(row, KV head) top-k: block
// scores never leave the chip.
//
// At a 1M-token context (the window named in the talk summary "How MiniMax M3
// Was Built", section "MiniMax M3 combines agentic coding, long context, and
// native multimodality") a chunk of 8192 rows has 4 x 8192 x 16384 block
// scores, 2 GiB in fp32; here they stream through a running top-k instead.
// Each KV head keeps its own list (news write-up "MiniMax Researcher Olive
// Song: Sparse Attention Cannot Be Directly Ported…", paragraph 6).
//
// Pass 1 (fused_sweep_kernel): one work-group per (64-row tile, key split).
// The index sweep (index_sweep.h) stages 32 blocks of maxima at a time.  Each
// (row, KV head) list lives in the workspace as packed (key, block) words in
// ascending block order; lane `row` of wave h keeps its count and threshold
// in registers.  At each flush the wave takes its 64 lists two at a time, one
// per half-wave: the 32 staged maxima of a list are tested against its
// threshold and the survivors appended contiguously (ballot prefix counts),
// so one store instruction writes a run of one list rather than one entry of
// 64 lists.  A list that could overflow on the next flush is compacted in
// place to the best k-1 by the whole wave (select.h), which also raises its
// threshold.  Splits of the key range fill the GPU when there are few tiles;
// split s of every tile runs on the same XCD (work-group ids are dealt
// round-robin over the 8 XCDs), so that XCD's L2 serves one key range.
// Pass 2 (fused_merge_kernel): one wave per list merges the splits' lists
// (each ascending, ranges ascending) with the same selection, appends the
// own block and writes the ascending selection.
#include "common.h"
#include "index_sweep.h"
#include "kernels.h"
#include "select.h"

namespace msa {
namespace {

struct FusedArgs {
  const uint16_t* iq;
  const uint16_t* ik;
  int32_t* sel;       // [B][Hkv][Sq][k]
  uint64_t* went;     // [S][B*Hkv*Sq][cap] packed candidates (pack_cand)
  int32_t* wcnt;      // [S][B*Hkv*Sq]
  int B, Sq, Skv, q_start, Hkv, nsplit, ntiles, k, cap;
};

constexpr int kFusedMaxE = 8;  // list capacity at most 8 x 64 entries

// Candidate-list capacity: k-1 (the own block is added at the end) plus at
// least 257 more entries.  A split of n blocks streams about k (1 + ln(n / k))
// candidates past its running threshold, so at k = 64..128 and splits of about
// a thousand blocks a list is compacted about once, when it first fills.
__host__ __device__ inline int fused_cap(int k) {
  const int c = 64 * ((k - 1 + 257 + 63) / 64);
  return c < 64 * kFusedMaxE ? c : 64 * kFusedMaxE;
}

template <int HKV, int MAXE>
__global__ void __launch_bounds__(256) fused_sweep_kernel(FusedArgs a) {
  __shared__ IndexLds<> lds;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int s = blockIdx.x % a.nsplit;
  const int tile = a.ntiles - 1 - blockIdx.x / a.nsplit;  // late (long) tiles first
  const int b = blockIdx.y;
  const int t0 = tile * kTileRows;
  const int rows = min(kTileRows, a.Sq - t0);
  const int cur_last = (a.q_start + t0 + rows - 1) / kBlock;
  const int cbeg = (int)((long long)s * cur_last / a.nsplit);
  const int cend = (int)((long long)(s + 1) * cur_last / a.nsplit);
  const int m = a.k - 1;  // candidates kept per list (own block excluded)
  const long long nlist = (long long)a.B * HKV * a.Sq;
  // Wave h < HKV handles the lists of KV head h; lane r holds the count and
  // threshold of row r's list.
  const int h = wave;
  uint64_t* const tile_lists =
      a.went + ((long long)s * nlist + ((long long)b * HKV + h) * a.Sq + t0) * a.cap;
  uint32_t thr = 0;
  int cnt = 0;

  // compacts every list of this wave holding more than `limit` entries
  auto compact_over = [&](int limit) {
    uint64_t over = ballot(lane < rows && cnt > limit);
    if (over == 0ull) return;
    // the entries were stored by other lanes of this wave: make them visible
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    while (over != 0ull) {
      const int l = __builtin_ctzll(over);
      over &= over - 1;
      const int n = __builtin_amdgcn_readlane(cnt, l);
      const uint32_t t = wave_compact_topm_packed<MAXE>(tile_lists + (long long)l * a.cap, n, m);
      if (lane == l) {
        thr = t;
        cnt = m;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  if (m > 0) {
    const int half = lane / 32, e = lane % 32;
    index_sweep(IndexTile{a.iq, a.ik, b, t0, rows, a.Sq, a.Skv}, cbeg, cend, lds,
                [&](int c0, int len, u32x4*) {
      if (wave >= HKV) return;
      const int c = c0 + e;
      // rows 2p (lanes 0-31) and 2p+1 (lanes 32-63); column e of the stage
      for (int p = 0; p < kTileRows / 2; ++p) {
        const int r = 2 * p + half;
        float v = lds.stage[h][r][e];
#pragma unroll
        for (int j = 1; j < kIdxHeads / HKV; ++j) v = fmax_nn(v, lds.stage[h + j * HKV][r][e]);
        const uint32_t key = score_key(v);
        const int cnt0 = __builtin_amdgcn_readlane(cnt, 2 * p);
        const int cnt1 = __builtin_amdgcn_readlane(cnt, 2 * p + 1);
        const uint32_t thr0 = __builtin_amdgcn_readlane(thr, 2 * p);
        const uint32_t thr1 = __builtin_amdgcn_readlane(thr, 2 * p + 1);
        const int cur_r = (a.q_start + t0 + r) / kBlock;
        const bool take = e < len && r < rows && c < cur_r && key > (half ? thr1 : thr0);
        const uint64_t bal = ballot(take);
        const int n0 = __popc((uint32_t)bal), n1 = __popc((uint32_t)(bal >> 32));
        if (take) {
          const int pos = (half ? cnt1 - n0 : cnt0) + prefix_count(bal);
          tile_lists[(long long)r * a.cap + pos] = pack_cand(key, c);
        }
        if (lane == 2 * p) cnt += n0;
        if (lane == 2 * p + 1) cnt += n1;
      }
      // a list takes at most kStageCols entries per flush
      compact_over(a.cap - kStageCols);
    });
  }
  // the list goes to the merge as it stands (up to cap entries, ascending)
  if (wave < HKV && lane < rows)
    a.wcnt[(long long)s * nlist + ((long long)b * HKV + h) * a.Sq + t0 + lane] = cnt;
}

template <int MAXE>
__global__ void __launch_bounds__(256) fused_merge_kernel(FusedArgs a) {
  constexpr int CAP = MAXE * kWave;
  __shared__ uint32_t skeys[4][CAP];
  __shared__ int32_t sidx[4][CAP];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  uint32_t* keys = skeys[wave];
  int32_t* idxs = sidx[wave];
  const long long nlist = (long long)a.B * a.Hkv * a.Sq;
  const int m = a.k - 1;
  for (long long L = (long long)blockIdx.x * 4 + wave; L < nlist; L += (long long)gridDim.x * 4) {
    const int t = (int)(L % a.Sq);
    const int cur = (a.q_start + t) / kBlock;
    int32_t* dst = a.sel + L * a.k;
    if (a.nsplit == 1 && m > 0) {
      // one split: its list (ascending, at most cap = 64 * MAXE entries) is
      // selected straight from registers into the output
      const int n = a.wcnt[L];
      const uint64_t* src = a.went + L * a.cap;
      if (n > m) {
        uint32_t kr[MAXE];
        int32_t ir[MAXE];
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
          const int i = e * kWave + lane;
          const uint64_t v = i < n ? src[i] : 0ull;
          kr[e] = (uint32_t)(v >> 32);
          ir[e] = (int32_t)(uint32_t)v;
        }
        wave_topm_regs<MAXE>(kr, ir, n, m, [&](int d, uint32_t, int32_t i) { dst[d] = i; });
        if (lane == 0) dst[m] = cur;
      } else {
        for (int i = lane; i < a.k; i += kWave)
          dst[i] = i < n ? (int32_t)(uint32_t)src[i] : (i == n ? cur : -1);
      }
      continue;
    }
    int cnt = 0;
    uint32_t thr = 0;
    if (m > 0) {
      for (int s = 0; s < a.nsplit; ++s) {
        const int n = a.wcnt[(long long)s * nlist + L];
        const uint64_t* src = a.went + ((long long)s * nlist + L) * a.cap;
        for (int off = 0; off < n; off += kWave) {
          const int i = off + lane;
          const bool ok = i < n;
          const uint64_t v = ok ? src[i] : 0ull;
          const uint32_t key = (uint32_t)(v >> 32);
          cnt = wave_append(keys, idxs, cnt, ok && key > thr, key, (int32_t)(uint32_t)v);
          if (cnt > CAP - kWave) {
            thr = wave_compact_topm<MAXE>(keys, idxs, cnt, m);
            cnt = m;
          }
        }
      }
      if (cnt > m) {
        wave_compact_topm<MAXE>(keys, idxs, cnt, m);
        cnt = m;
      }
    }
    for (int i = lane; i < a.k; i += kWave) dst[i] = i < cnt ? idxs[i] : (i == cnt ? cur : -1);
    __builtin_amdgcn_wave_barrier();
  }
}

int fused_nsplit(const Shape& s) {
  const int ntiles = ceil_div(s.Sq, kTileRows);
  const int cur_max = (s.q_start + s.Sq - 1) / kBlock;
  int n = ceil_div(1024, s.B * ntiles);
  n = std::min(n, 16);
  n = std::min(n, std::max(1, cur_max / 64));
  return std::max(n, 1);
}

template <int HKV>
hipError_t launch_hkv(const Shape& s, const FusedArgs& a, hipStream_t st) {
  dim3 g1(a.ntiles * a.nsplit, s.B);
  const long long nlist = (long long)s.B * s.Hkv * s.Sq;
  const int g2 = (int)std::min<long long>((nlist + 3) / 4, 16384);
  // cap is a multiple of 64 in [128, 64 * kFusedMaxE]
  switch (a.cap / kWave) {
#define MSA_FUSED_CASE(E)                                 \
  case E:                                                 \
    fused_sweep_kernel<HKV, E><<<g1, 256, 0, st>>>(a);    \
    fused_merge_kernel<E><<<g2, 256, 0, st>>>(a);         \
    break;
    MSA_FUSED_CASE(2)
    MSA_FUSED_CASE(3)
    MSA_FUSED_CASE(4)
    MSA_FUSED_CASE(5)
    MSA_FUSED_CASE(6)
    MSA_FUSED_CASE(7)
    MSA_FUSED_CASE(8)
#undef MSA_FUSED_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t fused_workspace_bytes(const Shape& s) {
  const size_t nlist = (size_t)s.B * s.Hkv * s.Sq;
  const size_t ns = (size_t)fused_nsplit(s);
  return ns * nlist * ((size_t)fused_cap(s.top_k) * 8 + 4) + 256;
}

hipError_t launch_index_topk_fused(const Shape& s, const void* iq, const void* ik, int32_t* sel,
                                   void* ws, hipStream_t st) {
  const int nsplit = fused_nsplit(s);
  const size_t nlist = (size_t)s.B * s.Hkv * s.Sq;
  const int cap = fused_cap(s.top_k);
  uint64_t* went = static_cast<uint64_t*>(ws);
  int32_t* wcnt = reinterpret_cast<int32_t*>(went + (size_t)nsplit * nlist * cap);
  FusedArgs a{static_cast<const uint16_t*>(iq), static_cast<const uint16_t*>(ik), sel, went, wcnt, s.B, s.Sq, s.Skv, s.q_start, s.Hkv, nsplit, ceil_div(s.Sq, kTileRows),
              s.top_k, cap};
  switch (s.Hkv) {
    case 1: return launch_hkv<1>(s, a, st);
    case 2: return launch_hkv<2>(s, a, st);
    case 4: return launch_hkv<4>(s, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
