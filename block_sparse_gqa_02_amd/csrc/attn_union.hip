// attn_union.hip — sparse GQA prefill attention, tile-union schedule.
//
// The main branch attends only to the blocks each KV head selected (topic page
// "MiniMax稀疏注意力", summary paragraph).  With independent selections per
// row, a 64-row tile of one KV head touches nearly every causal block, but any
// one block is wanted by only a few of its rows.  Loading each block once per
// tile and reusing it across the rows that picked it cuts K/V traffic several
// times against one gather per (row, block); the pages make the same point
// about contiguous reads and the compute-to-memory ratio (talk summary "How
// MiniMax M3 Was Built", section "Block-level retrieval makes sparse attention
// easier to run on GPUs").
//
// One work-group of eight waves per (sequence, KV head, tile of 512/G rows).
// Wave w owns 64/G rows as 4 MFMA groups of 16/G rows x G heads (the 16
// columns of v_mfma_f32_16x16x32_bf16); their queries stay in registers and
// their output accumulators stay in (accumulation) registers for the whole
// sweep.  Per window of 512 blocks the tile builds, in LDS, a row bitmask per
// block from the rows' selections, then walks the union in ascending order:
// each block's K and V (32 KiB) are fetched once into a 4-deep LDS
// ring by direct global->LDS loads, several blocks ahead of the compute, and
// every wave runs only the groups that have a row wanting the block.  Rows of
// a group that did not pick the block are masked to -inf.  The softmax max is
// rescaled lazily: the reference max only moves when a block exceeds it by
// more than 2^8, so the accumulators are rarely touched outside the MFMAs.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWin = 512;          // blocks per union window
constexpr float kRescale = 8.0f;   // lazy-rescale threshold (log2 units)
constexpr int kGroups = 3;         // MFMA groups per wave
constexpr int kWaves = 8;          // waves per work-group (2 per SIMD)
constexpr int kStages = 4;         // K/V tiles in flight (LDS ring)

struct UnionArgs {
  const uint16_t* q;    // [B][Sq][Hq][128]
  const uint16_t* k;    // [B][Hkv][Skv][128]
  const uint16_t* v;
  const int32_t* sel;   // [B][Hkv][Sq][k]
  uint16_t* out;        // [B][Sq][Hq][128]
  float* lse;           // [B][Hq][Sq] or null
  int Sq, Skv, q_start, Hq, Hkv, top_k, ntiles;
  float scale_log2;
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// Swizzles (16-byte chunk index within a 256-byte K or V row).
__device__ __forceinline__ int kswz(int row) { return row & 15; }
__device__ __forceinline__ int vswz(int row) { return ((row >> 2) & 1) << 3; }

// s_waitcnt vmcnt(4 * later) with expcnt and lgkmcnt unconstrained: waits
// until at most `later` blocks' worth of this wave's fetches (4 loads each)
// are still in flight.
__device__ __forceinline__ void wait_fetches(int later) {
  asm volatile("" ::: "memory");
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(0xf70 | 0); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xf70 | 4); break;
    default: __builtin_amdgcn_s_waitcnt(0xf70 | 8); break;
  }
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int G>
__global__ void __launch_bounds__(512, 1) union_prefill_kernel(UnionArgs a) {
  constexpr int RPG = 16 / G;           // rows per MFMA group
  constexpr int RW = kGroups * RPG;     // rows per wave
  constexpr int TR = kWaves * RW;       // rows per tile
  // row masks: wave w's rows occupy bits 16(w%2) .. of word w/2
  __shared__ u32x4 ktile[kStages][1024];
  __shared__ u32x4 vtile[kStages][1024];
  __shared__ uint32_t rmask[kWin][kWaves / 2];  // per block: bit per tile row
  __shared__ int32_t ulist[kWin];
  __shared__ int32_t wcount[kWaves];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  // work-groups: (b, h) major, tiles late-first.  Work-group ids are dealt
  // round-robin to the 8 XCDs; within every full run of 256 tiles, XCD x takes
  // 32 adjacent tiles, so the tiles sharing an XCD's L2 also share most of
  // their K/V blocks.
  const int i = (int)(blockIdx.x % a.ntiles);
  const int order = (i / 256 < a.ntiles / 256) ? (i / 256) * 256 + (i % 8) * 32 + (i / 8) % 32 : i;
  const int tile = a.ntiles - 1 - order;
  const int bh = (int)(blockIdx.x / a.ntiles);
  const int h = bh % a.Hkv, b = bh / a.Hkv;
  const int t0 = tile * TR;
  const int rows = min(TR, a.Sq - t0);
  const int cur_last = (a.q_start + t0 + rows - 1) / kBlock;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const uint16_t* vh = a.v + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const int32_t* selh = a.sel + (((size_t)b * a.Hkv + h) * a.Sq + t0) * a.top_k;

  // this lane's column: row-in-group rr, head hh
  const int rr = n / G, hh = n % G;
  const int wrow0 = wave * RW;  // first tile row of this wave

  // queries: group gi, K-step ks -> dims 32ks + 8g .. +7 of (row, head)
  bf16x8 qf[kGroups][4];
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int row = wrow0 + gi * RPG + rr;
    const bool ok = row < rows;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.q + (((size_t)b * a.Sq + t0 + (ok ? row : 0)) * a.Hq + h * G + hh) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = src[4 * ks + g];
      qf[gi][ks] = as_bf16x8(v);
    }
  }
  f32x4 o[kGroups][8];
  float mref[kGroups], lsum[kGroups];
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[gi][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    mref[gi] = -__builtin_huge_valf();
    lsum[gi] = 0.f;
  }

  // direct global->LDS fetch of block c into buffer bf: wave w moves 16-byte
  // chunks 128w .. 128w+127 of K and of V (2 instructions each)
  auto fetch = [&](int c, int bf) {
    const int last = min(a.q_start + t0 + rows - 1 - c * kBlock, kBlock - 1);
    const uint16_t* kb = kh + (size_t)c * kBlock * kHeadDim;
    const uint16_t* vb = vh + (size_t)c * kBlock * kHeadDim;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int slot = (wave * 2 + j) * kWave;  // first LDS slot of this instruction
      const int row = (slot + lane) / 16, ph = lane % 16;
      const int srow = min(row, last);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(kb + srow * kHeadDim + 8 * (ph ^ kswz(row))),
          (lds_ptr)(&ktile[bf][slot]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(vb + srow * kHeadDim + 8 * (ph ^ vswz(row))),
          (lds_ptr)(&vtile[bf][slot]), 16, 0, 0);
    }
  };

  for (int wb = 0; wb <= cur_last; wb += kWin) {
    const int we = min(wb + kWin, cur_last + 1);
    // 1. row bitmasks of the window's blocks
    for (int i = tid; i < kWin * kWaves / 2; i += kWaves * kWave) (&rmask[0][0])[i] = 0u;
    __syncthreads();
    {
      constexpr int parts = kWaves * kWave / TR;
      const int row = tid % TR, part = tid / TR;
      if (row < rows && part < parts) {
        const int cur = (a.q_start + t0 + row) / kBlock;
        const int32_t* lst = selh + (size_t)row * a.top_k;
        for (int i = part; i < a.top_k; i += parts) {
          const int c = lst[i];
          if (c >= wb && c < we && c <= cur)
            atomicOr(&rmask[c - wb][(row / RW) / 2], 1u << (16 * ((row / RW) % 2) + row % RW));
        }
      }
    }
    __syncthreads();
    // 2. union list of the window, ascending
    int nu = 0;
    for (int j = 0; j < kWin; j += kWaves * kWave) {
      const int pidx = j + tid;
      bool nz = false;
      if (pidx < we - wb) {
#pragma unroll
        for (int x = 0; x < kWaves / 2; ++x) nz |= rmask[pidx][x] != 0u;
      }
      const uint64_t bal = ballot(nz);
      if (lane == 0) wcount[wave] = __popcll(bal);
      __syncthreads();
      int before = nu;
      for (int w = 0; w < wave; ++w) before += wcount[w];
      if (nz) ulist[before + prefix_count(bal)] = wb + pidx;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) nu += wcount[w];
      __syncthreads();
    }
    // 3. sweep the union.  Every LDS operand read is a per-lane base plus an
    // immediate: the K swizzle of row 16mt + n is n, the V swizzle of every
    // key a lane reads is (g & 1) << 3.
    const int kbyte[4] = {n * 256 + (((0 + g) ^ n) << 4), n * 256 + (((4 + g) ^ n) << 4),
                          n * 256 + (((8 + g) ^ n) << 4), n * 256 + (((12 + g) ^ n) << 4)};
    const int vbyte0 = 4 * g * 256 + (((n / 2) ^ ((g & 1) << 3)) << 4) + 8 * (n & 1);
    const int vbyte1 = 4 * g * 256 + (((8 + n / 2) ^ ((g & 1) << 3)) << 4) + 8 * (n & 1);
    auto block = [&](int bf, int c) {
      const char* kt = reinterpret_cast<const char*>(&ktile[bf][0]);
      const char* vt0 = reinterpret_cast<const char*>(&vtile[bf][0]) + vbyte0;
      const char* vt1 = reinterpret_cast<const char*>(&vtile[bf][0]) + vbyte1;
      const uint32_t wm = rmask[c - wb][wave / 2] >> (16 * (wave % 2));
      const int key0 = c * kBlock + 4 * g;
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) {
        const uint32_t gm = (wm >> (gi * RPG)) & ((1u << RPG) - 1u);
        if (gm == 0u) continue;
        // S^T = K Q^T
        f32x4 sc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[ks] + mt * 4096));
            sc[mt] = mfma16(kf, qf[gi][ks], sc[mt]);
          }
        }
        const bool active = (gm >> rr) & 1u;
        const int pc = a.q_start + t0 + wrow0 + gi * RPG + rr;  // this column's position
        float bmax = -__builtin_huge_valf();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float z = sc[mt][r] * a.scale_log2;
            if (!active || key0 + 16 * mt + r > pc) z = -__builtin_huge_valf();
            sc[mt][r] = z;
            bmax = fmaxf(bmax, z);
          }
        bmax = wave_max_xor16_32(bmax);
        // lazy rescale: move the reference max only when this block exceeds it by > 2^8
        const bool grow = bmax > mref[gi] + kRescale;
        if (ballot(grow) != 0ull) {
          const float mn = grow ? bmax : mref[gi];
          const float alpha = grow ? exp2f(mref[gi] - mn) : 1.f;  // 0 when mref was -inf
#pragma unroll
          for (int i = 0; i < 8; ++i) o[gi][i] *= alpha;
          lsum[gi] *= alpha;
          mref[gi] = mn;
        }
        const float mr = mref[gi];
        float ps = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float z = sc[2 * kv + i / 4][i % 4];
            p[i] = z == -__builtin_huge_valf() ? 0.f : exp2f(z - mr);
            ps += p[i];
          }
          u32x4 pw;
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) pw[w2] = pack_bf16x2(p[2 * w2], p[2 * w2 + 1]);
          pb[kv] = as_bf16x8(pw);
        }
        lsum[gi] += ps;
        // O^T += V^T P^T; k-slot i of K-step kv is key 32kv + 16(i/4) + 4g + i%4,
        // and a 4-byte read at dims 64hf + 4n + 2jp feeds M-tiles (hf, 2jp), (hf, 2jp+1)
#pragma unroll
        for (int kv = 0; kv < 2; ++kv)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
              uint32_t rd[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const int koffs = (32 * kv + 16 * (i / 4) + (i % 4)) * 256 + 4 * jp;
                rd[i] = *reinterpret_cast<const uint32_t*>((hf ? vt1 : vt0) + koffs);
              }
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                u32x4 av;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                  const uint32_t x = rd[2 * w2], y = rd[2 * w2 + 1];
                  av[w2] = jj ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
                }
                const int j = 2 * jp + jj;
                o[gi][4 * hf + j] = mfma16(as_bf16x8(av), pb[kv], o[gi][4 * hf + j]);
              }
            }
      }
    };
    // ring of kStages tiles: blocks u+1 .. u+kStages-2 are in flight while u
    // is computed; the tile of block u-1 is refilled once every wave is past it
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j)
      if (j < nu) fetch(ulist[j], j);
    for (int u = 0; u < nu; ++u) {
      const int c = ulist[u];
      wait_fetches(min(kStages - 2, nu - 1 - u));
      raw_barrier();
      if (u + kStages - 1 < nu) fetch(ulist[u + kStages - 1], (u + kStages - 1) % kStages);
      block(u % kStages, c);
    }
    raw_barrier();
    __syncthreads();
  }

  // epilogue: normalise and store
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int row = wrow0 + gi * RPG + rr;
    const float L = wave_sum_xor16_32(lsum[gi]);
    if (row < rows) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = a.out + (((size_t)b * a.Sq + t0 + row) * a.Hq + h * G + hh) * kHeadDim;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w0, w1;
#pragma unroll
        for (int qd = 0; qd < 8; ++qd) {
          const int e0 = 2 * qd, e1 = 2 * qd + 1;
          const uint32_t v = pack_bf16x2(o[gi][4 * hf + (e0 & 3)][e0 >> 2] * inv,
                                         o[gi][4 * hf + (e1 & 3)][e1 >> 2] * inv);
          if (qd < 4) w0[qd] = v; else w1[qd - 4] = v;
        }
        u32x4* d = reinterpret_cast<u32x4*>(dst + 64 * hf + 16 * g);
        d[0] = w0;
        d[1] = w1;
      }
      if (a.lse && g == 0)
        a.lse[((size_t)b * a.Hq + h * G + hh) * a.Sq + t0 + row] =
            L > 0.f ? (mref[gi] + __log2f(L)) * kLn2 : -__builtin_huge_valf();
    }
  }
}

}  // namespace

bool union_prefill_supported(const Shape& s) { return s.G == 8 || s.G == 4; }

hipError_t launch_union_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                const int32_t* sel, void* out, float* lse, hipStream_t st) {
  const int TR = kWaves * kGroups * 16 / s.G;
  const int ntiles = ceil_div(s.Sq, TR);
  UnionArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
              static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse,
              s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, s.top_k, ntiles, s.scale * kLog2e};
  const long long grid = (long long)ntiles * s.Hkv * s.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (s.G == 8) union_prefill_kernel<8><<<(unsigned)grid, kWaves * kWave, 0, st>>>(a);
  else if (s.G == 4) union_prefill_kernel<4><<<(unsigned)grid, kWaves * kWave, 0, st>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
