// attn_union.hip — sparse GQA prefill attention, tile-union schedule.
//
// The main branch attends only to the blocks each KV head selected (topic page
// "MiniMax稀疏注意力", summary paragraph).  With independent selections per
// row, a tile of rows of one KV head touches nearly every causal block, but any
// one block is wanted by only a few of its rows.  Loading each block once per
// tile and reusing it across the rows that picked it cuts K/V traffic several
// times against one gather per (row, block); the pages make the same point
// about contiguous reads and the compute-to-memory ratio (talk summary "How
// MiniMax M3 Was Built", section "Block-level retrieval makes sparse attention
// easier to run on GPUs").
//
// Work-group: eight waves on one (sequence, KV head, tile of 24 row groups); a
// row group is 16/G rows x G query heads, the 16 columns of
// v_mfma_f32_16x16x32_bf16, and wave w owns groups w, w+8, w+16 (queries and
// output accumulators in registers for the whole sweep).  Per window of 512
// blocks the tile builds, in LDS, the row and row-group bitmasks of every block
// from the rows' selections and walks the union of the blocks in ascending
// order; each block's K and V (32 KiB) are fetched once into a ring of LDS
// slots by direct global->LDS loads.
//
// The waves do not meet at a barrier per block: any one block is wanted by a
// few rows only, so per-block work is very uneven across waves, and a barrier
// would make every block cost its busiest wave.  Instead each slot carries a
// ready tag (which union entry it holds) and a done count: a wave spins on the
// tag of the block it needs, runs its own active groups, and counts itself
// done; the last wave done with a slot refills it with the block kRing entries
// ahead and publishes the new tag two blocks before anyone can need it.  Every
// wait is bounded: past the bound the kernel stops waiting and raises a flag
// in the output (a caller-visible failure, never a hang).
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWin = 512;          // blocks per union window
constexpr float kRescale = 8.0f;   // lazy-rescale threshold (log2 units)
constexpr int kWaves = 8;          // waves per work-group (2 per SIMD)
constexpr int kGPW = 3;            // row groups owned per wave
constexpr int kNG = kWaves * kGPW; // row groups per tile
constexpr int kRing = 4;           // K/V slots in the LDS ring
constexpr int kSpinLimit = 1 << 22;

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

// 16-byte chunk swizzles of a 256-byte K or V row.  K: the 16 rows 16mt+n read
// at one chunk hit 16 distinct chunks.  V: the keys a lane group reads share
// bit 2, which picks the half of the row, so the four groups of an 8-byte
// column read hit disjoint bank halves.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
__device__ __forceinline__ int vswz(int row) { return ((row >> 2) & 1) << 3; }

__device__ __forceinline__ void cbarrier() { asm volatile("" ::: "memory"); }

// Ring-tag accesses as plain LDS instructions.  The compiler would otherwise
// put a wait for every outstanding global->LDS load in front of them; the
// kernel orders them against those loads with its own vmcnt waits.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ int lds_load_tag(const int32_t* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ void lds_store_tag(int32_t* p, int v) {
  asm volatile("ds_write_b32 %0, %1" :: "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_fetch_add_tag(int32_t* p, int v) {
  int old;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(old) : "v"(lds_addr(p)), "v"(v) : "memory");
  return old;
}

// s_waitcnt vmcnt(n) for n in {0, 32}, expcnt and lgkmcnt unconstrained
// (vmcnt bits 3:0 and 15:14).
__device__ __forceinline__ void wait_vm(int n) {
  cbarrier();
  if (n == 0) __builtin_amdgcn_s_waitcnt(0xf70);
  else __builtin_amdgcn_s_waitcnt(0xf70 | (2 << 14));  // vmcnt = 32
  cbarrier();
}

template <int G>
__global__ void __launch_bounds__(kWaves * kWave, 1) union_prefill_kernel(UnionArgs a) {
  constexpr int RPG = 16 / G;               // rows per group
  constexpr int TR = kNG * RPG;             // rows per tile
  constexpr int NWR = (TR + 31) / 32;       // row-mask words per block
  __shared__ u32x4 ktile[kRing][1024];
  __shared__ u32x4 vtile[kRing][1024];
  __shared__ uint32_t rmask[kWin][NWR];     // per block: tile rows that picked it
  __shared__ uint32_t gmask[kWin];          // per block: row groups that picked it
  __shared__ int32_t ulist[kWin];
  __shared__ int32_t wcount[kWaves];
  __shared__ int32_t ready[kRing];          // union entry held by each slot
  __shared__ int32_t done[kRing];           // waves finished with the slot's entry
  __shared__ int32_t failed;

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  // work-groups: (b, h) major, tiles late-first; within every full run of 256
  // tiles, XCD x (ids are dealt round-robin to the 8 XCDs) takes 32 adjacent
  // tiles, which share most of their K/V blocks through that XCD's L2
  const int i = (int)(blockIdx.x % a.ntiles);
  const int order = (i / 256 < a.ntiles / 256) ? (i / 256) * 256 + (i % 8) * 32 + (i / 8) % 32 : i;
  const int tile = a.ntiles - 1 - order;
  const int bh = (int)(blockIdx.x / a.ntiles);
  const int h = bh % a.Hkv, b = bh / a.Hkv;
  const int t0 = tile * TR;
  const int rows = min(TR, a.Sq - t0);
  const int pos_last = a.q_start + t0 + rows - 1;
  const int cur_last = pos_last / kBlock;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const uint16_t* vh = a.v + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const int32_t* selh = a.sel + (((size_t)b * a.Hkv + h) * a.Sq + t0) * a.top_k;
  const int rr = n / G, hh = n % G;  // this lane's column: row in group, head

  // owned groups gi = wave + 8j
  bf16x8 qf[kGPW][4];
  float mref[kGPW], lsum[kGPW];
  f32x4 o[kGPW][8];
#pragma unroll
  for (int j = 0; j < kGPW; ++j) {
    const int row = (wave + kWaves * j) * RPG + rr;
    const bool ok = row < rows;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.q + (((size_t)b * a.Sq + t0 + (ok ? row : 0)) * a.Hq + h * G + hh) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = src[4 * ks + g];
      qf[j][ks] = as_bf16x8(v);
    }
    mref[j] = -__builtin_huge_valf();
    lsum[j] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[j][x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid == 0) failed = 0;

  // direct global->LDS copy of instructions [j0, j1) (64 lanes x 16 B each) of
  // block c into slot sl; instruction j covers rows 4j..4j+3
  auto fetch = [&](int c, int sl, int j0, int j1) {
    const int last = min(pos_last - c * kBlock, kBlock - 1);
    const uint16_t* kb = kh + (size_t)c * kBlock * kHeadDim;
    const uint16_t* vb = vh + (size_t)c * kBlock * kHeadDim;
    for (int j = j0; j < j1; ++j) {
      const int row = 4 * j + lane / 16, ph = lane % 16;
      const int srow = min(row, last);  // rows past every tile row's position are never used
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(kb + srow * kHeadDim + 8 * (ph ^ kswz(row))),
          (lds_ptr)(&ktile[sl][j * kWave]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(vb + srow * kHeadDim + 8 * (ph ^ vswz(row))),
          (lds_ptr)(&vtile[sl][j * kWave]), 16, 0, 0);
    }
  };

  // per-lane LDS byte offsets (plus immediates inside the loops)
  int kbyte[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kbyte[ks] = n * 256 + (((4 * ks + g) ^ n) << 4);
  // V: 8-byte read at key 32kv + 16(i/4) + 4g + i%4, dims 64hf + 4n .. +3
  const int vbyte0 = 4 * g * 256 + (((n / 2) ^ ((g & 1) << 3)) << 4) + 8 * (n & 1);
  const int vbyte1 = 4 * g * 256 + (((8 + n / 2) ^ ((g & 1) << 3)) << 4) + 8 * (n & 1);

  auto compute = [&](int sl, int c, int wb) {
    const char* kt = reinterpret_cast<const char*>(&ktile[sl][0]);
    const char* vt0 = reinterpret_cast<const char*>(&vtile[sl][0]) + vbyte0;
    const char* vt1 = reinterpret_cast<const char*>(&vtile[sl][0]) + vbyte1;
    const uint32_t gm = gmask[c - wb];
    const int key0 = c * kBlock + 4 * g;
#pragma unroll
    for (int j = 0; j < kGPW; ++j) {
      const int gi = wave + kWaves * j;
      if (!((gm >> gi) & 1u)) continue;
      // S^T = K Q^T
      f32x4 sc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[ks] + mt * 4096));
          sc[mt] = mfma16(kf, qf[j][ks], sc[mt]);
        }
      }
      const int row = gi * RPG + rr;
      const bool active = (rmask[c - wb][row / 32] >> (row % 32)) & 1u;
      const int pc = a.q_start + t0 + row;
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
      // lazy rescale: move the reference max only when a block exceeds it by > 2^8
      const bool grow = bmax > mref[j] + kRescale;
      if (ballot(grow) != 0ull) {
        const float alpha = grow ? exp2f(mref[j] - bmax) : 1.f;  // 0 when mref was -inf
#pragma unroll
        for (int x = 0; x < 8; ++x) o[j][x] *= alpha;
        lsum[j] *= alpha;
        mref[j] = grow ? bmax : mref[j];
      }
      const float mr = mref[j];
      float ps = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = sc[2 * kv + e / 4][e % 4];
          p[e] = z == -__builtin_huge_valf() ? 0.f : exp2f(z - mr);
          ps += p[e];
        }
        u32x4 pw;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) pw[w2] = pack_bf16x2(p[2 * w2], p[2 * w2 + 1]);
        pb[kv] = as_bf16x8(pw);
      }
      lsum[j] += ps;
      // O^T += V^T P^T: k-slot e of K-step kv is key 32kv + 16(e/4) + 4g + e%4
      // (the lane's own S^T registers); a 4-byte read at dims 64hf + 4n + 2jp
      // feeds M-tiles (hf, 2jp) and (hf, 2jp+1)
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) {
            uint32_t rd[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int koff = (32 * kv + 16 * (e / 4) + (e % 4)) * 256 + 4 * jp;
              rd[e] = *reinterpret_cast<const uint32_t*>((hf ? vt1 : vt0) + koff);
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              u32x4 av;
#pragma unroll
              for (int w2 = 0; w2 < 4; ++w2) {
                const uint32_t x = rd[2 * w2], y = rd[2 * w2 + 1];
                av[w2] = jj ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
              }
              o[j][4 * hf + 2 * jp + jj] = mfma16(as_bf16x8(av), pb[kv], o[j][4 * hf + 2 * jp + jj]);
            }
          }
    }
  };

  bool ok_run = true;
  for (int wb = 0; wb <= cur_last && ok_run; wb += kWin) {
    const int we = min(wb + kWin, cur_last + 1);
    // 1. row and group bitmasks of the window's blocks
    for (int x = tid; x < kWin * NWR; x += kWaves * kWave) (&rmask[0][0])[x] = 0u;
    for (int x = tid; x < kWin; x += kWaves * kWave) gmask[x] = 0u;
    if (tid < kRing) {
      ready[tid] = -1;
      done[tid] = 0;
    }
    __syncthreads();
    {
      constexpr int parts = kWaves * kWave / TR;
      const int row = tid % TR, part = tid / TR;
      if (row < rows && part < parts) {
        const int cur = (a.q_start + t0 + row) / kBlock;
        const int32_t* lst = selh + (size_t)row * a.top_k;
        for (int x = part; x < a.top_k; x += parts) {
          const int c = lst[x];
          if (c >= wb && c < we && c <= cur) {
            atomicOr(&rmask[c - wb][row / 32], 1u << (row % 32));
            atomicOr(&gmask[c - wb], 1u << (row / RPG));
          }
        }
      }
    }
    __syncthreads();
    // 2. union list of the window, ascending
    int nu = 0;
    for (int j = 0; j < kWin; j += kWaves * kWave) {
      const int pidx = j + tid;
      const bool nz = pidx < we - wb && gmask[pidx] != 0u;
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
    // 3. first kRing entries: every wave moves 2 of the 16 instructions of each
    for (int s = 0; s < kRing && s < nu; ++s) fetch(ulist[s], s, 2 * wave, 2 * wave + 2);
    wait_vm(0);
    __syncthreads();
    if (tid < kRing && tid < nu) ready[tid] = tid;
    __syncthreads();
    // 4. decoupled sweep
    int pend_u[2] = {-1, -1}, pend_n = 0;  // this wave's refills not yet published
    for (int u = 0; u < nu; ++u) {
      const int sl = u % kRing;
      // publish own refills due by u + 2 (entry x is published once u >= x - 2)
      while (pend_n > 0 && pend_u[0] <= u + 2) {
        wait_vm(pend_n > 1 ? 32 : 0);
        // the wait above retired the slot's global->LDS loads (vmcnt), so the
        // data is in LDS before the tag is written
        if (lane == 0) lds_store_tag(&ready[pend_u[0] % kRing], pend_u[0]);
        cbarrier();
        pend_u[0] = pend_u[1];
        pend_u[1] = -1;
        --pend_n;
      }
      // wait for entry u
      int spins = 0;
      // a wave's LDS operations complete in order, so once the tag reads u the
      // slot's data reads below see the published block
      while (lds_load_tag(&ready[sl]) != u) {
        if (++spins > kSpinLimit) {
          ok_run = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (!ok_run) {
        if (lane == 0) failed = 1;
        break;
      }
      cbarrier();
      compute(sl, ulist[u], wb);
      cbarrier();
      // count this wave done (its slot reads precede the increment in the
      // wave's in-order LDS stream); the last one refills the slot with entry
      // u + kRing
      int prev = 0;
      if (lane == 0) prev = lds_fetch_add_tag(&done[sl], 1);
      prev = __shfl(prev, 0);
      if (prev == kWaves - 1) {
        if (lane == 0) lds_store_tag(&done[sl], 0);
        if (u + kRing < nu) {
          fetch(ulist[u + kRing], sl, 0, 16);
          pend_u[pend_n++] = u + kRing;
        }
      }
    }
    wait_vm(0);
    __syncthreads();
    if (failed) ok_run = false;
  }

  // epilogue: normalise and store this wave's groups
#pragma unroll
  for (int j = 0; j < kGPW; ++j) {
    const int row = (wave + kWaves * j) * RPG + rr;
    const float L = wave_sum_xor16_32(lsum[j]);
    if (row < rows) {
      // a failed sweep (bounded wait exceeded) stores NaN so the caller sees it
      const float inv = !ok_run ? __builtin_nanf("") : (L > 0.f ? 1.f / L : 0.f);
      uint16_t* dst = a.out + (((size_t)b * a.Sq + t0 + row) * a.Hq + h * G + hh) * kHeadDim;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w0, w1;
#pragma unroll
        for (int qd = 0; qd < 8; ++qd) {
          const int e0 = 2 * qd, e1 = 2 * qd + 1;  // element e = 4r + jx of run 64hf + 16g
          const uint32_t v = pack_bf16x2(o[j][4 * hf + (e0 & 3)][e0 >> 2] * inv,
                                         o[j][4 * hf + (e1 & 3)][e1 >> 2] * inv);
          if (qd < 4) w0[qd] = v; else w1[qd - 4] = v;
        }
        u32x4* d = reinterpret_cast<u32x4*>(dst + 64 * hf + 16 * g);
        d[0] = w0;
        d[1] = w1;
      }
      if (a.lse && g == 0)
        a.lse[((size_t)b * a.Hq + h * G + hh) * a.Sq + t0 + row] =
            L > 0.f ? (mref[j] + __log2f(L)) * kLn2 : -__builtin_huge_valf();
    }
  }
}

}  // namespace

bool union_prefill_supported(const Shape& s) { return s.G == 8 || s.G == 4; }

hipError_t launch_union_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                const int32_t* sel, void* out, float* lse, hipStream_t st) {
  const int TR = kNG * 16 / s.G;
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
