// attn_dense.hip — dense causal GQA attention, prefill (the full-attention
// baseline every speed-up on the pages is quoted against: news write-up
// "MiniMax Researcher Olive Song: Sparse Attention Cannot Be Directly Ported…",
// paragraph 7; topic page "MiniMax稀疏注意力", summary paragraph).
//
// Flash-style: a work-group of eight waves owns 16/G*16 rows x G heads of one
// KV head; every wave holds NT = 2 MFMA groups (16 columns each) of query
// vectors, so every K/V operand read from LDS feeds two
// v_mfma_f32_16x16x32_bf16.  Causal K/V blocks stream through a 4-slot LDS
// ring by direct global->LDS loads, each wave moving 1/8 of every block, three
// blocks ahead of the compute; all waves use every block, so one barrier per
// block keeps them in step.  Online softmax in the log2 domain with a lazily
// rescaled reference max; P rounded to bf16 for PV.
#include "common.h"
#include "kernels.h"
#include "lds_ring.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;
constexpr int kWaves = 8;
constexpr int kNT = 2;       // MFMA column groups per wave
constexpr int kRing = 4;

struct DenseArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  int Sq, Skv, q_start, Hq, Hkv, ntiles;
  float scale_log2;
};

// s_waitcnt vmcnt(4 * later): each wave issues 4 loads per block
__device__ __forceinline__ void wait_blocks(int later) {
  cbarrier();
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(0xf70 | 0); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xf70 | 4); break;
    default: __builtin_amdgcn_s_waitcnt(0xf70 | 8); break;
  }
  cbarrier();
}

template <int G>
__global__ void __launch_bounds__(kWaves * kWave, 1) dense_prefill_kernel(DenseArgs a) {
  constexpr int RPG = 16 / G;                 // rows per MFMA group
  constexpr int TR = kWaves * kNT * RPG;      // rows per tile
  __shared__ u32x4 ktile[kRing][1024];
  __shared__ u32x4 vtile[kRing][1024];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const int i = (int)(blockIdx.x % a.ntiles);
  const int order = (i / 256 < a.ntiles / 256) ? (i / 256) * 256 + (i % 8) * 32 + (i / 8) % 32 : i;
  const int tile = a.ntiles - 1 - order;  // late (long) tiles first
  const int bh = (int)(blockIdx.x / a.ntiles);
  const int h = bh % a.Hkv, b = bh / a.Hkv;
  const int t0 = tile * TR;
  const int rows = min(TR, a.Sq - t0);
  const int pos_first = a.q_start + t0, pos_last = a.q_start + t0 + rows - 1;
  const int nblk = pos_last / kBlock + 1;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const uint16_t* vh = a.v + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const int rr = n / G, hh = n % G;

  // column group gq of this wave: rows (wave*kNT + gq)*RPG + rr
  bf16x8 qf[kNT][4];
  float mref[kNT], lsum[kNT];
  f32x4 o[kNT][8];
  int pos_col[kNT];
#pragma unroll
  for (int gq = 0; gq < kNT; ++gq) {
    const int row = (wave * kNT + gq) * RPG + rr;
    const bool ok = row < rows;
    pos_col[gq] = ok ? a.q_start + t0 + row : -1;  // -1: masks every key
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.q + (((size_t)b * a.Sq + t0 + (ok ? row : 0)) * a.Hq + h * G + hh) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = src[4 * ks + g];
      qf[gq][ks] = as_bf16x8(v);
    }
    mref[gq] = -__builtin_huge_valf();
    lsum[gq] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[gq][x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto fetch = [&](int c, int sl) {
    const int last = min(pos_last - c * kBlock, kBlock - 1);
    load_block_rows<kswz>(kh + (size_t)c * kBlock * kHeadDim, last, &ktile[sl][0], 2 * wave, 2 * wave + 2);
    load_block_rows<vswz>(vh + (size_t)c * kBlock * kHeadDim, last, &vtile[sl][0], 2 * wave, 2 * wave + 2);
  };

  int kbyte[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kbyte[ks] = n * 256 + (((4 * ks + g) ^ n) << 4);
  const int vbyte0 = 4 * g * 256 + (((n / 2) ^ ((g & 1) << 3)) << 4) + 8 * (n & 1);
  const int vbyte1 = 4 * g * 256 + (((8 + n / 2) ^ ((g & 1) << 3)) << 4) + 8 * (n & 1);

#pragma unroll
  for (int s = 0; s < kRing - 1; ++s)
    if (s < nblk) fetch(s, s);
  for (int c = 0; c < nblk; ++c) {
    const int sl = c % kRing;
    wait_blocks(min(kRing - 2, nblk - 1 - c));
    raw_barrier();  // block c landed for every wave; every wave is done with c-1
    if (c + kRing - 1 < nblk) fetch(c + kRing - 1, (c + kRing - 1) % kRing);
    const char* kt = reinterpret_cast<const char*>(&ktile[sl][0]);
    const char* vt0 = reinterpret_cast<const char*>(&vtile[sl][0]) + vbyte0;
    const char* vt1 = reinterpret_cast<const char*>(&vtile[sl][0]) + vbyte1;
    // S^T = K Q^T for both groups, one K operand read per pair of MFMAs
    f32x4 sc[kNT][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int gq = 0; gq < kNT; ++gq) sc[gq][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[ks] + mt * 4096));
#pragma unroll
        for (int gq = 0; gq < kNT; ++gq) sc[gq][mt] = mfma16(kf, qf[gq][ks], sc[gq][mt]);
      }
    }
    const bool diag = c * kBlock + kBlock - 1 > pos_first;  // some key may follow some row
    const int key0 = c * kBlock + 4 * g;
    bf16x8 pb[kNT][2];
#pragma unroll
    for (int gq = 0; gq < kNT; ++gq) {
      float bmax = -__builtin_huge_valf();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z = sc[gq][mt][r] * a.scale_log2;
          if (diag && key0 + 16 * mt + r > pos_col[gq]) z = -__builtin_huge_valf();
          sc[gq][mt][r] = z;
          bmax = fmaxf(bmax, z);
        }
      bmax = wave_max_xor16_32(bmax);
      const bool grow = bmax > mref[gq] + kRescale;
      if (ballot(grow) != 0ull) {
        const float alpha = grow ? exp2f(mref[gq] - bmax) : 1.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) o[gq][x] *= alpha;
        lsum[gq] *= alpha;
        mref[gq] = grow ? bmax : mref[gq];
      }
      const float mr = mref[gq];
      float ps = 0.f;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = sc[gq][2 * kv + e / 4][e % 4];
          p[e] = z == -__builtin_huge_valf() ? 0.f : exp2f(z - mr);
          ps += p[e];
        }
        u32x4 pw;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) pw[w2] = pack_bf16x2(p[2 * w2], p[2 * w2 + 1]);
        pb[gq][kv] = as_bf16x8(pw);
      }
      lsum[gq] += ps;
    }
    // O^T += V^T P^T, one V operand per pair of MFMAs
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
            const bf16x8 avb = as_bf16x8(av);
#pragma unroll
            for (int gq = 0; gq < kNT; ++gq)
              o[gq][4 * hf + 2 * jp + jj] = mfma16(avb, pb[gq][kv], o[gq][4 * hf + 2 * jp + jj]);
          }
        }
  }

#pragma unroll
  for (int gq = 0; gq < kNT; ++gq) {
    const int row = (wave * kNT + gq) * RPG + rr;
    const float L = wave_sum_xor16_32(lsum[gq]);
    if (row < rows) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = a.out + (((size_t)b * a.Sq + t0 + row) * a.Hq + h * G + hh) * kHeadDim;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w0, w1;
#pragma unroll
        for (int qd = 0; qd < 8; ++qd) {
          const int e0 = 2 * qd, e1 = 2 * qd + 1;
          const uint32_t v = pack_bf16x2(o[gq][4 * hf + (e0 & 3)][e0 >> 2] * inv,
                                         o[gq][4 * hf + (e1 & 3)][e1 >> 2] * inv);
          if (qd < 4) w0[qd] = v; else w1[qd - 4] = v;
        }
        u32x4* d = reinterpret_cast<u32x4*>(dst + 64 * hf + 16 * g);
        d[0] = w0;
        d[1] = w1;
      }
      if (a.lse && g == 0)
        a.lse[((size_t)b * a.Hq + h * G + hh) * a.Sq + t0 + row] =
            L > 0.f ? (mref[gq] + __log2f(L)) * kLn2 : -__builtin_huge_valf();
    }
  }
}

}  // namespace

hipError_t launch_dense_attn_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                     void* out, float* lse, hipStream_t st) {
  if (s.G != 8 && s.G != 4) return launch_dense_attn_prefill_rowwise(s, q, k, v, out, lse, st);
  const int TR = kWaves * kNT * 16 / s.G;
  const int ntiles = ceil_div(s.Sq, TR);
  DenseArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
              static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse,
              s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, ntiles, s.scale * kLog2e};
  const long long grid = (long long)ntiles * s.Hkv * s.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (s.G == 8) dense_prefill_kernel<8><<<(unsigned)grid, kWaves * kWave, 0, st>>>(a);
  else dense_prefill_kernel<4><<<(unsigned)grid, kWaves * kWave, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
