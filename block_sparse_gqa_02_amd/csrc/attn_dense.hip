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
// rescaled reference max; P rounded to bf16 for PV.  The V operand of
// O^T += V^T P^T comes from ds_read_b64_tr_b16 (each lane receives one dim of
// four consecutive keys), read three MFMA steps ahead.
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

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
  // V operand: lane (g, n) of the transposed read for M-tile mt, K-step kv and
  // half hf loads dims 16mt + 4(n%4) .. +3 of key 32kv + 16hf + 4g + n/4; with
  // that key's swizzle the byte offset is (32kv + 16hf) * 256 + (vlane ^ 32mt)
  const int r7 = (4 * g + n / 4) & 7;
  const int vlane = (4 * g + n / 4) * 256 + 32 * r7 + 16 * ((n >> 1) & 1) + 8 * (n & 1);

#pragma unroll
  for (int s = 0; s < kRing - 1; ++s)
    if (s < nblk) fetch(s, s);
  for (int c = 0; c < nblk; ++c) {
    const int sl = c % kRing;
    wait_blocks(min(kRing - 2, nblk - 1 - c));
    raw_barrier();  // block c landed for every wave; every wave is done with c-1
    if (c + kRing - 1 < nblk) fetch(c + kRing - 1, (c + kRing - 1) % kRing);
    const char* kt = reinterpret_cast<const char*>(&ktile[sl][0]);
    const uint32_t vt = lds_addr(&vtile[sl][0]);
    // S^T = K Q^T for both groups, one K operand read per pair of MFMAs; K-step
    // outer so consecutive MFMAs use independent accumulators, K fragments read
    // three steps ahead
    f32x4 sc[kNT][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int gq = 0; gq < kNT; ++gq) sc[gq][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kf[4];
#pragma unroll
    for (int st = 0; st < 3; ++st)
      kf[st] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[st / 4] + (st % 4) * 4096));
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int ks = st / 4, mt = st % 4;
      if (st < 13)
        kf[(st + 3) & 3] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[(st + 3) / 4] + ((st + 3) % 4) * 4096));
#pragma unroll
      for (int gq = 0; gq < kNT; ++gq) sc[gq][mt] = mfma16(kf[st & 3], qf[gq][ks], sc[gq][mt]);
    }
    const bool diag = c * kBlock + kBlock - 1 > pos_first;  // some key may follow some row
    const int key0 = c * kBlock + 4 * g;
    bf16x8 pb[kNT][2];
#pragma unroll
    for (int gq = 0; gq < kNT; ++gq) {
      if (diag) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + 16 * mt + r > pos_col[gq]) sc[gq][mt][r] = -__builtin_huge_valf();
      }
      float bm = -__builtin_huge_valf();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        bm = fmax_nn(bm, fmax_nn(fmax_nn(sc[gq][mt][0], sc[gq][mt][1]), fmax_nn(sc[gq][mt][2], sc[gq][mt][3])));
      bm = wave_max_xor16_32(bm) * a.scale_log2;
      const bool grow = bm > mref[gq] + kRescale;
      if (ballot(grow) != 0ull) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(mref[gq] - bm) : 1.f;  // 0 from -inf
#pragma unroll
        for (int x = 0; x < 8; ++x) o[gq][x] *= alpha;
        lsum[gq] *= alpha;
        mref[gq] = grow ? bm : mref[gq];
      }
      // columns past the tile get P = 0 (exp2 of -inf)
      const float msub = pos_col[gq] >= 0 ? mref[gq] : __builtin_huge_valf();
      float ps = 0.f;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sc[gq][2 * kv + e / 4][e % 4], a.scale_log2, -msub));
          ps += p[e];
        }
        u32x4 pw;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) pw[w2] = pack_bf16x2(p[2 * w2], p[2 * w2 + 1]);
        pb[gq][kv] = as_bf16x8(pw);
      }
      lsum[gq] += ps;
    }
    // O^T += V^T P^T, one V operand per pair of MFMAs; k-slot e of K-step kv is
    // key 32kv + 16(e/4) + 4g + e%4, matching the lane's own P registers
    auto vfrag = [&](int kv, int mt) {
      const uint32_t va = vt + (uint32_t)(vlane ^ (32 * mt)) + (32 * kv) * 256;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(uintptr_t)va);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(uintptr_t)(va + 16 * 256));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vf[4];
    vf[0] = vfrag(0, 0);
    vf[1] = vfrag(0, 1);
    vf[2] = vfrag(0, 2);
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kv = st / 8, mt = st % 8;
      if (st < 13) vf[(st + 3) & 3] = vfrag((st + 3) / 8, (st + 3) % 8);
#pragma unroll
      for (int gq = 0; gq < kNT; ++gq) o[gq][mt] = mfma16(vf[st & 3], pb[gq][kv], o[gq][mt]);
    }
  }

#pragma unroll
  for (int gq = 0; gq < kNT; ++gq) {
    const int row = (wave * kNT + gq) * RPG + rr;
    const float L = wave_sum_xor16_32(lsum[gq]);
    if (row < rows) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = a.out + (((size_t)b * a.Sq + t0 + row) * a.Hq + h * G + hh) * kHeadDim;
      // register r of o[gq][mt] is dim 16mt + 4g + r of this lane's column
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        u32x2 w;
        w[0] = pack_bf16x2(o[gq][mt][0] * inv, o[gq][mt][1] * inv);
        w[1] = pack_bf16x2(o[gq][mt][2] * inv, o[gq][mt][3] * inv);
        *reinterpret_cast<u32x2*>(dst + 16 * mt + 4 * g) = w;
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
