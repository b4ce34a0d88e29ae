// index_kl.hip — gradient of the index branch's KL training signal.
//
// The talk summary "How MiniMax M3 Was Built: Sparse Attention and Native
// Multimodality" (section "MSA uses a lightweight index branch before sparse
// attention") says the index branch is trained with a KL divergence so that it
// follows the main branch's attention; the pages give no formula.  The reading
// implemented here: for query row t and index head i, whose KV head is
// h = i mod Hkv, over the tokens T that h attends (its selected blocks, keys
// j <= pos),
//   P_j = mean over the G query heads of h of the main branch's softmax weights
//         (a fixed target: the forward's log-sum-exp gives them),
//   Q_j = softmax over T of the raw index dot products s_j = iq_i . ik_j,
//   loss = KL(P || Q) = sum_j P_j (log P_j - log Q_j).
// d loss / d s_j = Q_j - P_j, so diq_i = sum_j (Q_j - P_j) ik_j and
// dik_j = sum over the (t, i) attending j of (Q_j - P_j) iq_i.
//
// Kernels, in launch order:
//   inverse lists  (shared with the main-branch gradient) the ascending rows
//                  that selected each (sequence, KV head, block).
//   kl_row_kernel  a work-group per 16 rows of one (sequence, KV head) walks the
//                  union of the rows' selected blocks, each block's K and index
//                  K fetched once into double-buffered LDS tiles.  A row group
//                  (16 / G rows) owns 16 main-branch columns (row, query head),
//                  each row a segment of G lanes, and 16 index columns laid in
//                  the same segments: lane e < nih of a row's segment is (row,
//                  index head e) (nih = index heads per KV head), lane
//                  nih <= e < 2 nih repeats (row, e - nih).  Per block: S^T =
//                  K Q^T gives P per head, summed over the row's segment (DPP
//                  lane swaps, so every lane of the row holds its P); the index
//                  scores of the columns; an online log-sum-exp of the index
//                  scores; and one product over the block's index-key rows
//                  whose first copy of each column weighs them by e^{s - m}
//                  (U, rescaled as m grows) and whose second by P (V), so that
//                  diq = U / l - V comes out of one sweep.  The loss is
//                  gathered from sum P log P, sum P s and sum P.  Writes loss,
//                  diq and the index log-sum-exp.
//   kl_key_kernel  a work-group per (block, sequence); wave w owns keys
//                  16w..16w+15.  For each KV head the rows that selected the
//                  block come in chunks of 64 / G rows (64 main-branch columns,
//                  staged with the matching index-query columns by LDS-bound
//                  loads, the next chunk's while one is computed): X = Q K^T
//                  gives P per row, the index scores and the saved log-sum-exp
//                  give Q, and dik^T += iq^T (Q - P)^T.  Each key's gradient is
//                  written once (zero for keys no row attends): deterministic,
//                  no atomics.
// Products take bf16 operands (P, e^{s-m} and Q - P rounded to bf16) with fp32
// accumulation; softmax statistics are fp32.
#include "bwd_tiles.h"
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKlTileRows = 16;  // rows per work-group of the row pass
// A block's job list (chunks of rows over every KV head) is cut into up to
// kKeySplits work-groups of at least kKeyMinJobs jobs: a block early in the
// context is a candidate for every later row, so its list runs to several
// times the mean, and one work-group per block would leave a long tail.
constexpr int kKeySplits = 8;
constexpr int kKeyMinJobs = 64;

__device__ __forceinline__ int key_splits(int total) {
  return max(1, min(kKeySplits, total / kKeyMinJobs));
}

struct KlArgs {
  const uint16_t* q;     // [B][Sq][Hq][128]
  const uint16_t* k;     // [B][Hkv][Skv][128]
  const uint16_t* iq;    // [B][Sq][4][64]
  const uint16_t* ik;    // [B][Skv][64]
  const int32_t* sel;    // [B][Hkv][Sq][top_k]
  const float* lse;      // [B][Hq][Sq], natural log
  float* loss;           // [B][Sq][4]
  float* diq;            // [B][Sq][4][64]
  float* dik;            // [B][Skv][64]
  float* lse_idx;        // workspace [B][4][Sq]: index log-sum-exp, log2 domain
  float* dikp;           // workspace [B][nblk][kKeySplits][64][64]: split partials of dik
  const int32_t* base;   // inverse lists: starts per (sequence, KV head, block), then the total
  const int32_t* lists;  // rows
  int B, Sq, Skv, q_start, Hq, Hkv, G, top_k, nblk, nih;
  float scale_log2;
};

// Index-key / index-query tiles: rows of 64 bf16 (8 chunks of 16 bytes), chunk
// c of row r at chunk c ^ (r & 7).
__device__ __forceinline__ int islot(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// acc^T += T^T W^T over the first 32 KV rows of a 128-byte-row tile T (islot
// layout; its rows are the contraction index), W^T in S^T register layout:
// w[mt] register r is tile row 16mt + 4g + r, column n (rounded to bf16 here).
// KV: K-steps of 32 rows.  The T^T operand is read with ds_read_b64_tr_b16:
// lane (g, n) of the read for K-step kv, half hf and M-tile mt loads dims
// 16mt + 4(n%4) .. +3 of row 32kv + 16hf + 4g + n/4 and receives dim 16mt + n
// of rows 32kv + 16hf + 4g + 0..3, so k-slot i is row 32kv + 16(i/4) + 4g + i%4,
// the row of the lane's own W^T register.  acc[mt] register r is dim
// 16mt + 4g + r of column n.
template <int KV>
__device__ __forceinline__ void pv_idx(const f32x4 (&w)[2 * KV], const u32x4* tile,
                                       f32x4 (&acc)[4]) {
  const int lane = lane_id(), n = lane % 16, g = lane / 16;
  const int r15 = 4 * g + n / 4;
  const uint32_t tb = lds_byte_addr(tile) + (uint32_t)(r15 * 128 + 8 * (n & 1));
#pragma unroll
  for (int kv = 0; kv < KV; ++kv) {
    u32x4 pw;
    pw[0] = pack_bf16x2(w[2 * kv][0], w[2 * kv][1]);
    pw[1] = pack_bf16x2(w[2 * kv][2], w[2 * kv][3]);
    pw[2] = pack_bf16x2(w[2 * kv + 1][0], w[2 * kv + 1][1]);
    pw[3] = pack_bf16x2(w[2 * kv + 1][2], w[2 * kv + 1][3]);
    const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t ch = (uint32_t)((2 * mt + ((n >> 1) & 1)) ^ (r15 & 7));
      const uint32_t va = tb + (uint32_t)(32 * kv * 128) + 16 * ch;
      const s16x4 lo = lds_read_tr(va);
      const s16x4 hi = lds_read_tr(va + 16 * 128);
      const bf16x8 tf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[mt] = mfma16(tf, pb, acc[mt]);
    }
  }
}

// Sum over the G-lane segment of each 16-lane row (G = 4, 8, 16), in every
// lane of the segment: DPP swaps of neighbours and of pairs (quads), then
// the half-row mirror (the other quad of 8 lanes) and the row mirror (the
// other 8 of 16).
template <int G>
__device__ __forceinline__ float segment_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (G >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  if (G >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float max16(const f32x4 (&v)[4]) {
  float m = v[0][0];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, v[mt][r]);
  return m;
}

// Row pass.  Work-group (tile, KV head, sequence), 16 / G row groups of 16 / G
// rows, two groups per wave.
template <int G>
__global__ void __launch_bounds__(512) kl_row_kernel(KlArgs a) {
  extern __shared__ u32x4 kl_lds[];
  u32x4* ktiles = kl_lds;                   // [2][1024]: K of the current / next block
  u32x4* itiles = kl_lds + 2 * 1024;        // [2][512]: its index-key rows
  uint32_t* rmask = reinterpret_cast<uint32_t*>(kl_lds + 3 * 1024);  // [cmax + 1]
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int nwaves = blockDim.x / kWave;
  const int n = lane % 16, g = lane / 16;
  const int h = blockIdx.y, b = blockIdx.z;
  constexpr int RPG = 16 / G;
  const int nih = a.nih;
  const int t0 = blockIdx.x * kKlTileRows;
  const int rows = min(kKlTileRows, a.Sq - t0);
  const int cmax = (a.q_start + t0 + rows - 1) / kBlock;
  const long long hb = (long long)b * a.Hkv + h;
  for (int c = tid; c <= cmax; c += blockDim.x) rmask[c] = 0u;
  __syncthreads();
  const int32_t* srow = a.sel + (hb * a.Sq + t0) * a.top_k;
  for (int idx = tid; idx < rows * a.top_k; idx += blockDim.x) {
    const int i = idx / a.top_k;
    const int c = srow[idx];
    if (c >= 0 && c <= (a.q_start + t0 + i) / kBlock) atomicOr(&rmask[c], 1u << i);
  }
  __syncthreads();
  // this lane's main column (row rloc, head n % G) and index column (the same
  // row, index head h + Hkv m) in each of the wave's two groups
  const int e = n % G;
  const bool is_u = e < nih;                        // U copy of the index column
  const int mloc = is_u ? e : e - nih;
  bf16x8 qf[2][4], iqf[2][2];
  float lse2[2];
  int pos[2], rloc[2], ihead[2];
  bool ivalid[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int grp = 2 * wave + j;
    rloc[j] = grp * RPG + n / G;
    const bool ok = rloc[j] < rows;
    const int t = t0 + (ok ? rloc[j] : 0), hq = h * G + e;
    const u32x4* qs = reinterpret_cast<const u32x4*>(a.q + (((long long)b * a.Sq + t) * a.Hq + hq) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 qv = {0, 0, 0, 0};
      if (ok) qv = qs[4 * ks + g];
      qf[j][ks] = as_bf16x8(qv);
    }
    lse2[j] = ok ? a.lse[((long long)b * a.Hq + hq) * a.Sq + t] * kLog2eB : 0.f;
    pos[j] = ok ? a.q_start + t : -1;
    ihead[j] = h + a.Hkv * (mloc < nih ? mloc : 0);
    ivalid[j] = ok && e < 2 * nih;
    const u32x4* is = reinterpret_cast<const u32x4*>(
        a.iq + (((long long)b * a.Sq + t) * kIdxHeads + ihead[j]) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (ivalid[j]) v = is[4 * ks + g];
      iqf[j][ks] = as_bf16x8(v);
    }
  }
  f32x4 acc[2][4];
  float m[2], l[2], A2[2], B2[2], Ps[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[j] = -__builtin_huge_valf();
    l[j] = A2[j] = B2[j] = Ps[j] = 0.f;
  }
  const float invG = 1.f / (float)G;
  // first block >= from with a nonzero mask (cmax + 1 if none); same in every wave
  auto next_block = [&](int from) {
    for (int base = from; base <= cmax; base += kWave) {
      const int c = base + lane;
      const uint64_t bal = ballot(c <= cmax && rmask[c] != 0u);
      if (bal != 0ull) return base + (int)__builtin_ctzll(bal);
    }
    return cmax + 1;
  };
  // LDS-bound loads of block c's K (16 instructions of 4 rows) and index-key
  // rows (8 instructions of 8 rows) into tiles bf; rows past the cache re-read
  // the last row (masked: they lie past every position)
  auto fetch = [&](int c, int bf) {
    const long long koff = (hb * a.Skv + (long long)c * kBlock) * kHeadDim;
    for (int inst = wave; inst < 24; inst += nwaves) {
      const int slot = (inst & 15) * kWave + lane;
      if (inst < 16) {
        const int key = slot >> 4;
        const int ch = (slot & 15) ^ (key & 15);
        const int krow = min(c * kBlock + key, a.Skv - 1);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(a.k + koff + (long long)(krow - c * kBlock) * kHeadDim + 8 * ch),
            (__attribute__((address_space(3))) void*)(ktiles + bf * 1024 + inst * kWave), 16, 0, 0);
      } else {
        const int key = slot >> 3;
        const int ch = (slot & 7) ^ (key & 7);
        const int krow = min(c * kBlock + key, a.Skv - 1);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(a.ik + ((long long)b * a.Skv + krow) * kIdxDim + 8 * ch),
            (__attribute__((address_space(3))) void*)(itiles + bf * 512 + (inst - 16) * kWave), 16, 0, 0);
      }
    }
  };
  int c = next_block(0), bf = 0;
  if (c <= cmax) fetch(c, 0);
  while (c <= cmax) {
    const int cn = next_block(c + 1);
    wait_all_loads();
    __syncthreads();  // block c's tiles complete in every wave
    if (cn <= cmax) fetch(cn, bf ^ 1);
    const uint32_t msk = rmask[c];
    const u32x4* kt = ktiles + bf * 1024;
    const u32x4* it = itiles + bf * 512;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int grp = 2 * wave + j;
      if (((msk >> (grp * RPG)) & ((1u << RPG) - 1u)) == 0u) continue;  // wave-uniform
      const bool wants = (msk >> rloc[j]) & 1u;
      const bool iwants = ivalid[j] && wants;
      f32x4 sv[4], si[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sv[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        si[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sv[mt] = mfma16(as_bf16x8(kt[swz_slot(16 * mt + n, 4 * ks + g)]), qf[j][ks], sv[mt]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          si[mt] = mfma16(as_bf16x8(it[islot(16 * mt + n, 4 * ks + g)]), iqf[j][ks], si[mt]);
      }
      // P of the main column, averaged over the row's G heads (every lane of
      // the row's segment); index scores in the log2 domain, masked
      f32x4 pr[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = c * kBlock + 16 * mt + 4 * g + r;
          const bool att = key <= pos[j];
          const float p = (wants && att) ? exp2f(sv[mt][r] * a.scale_log2 - lse2[j]) : 0.f;
          pr[mt][r] = segment_sum<G>(p) * invG;
          si[mt][r] = (iwants && att) ? si[mt][r] * kLog2eB : -__builtin_huge_valf();
        }
      const float mb = wave_max_xor16_32(max16(si));
      const float mn = fmaxf(m[j], mb);
      const float alpha = (mn == -__builtin_huge_valf()) ? 1.f : exp2f(m[j] - mn);
      m[j] = mn;
      float ls = 0.f, a2 = 0.f, b2 = 0.f, ps = 0.f;
      f32x4 w[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s2 = si[mt][r];
          const bool ok = s2 != -__builtin_huge_valf();
          const float ev = ok ? exp2f(s2 - mn) : 0.f;
          const float p = pr[mt][r];
          ls += ev;
          ps += p;
          if (p > 0.f) {  // p > 0 only at attended keys, where s2 is finite
            a2 += p * __log2f(p);
            b2 += p * s2;
          }
          w[mt][r] = is_u ? ev : p;
        }
      l[j] = l[j] * alpha + ls;
      A2[j] += a2;
      B2[j] += b2;
      Ps[j] += ps;
      if (is_u) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[j][mt] *= alpha;
      }
      pv_idx<2>(w, it, acc[j]);  // U (first copies) and V (second copies)
    }
    __syncthreads();  // tiles bf free for the block after cn
    c = cn;
    bf ^= 1;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float lt = wave_sum_xor16_32(l[j]);
    const float a2 = wave_sum_xor16_32(A2[j]);
    const float b2 = wave_sum_xor16_32(B2[j]);
    const float ps = wave_sum_xor16_32(Ps[j]);
    f32x4 vv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[mt][r] = __shfl(acc[j][mt][r], lane + nih);  // V copy
    if (is_u && ivalid[j]) {
      const int t = t0 + rloc[j];
      const bool any = lt > 0.f;
      const float inv = any ? 1.f / lt : 0.f;
      float* dst = a.diq + (((long long)b * a.Sq + t) * kIdxHeads + ihead[j]) * kIdxDim;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<f32x4*>(dst + 16 * mt + 4 * g) = any ? acc[j][mt] * inv - vv[mt] : f32x4{0.f, 0.f, 0.f, 0.f};
      if (g == 0) {
        const float lse_i = any ? m[j] + __log2f(lt) : -__builtin_huge_valf();
        a.loss[((long long)b * a.Sq + t) * kIdxHeads + ihead[j]] = any ? kLn2 * (a2 - b2 + lse_i * ps) : 0.f;
        a.lse_idx[((long long)b * kIdxHeads + ihead[j]) * a.Sq + t] = lse_i;
      }
    }
  }
}

// Key pass.  Work-group (block, sequence, split), 4 waves; wave w owns keys
// 64c + 16w .. +15.  Split s of a block with n splits takes jobs
// [s total / n, (s+1) total / n); with one split it writes dik itself, with
// more each writes its partial and kl_dik_merge_kernel adds them in split
// order (deterministic).  A chunk is R = 64 / G rows of one KV head's list: main
// columns (row i / G, head i % G), i < 64, and index columns (row i / nih,
// index head h + Hkv (i % nih)), i < R nih <= 32.
template <int G>
__global__ void __launch_bounds__(256) kl_key_kernel(KlArgs a) {
  constexpr int R = 64 / G;
  __shared__ u32x4 qtile[2][kBlock * 16];  // 64 main columns x 128 dims, swz_slot layout
  __shared__ u32x4 iqtile[2][32 * 8];      // 32 index columns x 64 dims, islot layout
  __shared__ float clse[2][64], ilse[2][32];
  __shared__ int cpos[2][64], ipos[2][32];
  __shared__ float ptab[4][16][17];        // per wave: P of chunk row x the wave's keys
  __shared__ int lbeg[4], llen[4], lnch[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const int nih = a.nih, NI = R * nih;
  const int key0 = c * kBlock + 16 * wave;
  const int nkeys = max(0, min(16, a.Skv - key0));
  const int key = key0 + n;
  // every KV head's list for this block, in (head, chunk) order
  if (tid < 4) {
    const bool hv = tid < a.Hkv;
    const long long e = ((long long)b * a.Hkv + (hv ? tid : 0)) * a.nblk + c;
    const int bg = hv ? a.base[e] : 0;
    const int ln = hv ? a.base[e + 1] - bg : 0;
    lbeg[tid] = bg;
    llen[tid] = ln;
    lnch[tid] = (ln + R - 1) / R;
  }
  // index-key operand (N = the wave's keys), zero past the cache
  bf16x8 ikf[2];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.ik + ((long long)b * a.Skv + min(key, a.Skv - 1)) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (n < nkeys) v = src[4 * ks + g];
      ikf[ks] = as_bf16x8(v);
    }
  }
  f32x4 dka[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dka[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const int total = lnch[0] + lnch[1] + lnch[2] + lnch[3];
  // (KV head, chunk) of job j < total
  auto head_of = [&](int j, int& chunk) {
    int h = 0;
    while (h < 3 && j >= lnch[h]) {
      j -= lnch[h];
      ++h;
    }
    chunk = j;
    return h;
  };
  // this thread's four 16-byte slots of a main tile (column colt, stored
  // chunk lane % 16 = dim chunk cht) and one slot of the index tile
  int colt[4], cht[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    colt[t] = 4 * (4 * wave + t) + lane / 16;
    cht[t] = (lane & 15) ^ (colt[t] & 15);
  }
  const int icol = tid / 8, ich = (tid & 7) ^ (icol & 7);
  // the chunk row a metadata thread describes: main column tid, index column tid - 64
  const int mrr = tid < 64 ? tid / G : min((tid - 64) / nih, R - 1);
  // list entry of chunk row rr (rows past the list repeat its first entry;
  // their columns are masked)
  auto row_at = [&](int h, int chunk, int rr) {
    const int e = chunk * R + rr;
    return a.lists[lbeg[h] + (e < llen[h] ? e : 0)];
  };
  int rt[4], rti = 0, rm = 0;  // rows of the next job to stage
  auto fetch_rows = [&](int j) {
    int chunk;
    const int h = head_of(j, chunk);
#pragma unroll
    for (int t = 0; t < 4; ++t) rt[t] = row_at(h, chunk, colt[t] / G);
    rti = row_at(h, chunk, min(icol / nih, R - 1));
    if (tid < 96) rm = row_at(h, chunk, mrr);
  };
  float ml = 0.f;
  int mp = -1;
  auto stage = [&](int j, int buf) {
    int chunk;
    const int h = head_of(j, chunk);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const long long e = (((long long)b * a.Sq + rt[t]) * a.Hq + h * G + colt[t] % G) * kHeadDim + 8 * cht[t];
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a.q + e),
                                       (__attribute__((address_space(3))) void*)(&qtile[buf][64 * (4 * wave + t)]),
                                       16, 0, 0);
    }
    {
      const long long e = (((long long)b * a.Sq + rti) * kIdxHeads + h + a.Hkv * (icol % nih)) * kIdxDim + 8 * ich;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a.iq + e),
                                       (__attribute__((address_space(3))) void*)(&iqtile[buf][64 * wave]),
                                       16, 0, 0);
    }
    if (tid < 64) {  // main column tid
      const bool ok = chunk * R + mrr < llen[h];
      ml = ok ? a.lse[((long long)b * a.Hq + h * G + tid % G) * a.Sq + rm] * kLog2eB : 0.f;
      mp = ok ? a.q_start + rm : -1;
    } else if (tid < 96) {  // index column tid - 64
      const int ic = tid - 64;
      const bool ok = ic < NI && chunk * R + ic / nih < llen[h];
      ml = ok ? a.lse_idx[((long long)b * kIdxHeads + h + a.Hkv * (ic % nih)) * a.Sq + rm] : 0.f;
      mp = ok ? a.q_start + rm : -1;
    }
  };
  bf16x8 kf[4];  // main-branch K operand of the wave's keys for the current head
  int kf_head = -1;
  const int nsplit = key_splits(total), split = blockIdx.z;
  if (split >= nsplit) return;  // uniform over the work-group
  const int j0 = (int)((long long)split * total / nsplit);
  const int j1 = (int)((long long)(split + 1) * total / nsplit);
  if (j0 < j1) {
    fetch_rows(j0);
    stage(j0, 0);
    if (j0 + 1 < j1) fetch_rows(j0 + 1);
  }
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    int chunk;
    const int h = head_of(j, chunk);
    if (h != kf_head) {  // uniform; loads complete at the wait below
      const u32x4* ks = reinterpret_cast<const u32x4*>(
          a.k + (((long long)b * a.Hkv + h) * a.Skv + min(key, a.Skv - 1)) * kHeadDim);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        u32x4 v = {0, 0, 0, 0};
        if (n < nkeys) v = ks[4 * s4 + g];
        kf[s4] = as_bf16x8(v);
      }
      kf_head = h;
    }
    wait_all_loads();  // job j's tiles and metadata values, job j + 1's rows
    if (tid < 64) {
      clse[buf][tid] = ml;
      cpos[buf][tid] = mp;
    } else if (tid < 96) {
      ilse[buf][tid - 64] = ml;
      ipos[buf][tid - 64] = mp;
    }
    __syncthreads();
    if (j + 1 < j1) {
      stage(j + 1, buf ^ 1);
      if (j + 2 < j1) fetch_rows(j + 2);
    }
    // X = Q K^T: M = main columns (16mt + 4g + r), N = the wave's keys
    f32x4 x[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      x[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        x[mt] = mfma16(as_bf16x8(qtile[buf][swz_slot(16 * mt + n, 4 * ks + g)]), kf[ks], x[mt]);
    }
    // P per row: the G columns of chunk row (16mt + 4g) / G are 16mt + 4g' + r
    // over the G / 4 lanes g' that share it
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = 16 * mt + 4 * g + r;
        sum += (n < nkeys && key <= cpos[buf][col])
                   ? exp2f(x[mt][r] * a.scale_log2 - clse[buf][col]) : 0.f;
      }
#pragma unroll
      for (int o = 16; o < 4 * G; o <<= 1) sum += __shfl_xor(sum, o);
      ptab[wave][(16 * mt + 4 * g) / G][n] = sum * (1.f / (float)G);
    }
    __builtin_amdgcn_wave_barrier();
    // index scores of the chunk's index columns: M = index columns, N = keys
    f32x4 xi[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      xi[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (16 * mt < NI) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          xi[mt] = mfma16(as_bf16x8(iqtile[buf][islot(16 * mt + n, 4 * ks + g)]), ikf[ks], xi[mt]);
      }
    }
    // C = Q - P at the attended (column, key) pairs
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ic = 16 * mt + 4 * g + r;
        const bool ok = n < nkeys && key <= ipos[buf][ic];
        const float pv = ptab[wave][min(ic / nih, 15)][n];
        xi[mt][r] = ok ? exp2f(xi[mt][r] * kLog2eB - ilse[buf][ic]) - pv : 0.f;
      }
    pv_idx<1>(xi, iqtile[buf], dka);  // dik^T += iq^T C^T
    __syncthreads();                  // buffers buf free for job j + 2
  }
  if (n < nkeys) {
    float* dst = nsplit == 1
                     ? a.dik + ((long long)b * a.Skv + key) * kIdxDim
                     : a.dikp + ((((long long)b * a.nblk + c) * kKeySplits + split) * kBlock +
                                 16 * wave + n) * kIdxDim;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt + 4 * g) = dka[mt];
  }
}

// dik of the blocks whose list was split: the splits' partials added in split
// order.  Work-group (block, sequence); thread = (key, 16-dim quarter).
__global__ void __launch_bounds__(256) kl_dik_merge_kernel(KlArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  int total = 0;
  for (int h = 0; h < a.Hkv; ++h) {
    const long long e = ((long long)b * a.Hkv + h) * a.nblk + c;
    total += (a.base[e + 1] - a.base[e] + 64 / a.G - 1) / (64 / a.G);
  }
  const int nsplit = key_splits(total);
  if (nsplit == 1) return;
  const int kl = threadIdx.x / 4, d0 = 16 * (threadIdx.x % 4);
  const int key = c * kBlock + kl;
  if (key >= a.Skv) return;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(
        a.dikp + ((((long long)b * a.nblk + c) * kKeySplits + s) * kBlock + kl) * kIdxDim + d0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += src[i];
  }
  f32x4* dst = reinterpret_cast<f32x4*>(a.dik + ((long long)b * a.Skv + key) * kIdxDim + d0);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = acc[i];
}

char* align256(char* p) { return reinterpret_cast<char*>(((uintptr_t)p + 255) & ~(uintptr_t)255); }

}  // namespace

bool index_kl_supported(const Shape& s) {
  const int nih = kIdxHeads / s.Hkv;
  return (s.G == 4 || s.G == 8 || s.G == 16) && (16 / s.G) * nih <= 8 && s.bs == kBlock;
}

size_t index_kl_workspace_bytes(const Shape& s) {
  return (size_t)s.B * kIdxHeads * s.Sq * 4 + 256 +                       // index log-sum-exp
         (size_t)s.B * s.nblk * kKeySplits * kBlock * kIdxDim * 4 + 256 +  // dik split partials
         inverse_lists_bytes(s);
}

namespace {
template <int G>
hipError_t launch_kl(const Shape& s, const KlArgs& a, hipStream_t st) {
  const size_t lds = (size_t)3 * 1024 * 16 + (size_t)s.nblk * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kl_row_kernel<G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  constexpr int waves = G / 2;  // G row groups, two per wave
  kl_row_kernel<G><<<dim3(ceil_div(s.Sq, kKlTileRows), s.Hkv, s.B), waves * kWave, lds, st>>>(a);
  kl_key_kernel<G><<<dim3(s.nblk, s.B, kKeySplits), 256, 0, st>>>(a);
  kl_dik_merge_kernel<<<dim3(s.nblk, s.B), 256, 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_index_kl_backward(const Shape& s, const void* q, const void* k, const void* iq,
                                    const void* ik, const int32_t* sel, const float* lse,
                                    float* loss, float* diq, float* dik, void* ws,
                                    hipStream_t st) {
  if (!index_kl_supported(s)) return hipErrorInvalidValue;
  char* p = align256(static_cast<char*>(ws));
  float* lse_idx = reinterpret_cast<float*>(p);
  p = align256(p + (size_t)s.B * kIdxHeads * s.Sq * 4);
  float* dikp = reinterpret_cast<float*>(p);
  p += (size_t)s.B * s.nblk * kKeySplits * kBlock * kIdxDim * 4;
  const int32_t* base = nullptr;
  const int32_t* lists = nullptr;
  hipError_t e = launch_inverse_lists(s, sel, p, &base, &lists, st);
  if (e != hipSuccess) return e;
  KlArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
           static_cast<const uint16_t*>(iq), static_cast<const uint16_t*>(ik), sel, lse, loss,
           diq, dik, lse_idx, dikp, base, lists, s.B, s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, s.G,
           s.top_k, s.nblk, kIdxHeads / s.Hkv, s.scale * kLog2eB};
  switch (s.G) {
    case 4: return launch_kl<4>(s, a, st);
    case 8: return launch_kl<8>(s, a, st);
    case 16: return launch_kl<16>(s, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
