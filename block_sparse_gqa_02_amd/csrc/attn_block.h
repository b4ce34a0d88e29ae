// attn_block.h — one wave attending one query row's GQA head group to a
// sequence of 64-token K/V blocks with an online softmax, on
// v_mfma_f32_16x16x32_bf16.
//
// Exact softmax attention over the selected blocks is the main branch of MSA
// (topic page "MiniMax稀疏注意力", summary paragraph).  Blocks are contiguous
// 16 KiB runs of one KV head's K and V (the block-level retrieval the pages
// credit with restoring contiguous reads: talk summary "How MiniMax M3 Was
// Built", section "Block-level retrieval makes sparse attention easier to run
// on GPUs").
//
// Mapping (lane l, g = l/16, n = l%16): column n is query head hq0 + n of the
// row (n < G; the other columns carry zero queries and are discarded).
//   S^T = K Q^T : A = K block (keys on M, 16 per M-tile, read straight from
//                 global memory as 16-byte runs), B = Q^T held in registers.
//                 Result reg r of M-tile mt is key 16mt + 4g + r, column n.
//   O^T += V^T P^T : B = P^T comes from the lane's own S^T registers (K-step kv
//                 uses M-tiles 2kv and 2kv+1, so no lane exchange is needed);
//                 A = V^T gathered from an LDS copy of the V block with 8-byte
//                 reads; the output dims are permuted so that one 8-byte read
//                 feeds four M-tiles.  O^T M-tile (hf, j) row 4g + r is dim
//                 64hf + 16g + 4r + j, so a lane ends up owning 2 runs of 16
//                 contiguous dims of its column.
// Softmax runs in the log2 domain with fp32 state (m, l); P is rounded to bf16
// for the PV product.
#pragma once

#include "common.h"

namespace msa {

// 16-byte chunk slot of chunk `ch` (0..15) of key row `key` in a V tile:
// flips the upper half for keys with bit 2 set, so that the four 16-lane groups
// of an 8-byte column read hit disjoint bank halves.
__device__ __forceinline__ int vtile_slot(int key, int ch) { return key * 16 + (ch ^ (((key >> 2) & 1) << 3)); }

struct WaveAttn {
  f32x4 o[8];     // O^T accumulators, M-tile index 4*hf + j
  float m;        // running max of the column (log2 domain)
  float l;        // this lane's share of the column's normaliser
  bf16x8 qf[4];   // Q^T operand, K-step ks: dims 32ks + 8g .. +7 of column n

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -__builtin_huge_valf();
    l = 0.f;
  }

  // q_row: the row's first query head of the group ([G][128] bf16 contiguous).
  __device__ __forceinline__ void load_q(const uint16_t* q_row, int G) {
    const int lane = lane_id(), n = lane % 16, g = lane / 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (n < G) v = reinterpret_cast<const u32x4*>(q_row + (size_t)n * kHeadDim)[4 * ks + g];
      qf[ks] = as_bf16x8(v);
    }
  }

  // Attends block `c` (keys 64c .. 64c+63 of k_head / v_head) with keys
  // j > pos masked.  vlds: this wave's 16 KiB V staging area.
  __device__ __forceinline__ void block(const uint16_t* k_head, const uint16_t* v_head, int c,
                                        int pos, float scale_log2, u32x4* vlds) {
    block_at(k_head + (size_t)c * kBlock * kHeadDim, v_head + (size_t)c * kBlock * kHeadDim, c,
             pos, scale_log2, vlds);
  }

  // The same with the block's 64 K and V rows at k_blk / v_blk (a cache page).
  __device__ __forceinline__ void block_at(const uint16_t* k_blk, const uint16_t* v_blk, int c,
                                           int pos, float scale_log2, u32x4* vlds) {
    u32x4 vr[16], kr[4][4];
    const int last = min(pos - c * kBlock, kBlock - 1);
    load_v(v_blk, last, vr);
    load_k(k_blk, last, kr);
    store_v(vr, vlds);
    attend(kr, c, pos, scale_log2, vlds, [] {}, [] {});
  }

  // The phases of block_at, for callers that overlap one block's loads with
  // the previous block's arithmetic.  Rows past `last` (= min(pos - 64c, 63);
  // only in the own block, which may also run past the end of the cache) are
  // read from row `last` instead and masked in attend().
  __device__ __forceinline__ static void load_v(const uint16_t* v_blk, int last, u32x4 (&vr)[16]) {
    const int lane = lane_id();
    const u32x4* vb = reinterpret_cast<const u32x4*>(v_blk);
    // V block: 1024 chunks of 16 B; chunk q = key q/16, dim chunk q%16
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int q = s * kWave + lane;
      vr[s] = vb[min(q / 16, last) * 16 + q % 16];
    }
  }
  // Stream: non-temporal loads, for data read once (decode caches).
  template <bool Stream = false>
  __device__ __forceinline__ static void load_k(const uint16_t* k_blk, int last,
                                                u32x4 (&kr)[4][4]) {
    const int lane = lane_id(), n = lane % 16, g = lane / 16;
    const u32x4* kb = reinterpret_cast<const u32x4*>(k_blk);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4* src = kb + min(16 * mt + n, last) * 16 + 4 * ks + g;
        kr[mt][ks] = Stream ? __builtin_nontemporal_load(src) : *src;
      }
  }
  // The V block straight into an LDS tile (laid out as store_v lays it out)
  // with 16-byte LDS-bound loads: load t writes slots 64t .. 64t+63, so lane
  // i fetches the chunk that belongs at slot 64t + i.  The data is in LDS once
  // these 16 loads have completed (vmcnt).  The loads are non-temporal (the
  // decode caches are read once).
  __device__ __forceinline__ static void load_v_lds(const uint16_t* v_blk, int last, u32x4* tile) {
    const int lane = lane_id();
    const u32x4* vb = reinterpret_cast<const u32x4*>(v_blk);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int slot = t * kWave + lane;
      const int key = slot >> 4;
      const int ch = (slot & 15) ^ (((key >> 2) & 1) << 3);  // vtile_slot is its own inverse
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vb + min(key, last) * 16 + ch),
                                       (__attribute__((address_space(3))) void*)(tile + t * kWave),
                                       16, 0, kCachePolicyNT);
    }
  }
  // Copies the V block into this wave's LDS tile.  The previous block's reads
  // of the tile must be complete (attend() ends with them).
  __device__ __forceinline__ static void store_v(const u32x4 (&vr)[16], u32x4* vlds) {
    const int lane = lane_id();
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int q = s * kWave + lane;
      vlds[vtile_slot(q / 16, q % 16)] = vr[s];
    }
  }

  // Attends block c from K in registers and V in the LDS tile; after_s() runs
  // once the S products have taken their K operands (kr may then be reloaded),
  // before_pv() right before the first read of the V tile.
  template <typename AfterS, typename BeforePV>
  __device__ __forceinline__ void attend(const u32x4 (&kr)[4][4], int c, int pos,
                                         float scale_log2, const u32x4* vlds, AfterS&& after_s,
                                         BeforePV&& before_pv) {
    const int lane = lane_id(), g = lane / 16;
    // S^T = K Q^T
    f32x4 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[mt] = mfma16(as_bf16x8(kr[mt][ks]), qf[ks], sc[mt]);
    }
    after_s();
    // online softmax (log2 domain, v_exp_f32 directly: weights below 2^-126
    // flush to zero); keys beyond pos are masked
    const int key0 = c * kBlock + 4 * g;
    const bool partial = c * kBlock + kBlock - 1 > pos;
    float bmax = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float z = sc[mt][r] * scale_log2;
        if (partial && key0 + 16 * mt + r > pos) z = -__builtin_huge_valf();
        sc[mt][r] = z;
        bmax = fmaxf(bmax, z);
      }
    bmax = wave_max_xor16_32(bmax);
    const float m_new = fmaxf(m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[mt][r] - m_new);
        sc[mt][r] = p;
        psum += p;
      }
    l = l * alpha + psum;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    __builtin_amdgcn_wave_barrier();  // V tile writes above precede the reads below
    before_pv();
    pv_step(sc, vlds, o);
    __builtin_amdgcn_wave_barrier();  // reads done before the next block overwrites the tile
  }

  // acc^T += T^T P^T over one 64-row tile: T is the tile in LDS ([64][128]
  // bf16 in the vtile_slot layout), P^T the probabilities in S^T layout (pt[mt]
  // reg r = tile row 16mt + 4g + r, column n; rounded to bf16 here); acc has
  // the O^T layout (M-tile 4hf + j, row 4g + r = dim 64hf + 16g + 4r + j).
  __device__ __forceinline__ static void pv_step(const f32x4 (&pt)[4], const u32x4* tile,
                                                 f32x4 (&acc)[8]) {
    const int lane = lane_id(), n = lane % 16, g = lane / 16;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      u32x4 pw;
      pw[0] = pack_bf16x2(pt[2 * kv][0], pt[2 * kv][1]);
      pw[1] = pack_bf16x2(pt[2 * kv][2], pt[2 * kv][3]);
      pw[2] = pack_bf16x2(pt[2 * kv + 1][0], pt[2 * kv + 1][1]);
      pw[3] = pack_bf16x2(pt[2 * kv + 1][2], pt[2 * kv + 1][3]);
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // key of k-slot i: 32kv + 16(i/4) + 4g + i%4; 8 bytes = dims 64hf+4n..+3
        u32x2 rd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = 32 * kv + 16 * (i / 4) + 4 * g + (i % 4);
          const int ch = 8 * hf + n / 2;
          const u32x2* p = reinterpret_cast<const u32x2*>(tile + vtile_slot(key, ch)) + (n & 1);
          rd[i] = *p;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 a;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = rd[2 * w][j / 2], y = rd[2 * w + 1][j / 2];
            a[w] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
          }
          acc[4 * hf + j] = mfma16(as_bf16x8(a), pb, acc[4 * hf + j]);
        }
      }
    }
  }

  // Column normaliser (sum over the four lane groups).
  __device__ __forceinline__ float total_l() const { return wave_sum_xor16_32(l); }

  // Writes this lane's 32 dims of column n, scaled by inv, as bf16 to
  // out_head (the column's [128] output row).
  __device__ __forceinline__ void store_bf16(uint16_t* out_head, float inv) const {
    const int g = lane_id() / 16;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 w0, w1;
      // element e = 4r + j of the run 64hf + 16g .. +15 is o[4hf + j][r]
#pragma unroll
      for (int qd = 0; qd < 8; ++qd) {
        const int e0 = 2 * qd, e1 = 2 * qd + 1;
        const uint32_t v = pack_bf16x2(o[4 * hf + (e0 & 3)][e0 >> 2] * inv,
                                       o[4 * hf + (e1 & 3)][e1 >> 2] * inv);
        if (qd < 4) w0[qd] = v; else w1[qd - 4] = v;
      }
      u32x4* dst = reinterpret_cast<u32x4*>(out_head + 64 * hf + 16 * g);
      dst[0] = w0;
      dst[1] = w1;
    }
  }

  // Writes the 32 dims of column n unnormalised in fp32 (split-K partials).
  __device__ __forceinline__ void store_f32(float* out_head) const {
    const int g = lane_id() / 16;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v = {o[4 * hf + 0][r], o[4 * hf + 1][r], o[4 * hf + 2][r], o[4 * hf + 3][r]};
        *reinterpret_cast<f32x4*>(out_head + 64 * hf + 16 * g + 4 * r) = v;
      }
    }
  }
};

}  // namespace msa
