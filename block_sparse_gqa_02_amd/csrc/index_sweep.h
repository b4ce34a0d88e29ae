// index_sweep.h — the index branch's inner loop, shared by the block-score
// kernel and the fused block-score + top-k kernel.
//
// A work-group of four waves owns 64 consecutive query rows of one sequence;
// wave w is index head w.  The rows' index queries stay in registers as the B
// operand of v_mfma_f32_32x32x16_bf16; each 64-key index-K block (8 KiB) is
// staged once in LDS (double-buffered, swizzled) for the four waves; keys are
// on the M side, so a block's max per query is a max over the lane's result
// registers plus one v_permlane32_swap.  Block maxima are staged in LDS,
// kStageCols blocks at a time, and handed to a consumer.
#pragma once

#include "common.h"

namespace msa {

constexpr int kTileRows = 64;   // query rows per work-group
constexpr int kStageCols = 32;  // blocks staged before the consumer runs (default)

template <int SC = kStageCols>
struct IndexLds {
  u32x4 ktile[2][64 * 8];                          // 2 x 8 KiB index-K tiles
  float stage[kIdxHeads][kTileRows][SC + 1];       // block maxima per (head, row, block)
};

// Swizzled 16-byte slot of chunk `ch` (0..7) of key row `key`: the 32-lane
// column reads of a K-step then spread over all LDS banks.
__device__ __forceinline__ int ktile_slot(int key, int ch) { return key * 8 + (ch ^ ((key >> 1) & 7)); }

struct IndexTile {
  const uint16_t* iq;  // [B][Sq][4][64]
  const uint16_t* ik;  // [B][Skv][64]
  int b, t0, rows, Sq, Skv;
};

// Sweeps blocks [cbeg, cend) for the tile.  After every SC blocks (and
// at the end) all threads call flush(c0, len, spare) with stage[i][row][e]
// holding the max over block c0+e's keys of head i's scores for row t0+row;
// `spare` is an 8 KiB index-K tile buffer that nothing reads or writes until
// flush returns (scratch for the consumer).  Must be called by all 256
// threads; contains barriers.
template <int SC, typename Flush>
__device__ __forceinline__ void index_sweep(const IndexTile& T, int cbeg, int cend,
                                            IndexLds<SC>& L, Flush&& flush) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;  // index head
  const int lane = tid % kWave;
  if (cbeg >= cend) return;

  // B operand: N-tile nt holds rows 32nt + l%32; K-step ks covers dims
  // 16ks..16ks+15, lane half l/32 holds dims 16ks + 8(l/32) .. +7.
  bf16x8 qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = 32 * nt + lane % 32;
    const bool ok = r < T.rows;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        T.iq + (((size_t)T.b * T.Sq + T.t0 + (ok ? r : 0)) * kIdxHeads + wave) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = src[2 * ks + lane / 32];
      qf[nt][ks] = as_bf16x8(v);
    }
  }

  const u32x4* ikb = reinterpret_cast<const u32x4*>(T.ik + (size_t)T.b * T.Skv * kIdxDim);
  // Index-K blocks travel through registers two blocks ahead of the MFMAs
  // (two register sets that swap roles every block) and through LDS one
  // block ahead (double-buffered tiles).
  struct Regs { u32x4 r0, r1; };
  auto load_tile = [&](int c, Regs& R) {
    const u32x4* src = ikb + (size_t)c * (kBlock * 8);
    R.r0 = src[tid];
    R.r1 = src[tid + 256];
  };
  auto store_tile = [&](int buf, const Regs& R) {
    const int q0 = tid, q1 = tid + 256;
    L.ktile[buf][ktile_slot(q0 / 8, q0 % 8)] = R.r0;
    L.ktile[buf][ktile_slot(q1 / 8, q1 % 8)] = R.r1;
  };

  Regs RA, RB;
  load_tile(cbeg, RA);
  store_tile(0, RA);
  // the loads ahead are unconditional (clamped to the last block) so that
  // every path has the same loads in flight and the waits stay precise
  load_tile(min(cbeg + 1, cend - 1), RA);
  __syncthreads();
  int c0 = cbeg;
  // block c: its tile is in LDS buffer (c - cbeg) & 1, block c + 1 is in
  // `next`, and block c + 2 is loaded into `ahead`
  auto step = [&](int c, Regs& next, Regs& ahead) {
    const int buf = (c - cbeg) & 1;
    const bool more = c + 1 < cend;
    load_tile(min(c + 2, cend - 1), ahead);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // all eight K fragments first, then the MFMAs: one LDS wait per block
    bf16x8 kfr[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + lane / 32;
      kfr[ks][0] = as_bf16x8(L.ktile[buf][ktile_slot(lane % 32, ch)]);
      kfr[ks][1] = as_bf16x8(L.ktile[buf][ktile_slot(32 + lane % 32, ch)]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      acc[0][0] = mfma32(kfr[ks][0], qf[0][ks], acc[0][0]);
      acc[0][1] = mfma32(kfr[ks][0], qf[1][ks], acc[0][1]);
      acc[1][0] = mfma32(kfr[ks][1], qf[0][ks], acc[1][0]);
      acc[1][1] = mfma32(kfr[ks][1], qf[1][ks], acc[1][1]);
    }
    float m0 = fmax_nn(acc[0][0][0], acc[1][0][0]), m1 = fmax_nn(acc[0][1][0], acc[1][1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      m0 = fmax_nn(m0, fmax_nn(acc[0][0][r], acc[1][0][r]));
      m1 = fmax_nn(m1, fmax_nn(acc[0][1][r], acc[1][1][r]));
    }
    // lane l now holds the block max of row l for head `wave`
    L.stage[wave][lane][c - c0] = halves_max(m0, m1);

    if (more) store_tile(buf ^ 1, next);
    __syncthreads();
    if (c + 1 - c0 == SC || !more) {
      flush(c0, c + 1 - c0, &L.ktile[buf][0]);
      c0 = c + 1;
      __syncthreads();
    }
  };
  int c = cbeg;
  for (; c + 1 < cend; c += 2) {
    step(c, RA, RB);
    step(c + 1, RB, RA);
  }
  if (c < cend) step(c, RA, RB);
}

}  // namespace msa
