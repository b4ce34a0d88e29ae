// attn_bwd.hip — gradient of the sparse GQA prefill attention (main branch).
//
// The pages say the authors wrote kernels for training as well as inference
// (talk summary "How MiniMax M3 Was Built", section "MSA uses a lightweight
// index branch before sparse attention"; news write-up "MiniMax Researcher
// Olive Song: Sparse Attention Cannot Be Directly Ported…", paragraph 5).  This
// is the gradient of the main branch for a given selection: with
// p = softmax(scale q.k) over the selected causal tokens and o = sum p v,
//   Dsum = dout . o,  dp_a = dout . v_a,  ds_a = p_a (dp_a - Dsum),
//   dq = scale sum ds_a k_a,  dk_a += scale ds_a q,  dv_a += p_a dout.
// The selection gets no gradient.  Softmax weights are recomputed from the
// forward's log-sum-exp; Dsum uses the forward's (bf16) output.
//
// Kernels, in launch order:
//   dsum_kernel      Dsum per (sequence, query head, row).
//   inverse kernels  for every (sequence, KV head, block) the ascending list of
//                    rows that selected it: per batch of 64 rows a bitmap over
//                    blocks in LDS (bit i = row i of the batch), counted, scanned
//                    over batches and over blocks, then filled in row order.
//                    Deterministic: no atomics outside LDS bit sets.
//   dq_tile_kernel   (groups of 4 or 8 heads) a work-group per 16-row tile
//                    walks the union of the tile's selected blocks, each
//                    block's K and V fetched once into LDS; per block and
//                    wanting row group S^T = K Q^T, dP^T = V dO^T, dS from the
//                    saved log-sum-exp, dQ^T += K^T dS^T (the forward's PV step
//                    with K in the V-tile role).
//   dq_kernel        the same per (row, KV head) wave, for other group sizes.
//   dkdv_kernel      one work-group per (KV head, block), wave w owning keys
//                    16w..16w+15: the block's rows are taken 64 query columns
//                    (rows x group heads) at a time through LDS tiles of Q and
//                    dO; X = Q K^T, Y = dO V^T, then dV^T += dO^T P and
//                    dK^T += Q^T dS, again the forward's PV step.
// Score-side operand layouts follow attn_block.h; the products with a transposed
// tile (dQ^T += K^T dS^T, dV^T += dO^T P, dK^T += Q^T dS) use pv_tr below.
#include "attn_block.h"
#include "bwd_tiles.h"
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kBatchRows = 64;  // rows per inverse-list batch (one bit each)

struct BwdArgs {
  const uint16_t* q;     // [B][Sq][Hq][128]
  const uint16_t* k;     // [B][Hkv][Skv][128]
  const uint16_t* v;
  const int32_t* sel;    // [B][Hkv][Sq][top_k]
  const uint16_t* out;   // [B][Sq][Hq][128] forward output
  const float* lse;      // [B][Hq][Sq] forward log-sum-exp (natural log)
  const uint16_t* dout;  // [B][Sq][Hq][128]
  float* dq;             // [B][Sq][Hq][128]
  float* dk;             // [B][Hkv][Skv][128]
  float* dv;
  float* dsum;           // workspace [B][Hq][Sq]
  int32_t* bcnt;         // workspace [B][Hkv][nbatch][nblk]: counts, then offsets in the list
  int32_t* base;         // workspace [B*Hkv*nblk + 1]: list starts (exclusive scan)
  int32_t* lists;        // workspace [B*Hkv*Sq*top_k]: rows per (sequence, KV head, block)
  int32_t* slotpos;      // optional [B][Hkv][Sq][top_k]: list position of each entry, or -1
  int B, Sq, Skv, q_start, Hq, Hkv, G, top_k, nblk, nbatch;
  float scale, scale_log2;
};

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// acc += T^T P^T over one tile T (swz_slot layout; its 64 rows are the
// contraction index) with P^T in S^T register layout: pt[mt] register r is
// tile row 16mt + 4g + r, column n; rounded to bf16 here.  The T^T operand is
// read with ds_read_b64_tr_b16: lane (g, n) of the read for K-step kv, half hf
// and M-tile mt loads dims 16mt + 4(n%4) .. +3 of tile row 32kv + 16hf + 4g +
// n/4 and receives dim 16mt + n of rows 32kv + 16hf + 4g + 0..3, so k-slot i
// of the operand is row 32kv + 16(i/4) + 4g + i%4, the row of the lane's own
// P^T register.  acc[mt] register r is dim 16mt + 4g + r of column n.
__device__ __forceinline__ void pv_tr(const f32x4 (&pt)[4], const u32x4* tile, f32x4 (&acc)[8]) {
  const int lane = lane_id(), n = lane % 16, g = lane / 16;
  // byte (32kv + 16hf) * 256 + (vlane ^ 32mt) of the tile
  const int r15 = 4 * g + n / 4;
  int vlane = r15 * 256 + 16 * (((n >> 1) & 1) ^ r15) + 8 * (n & 1);
  // opaque here, so that a caller's loop does not keep every tile's read
  // addresses live as loop invariants (registers)
  asm volatile("" : "+v"(vlane));
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    u32x4 pw;
    pw[0] = pack_bf16x2(pt[2 * kv][0], pt[2 * kv][1]);
    pw[1] = pack_bf16x2(pt[2 * kv][2], pt[2 * kv][3]);
    pw[2] = pack_bf16x2(pt[2 * kv + 1][0], pt[2 * kv + 1][1]);
    pw[3] = pack_bf16x2(pt[2 * kv + 1][2], pt[2 * kv + 1][3]);
    const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint32_t va = (uint32_t)(32 * kv * 256) + (uint32_t)(vlane ^ (32 * mt));
      const s16x4 lo = lds_read_tr_at(tile, va);
      const s16x4 hi = lds_read_tr_at(tile, va + 16 * 256);
      const bf16x8 tf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[mt] = mfma16(tf, pb, acc[mt]);
    }
  }
}

// acc in pv_tr's layout; writes column n's 128 dims times mul.
__device__ __forceinline__ void store_tr_f32(const f32x4 (&acc)[8], float* col_base, float mul) {
  const int g = lane_id() / 16;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(col_base + 16 * mt + 4 * g) = acc[mt] * mul;
}

// Dsum[b][hq][t] = sum_d dout * out; one wave per (b, t, hq), lanes over dim pairs.
__global__ void __launch_bounds__(256) dsum_kernel(BwdArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const long long w = (long long)blockIdx.x * 4 + wave;  // (b * Sq + t) * Hq + hq
  if (w >= (long long)a.B * a.Sq * a.Hq) return;
  const uint32_t o2 = reinterpret_cast<const uint32_t*>(a.out + w * kHeadDim)[lane];
  const uint32_t g2 = reinterpret_cast<const uint32_t*>(a.dout + w * kHeadDim)[lane];
  const float s = wave_sum64(bf16_lo(o2) * bf16_lo(g2) + bf16_hi(o2) * bf16_hi(g2));
  if (lane == 0) {
    const int hq = (int)(w % a.Hq);
    const long long bt = w / a.Hq;
    const int t = (int)(bt % a.Sq), b = (int)(bt / a.Sq);
    a.dsum[((long long)b * a.Hq + hq) * a.Sq + t] = s;
  }
}

// Inverse lists, pass 1 (FILL = false: per-batch counts) and pass 3 (FILL =
// true: rows written at their offsets; with slotpos, also the position in its
// block's list of every selection entry, -1 for entries that attend nothing).  One work-group per (sequence, KV
// head, batch of 64 rows); the bitmap (one 64-bit word per block, dynamic LDS)
// marks which rows of the batch selected each block.  A selection entry
// counts when 0 <= c <= the row's own block, the blocks the forward attends.
template <bool FILL>
__global__ void __launch_bounds__(256) inverse_kernel(BwdArgs a) {
  extern __shared__ unsigned long long bm[];
  const int batch = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = batch * kBatchRows;
  const int rows = min(kBatchRows, a.Sq - t0);
  const int cmax = (a.q_start + t0 + rows - 1) / kBlock;  // last block the batch can select
  for (int c = threadIdx.x; c <= cmax; c += 256) bm[c] = 0ull;
  __syncthreads();
  const int32_t* srow = a.sel + (((long long)b * a.Hkv + h) * a.Sq + t0) * a.top_k;
  for (int idx = threadIdx.x; idx < rows * a.top_k; idx += 256) {
    const int i = idx / a.top_k;
    const int c = srow[idx];
    const int cur = (a.q_start + t0 + i) / kBlock;
    if (c >= 0 && c <= cur) atomicOr(&bm[c], 1ull << i);
  }
  __syncthreads();
  const long long hb = (long long)b * a.Hkv + h;
  int32_t* cnt = a.bcnt + (hb * a.nbatch + batch) * a.nblk;
  for (int c = threadIdx.x; c <= cmax; c += 256) {
    unsigned long long m = bm[c];
    if (!FILL) {
      cnt[c] = __popcll(m);
    } else {
      int32_t* dst = a.lists + a.base[hb * a.nblk + c] + cnt[c];
      while (m != 0ull) {
        const int i = __builtin_ctzll(m);
        m &= m - 1;
        *dst++ = t0 + i;
      }
    }
  }
  if (FILL && a.slotpos) {
    // row i of the batch sits after the batch's earlier rows that chose c
    int32_t* sp = a.slotpos + (hb * a.Sq + t0) * a.top_k;
    for (int idx = threadIdx.x; idx < rows * a.top_k; idx += 256) {
      const int i = idx / a.top_k;
      const int c = srow[idx];
      const int cur = (a.q_start + t0 + i) / kBlock;
      int32_t pos = -1;
      if (c >= 0 && c <= cur)
        pos = a.base[hb * a.nblk + c] + cnt[c] + __popcll(bm[c] & ((1ull << i) - 1ull));
      sp[idx] = pos;
    }
  }
}

// Pass 2a: per (sequence, KV head, block), the exclusive scan of the batch
// counts (in place) and the list length.  A work-group takes 16 blocks and
// cuts the batches into 16 segments, a thread per (segment, block): segment
// sums, then each thread rewrites its segment from the sum of the segments
// before it.  A batch whose last row's block is below c holds no count for c
// (pass 1 never wrote it, pass 3 never reads it).
constexpr int kScanBlocks = 16, kScanSegs = 16;
__global__ void __launch_bounds__(256) batch_scan_kernel(BwdArgs a) {
  __shared__ int32_t part[kScanSegs][kScanBlocks];
  const int cl = threadIdx.x % kScanBlocks, seg = threadIdx.x / kScanBlocks;
  const int c = blockIdx.x * kScanBlocks + cl;
  const long long hb = blockIdx.y;  // b * Hkv + h
  const bool okc = c < a.nblk;
  int32_t* cnt = a.bcnt + hb * a.nbatch * a.nblk + (okc ? c : 0);
  const int j0 = (int)((long long)seg * a.nbatch / kScanSegs);
  const int j1 = (int)((long long)(seg + 1) * a.nbatch / kScanSegs);
  auto holds = [&](int j) {
    const int rows = min(kBatchRows, a.Sq - j * kBatchRows);
    return (a.q_start + j * kBatchRows + rows - 1) / kBlock >= c;
  };
  int sum = 0;
  if (okc)
    for (int j = j0; j < j1; ++j)
      if (holds(j)) sum += cnt[(long long)j * a.nblk];
  part[seg][cl] = sum;
  __syncthreads();
  int run = 0;
  for (int x = 0; x < seg; ++x) run += part[x][cl];
  if (okc) {
    for (int j = j0; j < j1; ++j) {
      if (!holds(j)) continue;
      const int x = cnt[(long long)j * a.nblk];
      cnt[(long long)j * a.nblk] = run;
      run += x;
    }
    if (seg == kScanSegs - 1) a.base[hb * a.nblk + c] = run;  // length; a start after pass 2b
  }
}

// Pass 2b: exclusive scan of the list lengths over all (sequence, KV head,
// block), in one work-group; base[n] receives the total.
__global__ void __launch_bounds__(256) base_scan_kernel(BwdArgs a) {
  __shared__ int32_t part[256];
  const long long n = (long long)a.B * a.Hkv * a.nblk;
  const long long per = (n + 255) / 256;
  const long long lo = threadIdx.x * per, hi = min(n, lo + per);
  int32_t s = 0;
  for (long long i = lo; i < hi; ++i) s += a.base[i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int i = 0; i < 256; ++i) {
      const int32_t x = part[i];
      part[i] = run;
      run += x;
    }
    a.base[n] = run;
  }
  __syncthreads();
  int32_t run = part[threadIdx.x];
  for (long long i = lo; i < hi; ++i) {
    const int32_t x = a.base[i];
    a.base[i] = run;
    run += x;
  }
}

// dQ: one wave per (sequence, KV head, row); columns n < G are the group's
// query heads.
__global__ void __launch_bounds__(256) dq_kernel(BwdArgs a) {
  __shared__ u32x4 ktile[4][kBlock * 16];  // per wave: the block's K in the swz_slot layout
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n = lane % 16, g = lane / 16;
  const long long w = (long long)blockIdx.x * 4 + wave;  // ((b * Hkv + h) * Sq + t)
  if (w >= (long long)a.B * a.Hkv * a.Sq) return;
  const int t = (int)(w % a.Sq);
  const long long hb = w / a.Sq;
  const int h = (int)(hb % a.Hkv), b = (int)(hb / a.Hkv);
  const int pos = a.q_start + t, cur = pos / kBlock;
  const int hq0 = h * a.G;
  WaveAttn qs, gs;  // Q^T and dO^T operands of the row's group
  qs.load_q(a.q + ((long long)b * a.Sq + t) * a.Hq * kHeadDim + (long long)hq0 * kHeadDim, a.G);
  gs.load_q(a.dout + ((long long)b * a.Sq + t) * a.Hq * kHeadDim + (long long)hq0 * kHeadDim, a.G);
  const bool col_ok = n < a.G;
  const float lse2 = col_ok ? a.lse[((long long)b * a.Hq + hq0 + n) * a.Sq + t] * kLog2eB : 0.f;
  const float ds0 = col_ok ? a.dsum[((long long)b * a.Hq + hq0 + n) * a.Sq + t] : 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int32_t* list = a.sel + w * a.top_k;
  u32x4* tile = ktile[wave];
  for (int r = 0; r < a.top_k; ++r) {
    const int c = list[r];
    if (c < 0 || c > cur) continue;
    const long long off = (hb * a.Skv + (long long)c * kBlock) * kHeadDim;
    const int last = min(pos - c * kBlock, kBlock - 1);
    u32x4 vr[16], vk[4][4];
    WaveAttn::load_v(a.k + off, last, vr);   // K, for the LDS tile
    WaveAttn::load_k(a.v + off, last, vk);   // V, as the A operand of dP^T
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // chunk q = 64 i + lane: key q / 16, dim chunk q % 16
      const int q = i * kWave + lane;
      tile[swz_slot(q >> 4, q & 15)] = vr[i];
    }
    __builtin_amdgcn_wave_barrier();
    f32x4 s[4], dp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = as_bf16x8(tile[swz_slot(16 * mt + n, 4 * ks + g)]);
        s[mt] = mfma16(kf, qs.qf[ks], s[mt]);
        dp[mt] = mfma16(as_bf16x8(vk[mt][ks]), gs.qf[ks], dp[mt]);
      }
    }
    // dS^T in the S^T layout: key 64c + 16mt + 4g + r, column n
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = c * kBlock + 16 * mt + 4 * g + rr;
        const float p = (col_ok && key <= pos) ? exp2f(s[mt][rr] * a.scale_log2 - lse2) : 0.f;
        s[mt][rr] = p * (dp[mt][rr] - ds0);
      }
    pv_tr(s, tile, acc);  // dQ^T += K^T dS^T
    __builtin_amdgcn_wave_barrier();  // tile reads done before the next block's writes
  }
  if (col_ok) store_tr_f32(acc, a.dq + (((long long)b * a.Sq + t) * a.Hq + hq0 + n) * kHeadDim,
                           a.scale);
}

// dK and dV of one block: work-group per (block, KV head, sequence), wave w
// owns keys 16w..16w+15.  Query columns (row slot i / G, head i % G) are taken
// 64 at a time ("chunks") from the block's row list.  Chunk j+1's Q and dO rows
// travel by LDS-bound loads into the second pair of tiles while chunk j is
// computed; the row indices that address them are loaded a chunk earlier.
__global__ void __launch_bounds__(256) dkdv_kernel(BwdArgs a) {
  // Two tile pairs (64 columns x 128 dims of Q and of dO, swz_slot layout),
  // each tile its own LDS object and the chunk loop unrolled by two, so that
  // every access names its tile and the compiler does not make the reads of
  // one pair wait for the LDS-bound loads into the other.
  __shared__ u32x4 qtile0[kBlock * 16], qtile1[kBlock * 16];
  __shared__ u32x4 gtile0[kBlock * 16], gtile1[kBlock * 16];
  __shared__ float clse[2][64], cds[2][64];
  __shared__ int cpos[2][64];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const long long hb = (long long)b * a.Hkv + h;
  const int key0 = c * kBlock + 16 * wave;          // this wave's first key
  const int nkeys = max(0, min(16, a.Skv - key0));  // keys of the wave inside the cache
  const long long koff = (hb * a.Skv + key0) * kHeadDim;
  WaveAttn ks_, vs_;  // K^T and V^T operands: column n = key key0 + n (zero past the cache)
  ks_.load_q(a.k + (nkeys > 0 ? koff : 0), nkeys);
  vs_.load_q(a.v + (nkeys > 0 ? koff : 0), nkeys);
  f32x4 dka[8], dva[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dka[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    dva[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int32_t beg = a.base[hb * a.nblk + c], len = a.base[hb * a.nblk + c + 1] - beg;
  const int32_t* rows = a.lists + beg;
  const int R = 64 / a.G;  // rows per chunk
  const int nchunk = (len + R - 1) / R;
  // This thread's four 16-byte slots of a tile: load t of the wave fills slots
  // 64 (4 wave + t) + lane, i.e. column 4 (4 wave + t) + lane / 16 and, through
  // the tile's XOR swizzle, dim chunk ch_t.
  int colt[4], cht[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    colt[t] = 4 * (4 * wave + t) + lane / 16;
    cht[t] = (lane & 15) ^ (colt[t] & 15);
  }
  // row of column col in chunk j (entries past the list repeat its first row;
  // their columns are masked through cpos = -1)
  auto row_of = [&](int j, int col) { return rows[min(j * R + col / a.G, len - 1)]; };
  int rt[4];          // rows of this thread's slots, next chunk to stage
  int rmeta = 0;      // row of column lane, next chunk to stage
  // Column lane's metadata, loaded raw with its chunk's tiles and turned into
  // LDS values at the next iteration (wave 0's are the ones kept): a value
  // used right after its load would make the wait for it, which the in-order
  // load counter extends to the tile loads issued before it, land inside the
  // iteration that is meant to overlap them.
  float ml = 0.f, md = 0.f;
  int mrow = 0;
  bool mok = false;
  auto stage = [&](int j, u32x4* qdst, u32x4* gdst) {  // chunk j's loads (rows in rt / rmeta)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const long long e = (((long long)b * a.Sq + rt[t]) * a.Hq + h * a.G + colt[t] % a.G) *
                          kHeadDim + 8 * cht[t];
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a.q + e),
                                       (__attribute__((address_space(3))) void*)(qdst + 64 * (4 * wave + t)),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a.dout + e),
                                       (__attribute__((address_space(3))) void*)(gdst + 64 * (4 * wave + t)),
                                       16, 0, 0);
    }
    mok = j * R + lane / a.G < len;
    mrow = rmeta;
    const long long li = ((long long)b * a.Hq + h * a.G + lane % a.G) * a.Sq + rmeta;
    ml = a.lse[li];
    md = a.dsum[li];
  };
  auto fetch_rows = [&](int j) {  // row indices of chunk j into rt / rmeta
#pragma unroll
    for (int t = 0; t < 4; ++t) rt[t] = row_of(j, colt[t]);
    rmeta = row_of(j, lane);
  };
  if (nchunk > 0) {
    fetch_rows(0);
    stage(0, qtile0, gtile0);
    if (nchunk > 1) fetch_rows(1);
  }
  // chunk j from tiles (qcur, gcur); chunk j + 1 staged into (qnext, gnext)
  auto step = [&](int j, int bf, const u32x4* qcur, const u32x4* gcur, u32x4* qnext,
                  u32x4* gnext) {
    wait_all_loads();  // chunk j's tiles (issued last iteration) and its metadata values
    if (tid < 64) {
      clse[bf][tid] = mok ? ml * kLog2eB : 0.f;
      cds[bf][tid] = mok ? md : 0.f;
      cpos[bf][tid] = mok ? a.q_start + mrow : -1;
    }
    __syncthreads();
    if (j + 1 < nchunk) {
      stage(j + 1, qnext, gnext);
      if (j + 2 < nchunk) fetch_rows(j + 2);
    }
    int nl = n, gl = g;  // opaque lane coordinates: the tile read addresses stay per step
    asm volatile("" : "+v"(nl), "+v"(gl));
    // X = Q K^T and Y = dO V^T: M = columns (M-tile mt: columns 16mt + 4g + r
    // in the result), N = this wave's keys
    f32x4 x[4], y[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      x[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      y[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 qa = as_bf16x8(qcur[swz_slot(16 * mt + nl, 4 * ks + gl)]);
        const bf16x8 ga = as_bf16x8(gcur[swz_slot(16 * mt + nl, 4 * ks + gl)]);
        x[mt] = mfma16(qa, ks_.qf[ks], x[mt]);
        y[mt] = mfma16(ga, vs_.qf[ks], y[mt]);
      }
    }
    const int key = key0 + n;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int col = 16 * mt + 4 * g + rr;
        const float p = (n < nkeys && key <= cpos[bf][col])
                            ? exp2f(x[mt][rr] * a.scale_log2 - clse[bf][col]) : 0.f;
        x[mt][rr] = p;                              // P (columns x keys)
        y[mt][rr] = p * (y[mt][rr] - cds[bf][col]);  // dS
      }
    pv_tr(x, gcur, dva);  // dV^T += dO^T P
    pv_tr(y, qcur, dka);  // dK^T += Q^T dS
    __syncthreads();      // tiles (qcur, gcur) free for chunk j + 2
  };
  for (int j = 0; j < nchunk; j += 2) {
    step(j, 0, qtile0, gtile0, qtile1, gtile1);
    __builtin_amdgcn_sched_barrier(0);  // the two steps are not interleaved (registers)
    if (j + 1 < nchunk) step(j + 1, 1, qtile1, gtile1, qtile0, gtile0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (n < nkeys) {
    store_tr_f32(dva, a.dv + (hb * a.Skv + key0 + n) * kHeadDim, 1.f);
    store_tr_f32(dka, a.dk + (hb * a.Skv + key0 + n) * kHeadDim, a.scale);
  }
}

// dQ, tile-union schedule (groups of 4 or 8 query heads): a work-group owns
// 16 consecutive rows of one (sequence, KV head), split into row groups of
// 16 / G rows x G heads (the 16 MFMA columns), two groups per wave.  A 32-bit
// mask per block (LDS) records which of the tile's rows selected it; the
// work-group walks the blocks with a nonzero mask in ascending order, fetching
// each one's K and V once into double-buffered LDS tiles by LDS-bound loads
// (the next block's while the current one is computed).  A group computes a
// block only if one of its rows selected it, and a column whose row did not
// gets P = 0.  Per block: S^T = K Q^T and dP^T = V dO^T from the tiles, dS,
// and dQ^T += K^T dS^T.
//
// The K and V tiles use the swz_slot layout; dQ^T += K^T dS^T is pv_tr with
// the K tile.
constexpr int kDqTileRows = 16;  // 4 waves at G = 8: two work-groups share a CU


__global__ void __launch_bounds__(512) dq_tile_kernel(BwdArgs a) {
  // K and V of the current and the next block, each tile its own LDS object,
  // and the block loop unrolled by two so that every access names its tile:
  // the compiler then tells the LDS-bound loads into one pair from the reads
  // of the other (and of the row masks) and makes neither wait for them.
  __shared__ u32x4 ktile0[kBlock * 16], ktile1[kBlock * 16];
  __shared__ u32x4 vtile0[kBlock * 16], vtile1[kBlock * 16];
  extern __shared__ uint32_t rmask[];  // [cmax + 1]
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int nwaves = blockDim.x / kWave;
  const int n = lane % 16, g = lane / 16;
  const int h = blockIdx.y, b = blockIdx.z;
  const int RPG = 16 / a.G;  // rows per group
  const int t0 = blockIdx.x * kDqTileRows;
  const int rows = min(kDqTileRows, a.Sq - t0);
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
  // this lane's column in each of the wave's two groups
  bf16x8 qf[2][4], gf[2][4];
  float lse2[2], dsv[2];
  int pos[2], rloc[2];
  long long colbase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    rloc[j] = (2 * wave + j) * RPG + n / a.G;
    const bool ok = rloc[j] < rows;
    const int t = t0 + (ok ? rloc[j] : 0), hq = h * a.G + n % a.G;
    colbase[j] = ((long long)b * a.Sq + t) * a.Hq + hq;
    const u32x4* qs = reinterpret_cast<const u32x4*>(a.q + colbase[j] * kHeadDim);
    const u32x4* gs = reinterpret_cast<const u32x4*>(a.dout + colbase[j] * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 qv = {0, 0, 0, 0}, gv = {0, 0, 0, 0};
      if (ok) {
        qv = qs[4 * ks + g];
        gv = gs[4 * ks + g];
      }
      qf[j][ks] = as_bf16x8(qv);
      gf[j][ks] = as_bf16x8(gv);
    }
    const long long li = ((long long)b * a.Hq + hq) * a.Sq + t;
    lse2[j] = ok ? a.lse[li] * kLog2eB : 0.f;
    dsv[j] = ok ? a.dsum[li] : 0.f;
    pos[j] = ok ? a.q_start + t : -1;
  }
  f32x4 acc[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // first block >= from with a nonzero mask (cmax + 1 if none); same in every wave
  auto next_block = [&](int from) {
    for (int base = from; base <= cmax; base += kWave) {
      const int c = base + lane;
      const uint64_t bal = ballot(c <= cmax && rmask[c] != 0u);
      if (bal != 0ull) return base + (int)__builtin_ctzll(bal);
    }
    return cmax + 1;
  };
  // LDS-bound loads of block c's K and V into tiles bf: load inst writes key
  // rows 4 inst .. 4 inst + 3, lane -> row 4 inst + lane/16, stored chunk lane%16
  auto fetch = [&](int c, u32x4* kdst, u32x4* vdst) {
    const long long off0 = (hb * a.Skv + (long long)c * kBlock) * kHeadDim;
    for (int inst = wave; inst < 16; inst += nwaves) {
      const int slot = inst * kWave + lane;
      const int key = slot >> 4;
      const int ch = (slot & 15) ^ (key & 15);
      const int krow = min(c * kBlock + key, a.Skv - 1) - c * kBlock;  // rows past the cache: masked
      const long long e = off0 + (long long)krow * kHeadDim + 8 * ch;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a.k + e),
                                       (__attribute__((address_space(3))) void*)(kdst + inst * kWave),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a.v + e),
                                       (__attribute__((address_space(3))) void*)(vdst + inst * kWave),
                                       16, 0, 0);
    }
  };
  // block c from tiles (kt, vt)
  auto compute = [&](int c, const u32x4* kt, const u32x4* vt) {
    const uint32_t m = rmask[c];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int grp = 2 * wave + j;
      if (((m >> (grp * RPG)) & ((1u << RPG) - 1u)) == 0u) continue;  // wave-uniform
      const bool wants = (m >> rloc[j]) & 1u;
      f32x4 sv[4], dp[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sv[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = as_bf16x8(kt[swz_slot(16 * mt + n, 4 * ks + g)]);
          const bf16x8 vf = as_bf16x8(vt[swz_slot(16 * mt + n, 4 * ks + g)]);
          sv[mt] = mfma16(kf, qf[j][ks], sv[mt]);
          dp[mt] = mfma16(vf, gf[j][ks], dp[mt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = c * kBlock + 16 * mt + 4 * g + rr;
          const float p = (wants && key <= pos[j])
                              ? exp2f(sv[mt][rr] * a.scale_log2 - lse2[j]) : 0.f;
          sv[mt][rr] = p * (dp[mt][rr] - dsv[j]);
        }
      pv_tr(sv, kt, acc[j]);  // dQ^T += K^T dS^T
    }
  };
  int c = next_block(0);
  if (c <= cmax) fetch(c, ktile0, vtile0);
  while (c <= cmax) {
    // tiles 0 hold block c; block cn goes to tiles 1
    int cn = next_block(c + 1);
    wait_all_loads();
    __syncthreads();  // block c's tiles complete in every wave
    if (cn <= cmax) fetch(cn, ktile1, vtile1);
    compute(c, ktile0, vtile0);
    __syncthreads();  // tiles 0 free for the block after cn
    c = cn;
    if (c > cmax) break;
    // tiles 1 hold block c; block cn goes to tiles 0
    cn = next_block(c + 1);
    wait_all_loads();
    __syncthreads();
    if (cn <= cmax) fetch(cn, ktile0, vtile0);
    compute(c, ktile1, vtile1);
    __syncthreads();  // tiles 1 free for the block after cn
    c = cn;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (rloc[j] < rows) store_tr_f32(acc[j], a.dq + colbase[j] * kHeadDim, a.scale);
}

}  // namespace

namespace {
char* align256(char* p) { return reinterpret_cast<char*>(((uintptr_t)p + 255) & ~(uintptr_t)255); }
}  // namespace

size_t inverse_lists_bytes(const Shape& s) {
  const size_t nbatch = (size_t)ceil_div(s.Sq, kBatchRows);
  size_t bytes = 0;
  bytes += (size_t)s.B * s.Hkv * nbatch * s.nblk * 4;       // batch counts / offsets
  bytes += ((size_t)s.B * s.Hkv * s.nblk + 1) * 4;          // list starts
  bytes += (size_t)s.B * s.Hkv * s.Sq * s.top_k * 4;        // row lists
  return bytes + 3 * 256;                                    // alignment slack
}

hipError_t launch_inverse_lists(const Shape& s, const int32_t* sel, void* ws,
                                const int32_t** base_out, const int32_t** lists_out,
                                hipStream_t st, int32_t* slotpos) {
  const int nbatch = ceil_div(s.Sq, kBatchRows);
  const size_t bm_bytes = (size_t)s.nblk * 8;
  if (bm_bytes > 160 * 1024) return hipErrorInvalidValue;
  char* p = align256(static_cast<char*>(ws));
  int32_t* bcnt = reinterpret_cast<int32_t*>(p);
  p = align256(p + (size_t)s.B * s.Hkv * nbatch * s.nblk * 4);
  int32_t* base = reinterpret_cast<int32_t*>(p);
  p = align256(p + ((size_t)s.B * s.Hkv * s.nblk + 1) * 4);
  int32_t* lists = reinterpret_cast<int32_t*>(p);
  BwdArgs a{};
  a.sel = sel;
  a.bcnt = bcnt;
  a.base = base;
  a.lists = lists;
  a.slotpos = slotpos;
  a.B = s.B;
  a.Sq = s.Sq;
  a.Skv = s.Skv;
  a.q_start = s.q_start;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.top_k = s.top_k;
  a.nblk = s.nblk;
  a.nbatch = nbatch;
  hipError_t e;
  if (bm_bytes > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&inverse_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bm_bytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&inverse_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bm_bytes);
    if (e != hipSuccess) return e;
  }
  inverse_kernel<false><<<dim3(nbatch, s.Hkv, s.B), 256, bm_bytes, st>>>(a);
  batch_scan_kernel<<<dim3(ceil_div(s.nblk, kScanBlocks), s.B * s.Hkv), 256, 0, st>>>(a);
  base_scan_kernel<<<1, 256, 0, st>>>(a);
  inverse_kernel<true><<<dim3(nbatch, s.Hkv, s.B), 256, bm_bytes, st>>>(a);
  *base_out = base;
  *lists_out = lists;
  return hipGetLastError();
}

size_t sparse_bwd_workspace_bytes(const Shape& s) {
  return (size_t)s.B * s.Hq * s.Sq * 4 + 256 + inverse_lists_bytes(s);  // dsum, then the lists
}

hipError_t launch_sparse_attn_backward(const Shape& s, const void* q, const void* k, const void* v,
                                       const int32_t* sel, const void* out, const float* lse,
                                       const void* dout, float* dq, float* dk, float* dv, void* ws,
                                       hipStream_t st) {
  if (s.G > 64 || 64 % s.G != 0) return hipErrorInvalidValue;
  char* p = align256(static_cast<char*>(ws));
  float* dsum = reinterpret_cast<float*>(p);
  p += (size_t)s.B * s.Hq * s.Sq * 4;
  const int32_t* base = nullptr;
  const int32_t* lists = nullptr;
  BwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
            static_cast<const uint16_t*>(v), sel, static_cast<const uint16_t*>(out), lse,
            static_cast<const uint16_t*>(dout), dq, dk, dv, dsum, nullptr, nullptr, nullptr,
            nullptr, s.B, s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, s.G, s.top_k, s.nblk,
            ceil_div(s.Sq, kBatchRows), s.scale, s.scale * kLog2eB};
  const long long nrows = (long long)s.B * s.Sq * s.Hq;
  dsum_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(a);
  hipError_t e = launch_inverse_lists(s, sel, p, &base, &lists, st);
  if (e != hipSuccess) return e;
  a.base = const_cast<int32_t*>(base);
  a.lists = const_cast<int32_t*>(lists);
  if (s.G == 4 || s.G == 8) {
    const size_t dq_lds = (size_t)s.nblk * 4;  // the row masks (the tiles are static)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dq_tile_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dq_lds);
    if (e != hipSuccess) return e;
    const int waves = (kDqTileRows / (16 / s.G)) / 2;  // two row groups per wave
    dq_tile_kernel<<<dim3(ceil_div(s.Sq, kDqTileRows), s.Hkv, s.B), waves * kWave, dq_lds, st>>>(a);
  } else {
    const long long nw = (long long)s.B * s.Hkv * s.Sq;
    dq_kernel<<<(unsigned)((nw + 3) / 4), 256, 0, st>>>(a);
  }
  dkdv_kernel<<<dim3(s.nblk, s.Hkv, s.B), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
