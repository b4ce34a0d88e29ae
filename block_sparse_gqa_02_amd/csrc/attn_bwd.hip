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
// forward's log-sum-exp with v_exp_f32 directly, as the forward forms them
// (weights below 2^-126 flush to zero); Dsum uses the forward's (bf16) output.
//
// Kernels, in launch order:
//   dsum_kernel      Dsum per (sequence, query head, row).
//   inverse kernels  for every (sequence, KV head, block) the ascending list of
//                    rows that selected it: per batch of 64 rows a bitmap over
//                    blocks in LDS (bit i = row i of the batch), counted, scanned
//                    over batches and over blocks, then filled in row order.
//                    Deterministic: no atomics outside LDS bit sets.
//   dq_union_kernel  (groups of 4 or 8 heads) a work-group per 32-row tile
//                    (64 at G = 4) walks the union of the tile's selected
//                    blocks through a ring of LDS slots, each block's K and V
//                    fetched once, the forward's tile-union protocol (only the
//                    waves that want a block wait for it); per block and
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
#include "lds_ring.h"

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
  int spin_limit;        // ring tag polls before a wave gives up (dq_union_kernel)
};

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

// Dsum[b][hq][t] = sum_d dout * out per column (b, t, hq): 16 lanes per
// column, 16 bytes (8 dims) each, summed over the 16 lanes; a thread takes
// kDsumCols columns 16 apart, every load issued before any is used.
constexpr int kDsumCols = 4;
__global__ void __launch_bounds__(256) dsum_kernel(BwdArgs a) {
  const long long ncol = (long long)a.B * a.Sq * a.Hq;
  const int sub = threadIdx.x & 15;  // this lane's 8 dims: 8 sub .. 8 sub + 7
  const long long col0 = (long long)blockIdx.x * (16 * kDsumCols) + (threadIdx.x >> 4);
  u32x4 ov[kDsumCols], gv[kDsumCols];
#pragma unroll
  for (int i = 0; i < kDsumCols; ++i) {
    const long long col = min(col0 + 16 * i, ncol - 1);
    ov[i] = reinterpret_cast<const u32x4*>(a.out + col * kHeadDim)[sub];
    gv[i] = reinterpret_cast<const u32x4*>(a.dout + col * kHeadDim)[sub];
  }
#pragma unroll
  for (int i = 0; i < kDsumCols; ++i) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += bf16_lo(ov[i][k]) * bf16_lo(gv[i][k]) + bf16_hi(ov[i][k]) * bf16_hi(gv[i][k]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);  // within the column's 16 lanes
    const long long col = col0 + 16 * i;
    if (sub == 0 && col < ncol) {
      const int hq = (int)(col % a.Hq);
      const long long bt = col / a.Hq;
      const int t = (int)(bt % a.Sq), b = (int)(bt / a.Sq);
      a.dsum[((long long)b * a.Hq + hq) * a.Sq + t] = s;
    }
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
        const float p = (col_ok && key <= pos) ? __builtin_amdgcn_exp2f(s[mt][rr] * a.scale_log2 - lse2) : 0.f;
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
// 64 at a time ("chunks") from the block's row list, from its end backwards:
// the work-groups resident together then start on the same late rows, whose
// Q and dO some of them find in cache.  Chunk j+1's Q and dO rows
// travel by LDS-bound loads into the second pair of tiles while chunk j is
// computed; the row indices that address them are loaded a chunk earlier.
__global__ void __launch_bounds__(256, 2) dkdv_kernel(BwdArgs a) {
  // Two tile pairs (64 columns x 128 dims of Q and of dO, swz_slot layout),
  // each tile its own LDS object and the chunk loop unrolled by two, so that
  // every access names its tile and the compiler does not make the reads of
  // one pair wait for the LDS-bound loads into the other.
  __shared__ u32x4 qtile0[kBlock * 16], qtile1[kBlock * 16];
  __shared__ u32x4 gtile0[kBlock * 16], gtile1[kBlock * 16];
  __shared__ float clse[2][64], cds[2][64];
  __shared__ int cpos[2][64];
  __shared__ int cpart[2];  // the chunk holds a row the block reaches past
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
  // row of column col in chunk j, which holds list entries (nchunk - 1 - j) R
  // .. + R - 1 (entries past the list repeat its last row; their columns are
  // masked through cpos = -1)
  auto row_of = [&](int j, int col) { return rows[min((nchunk - 1 - j) * R + col / a.G, len - 1)]; };
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
  // the parts of the staging addresses that do not change from chunk to
  // chunk: the sequence's Q and dO, each slot's head and chunk offset within
  // a row, and the column's (sequence, head) row of the LSE and Dsum
  const long long seq_elems = (long long)b * a.Sq * a.Hq * kHeadDim;
  const uint16_t* qseq = a.q + seq_elems;
  const uint16_t* gseq = a.dout + seq_elems;
  const int rstride = a.Hq * kHeadDim;  // elements per query row
  int coff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) coff[t] = (h * a.G + colt[t] % a.G) * kHeadDim + 8 * cht[t];
  const long long lrow = ((long long)b * a.Hq + h * a.G + lane % a.G) * a.Sq;
  auto stage = [&](int j, u32x4* qdst, u32x4* gdst) {  // chunk j's loads (rows in rt / rmeta)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const long long e = (long long)rt[t] * rstride + coff[t];
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(qseq + e),
                                       (__attribute__((address_space(3))) void*)(qdst + 64 * (4 * wave + t)),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gseq + e),
                                       (__attribute__((address_space(3))) void*)(gdst + 64 * (4 * wave + t)),
                                       16, 0, 0);
    }
    mok = (nchunk - 1 - j) * R + lane / a.G < len;
    mrow = rmeta;
    ml = a.lse[lrow + rmeta];
    md = a.dsum[lrow + rmeta];
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
    if (tid < 64) {  // wave 0, one lane per column; a column past the list gets P = 0
      clse[bf][tid] = mok ? ml * kLog2eB : __builtin_huge_valf();
      cds[bf][tid] = mok ? md : 0.f;
      cpos[bf][tid] = mok ? a.q_start + mrow : -1;
      const uint64_t part = ballot(mok && a.q_start + mrow < c * kBlock + kBlock - 1);
      if (tid == 0) cpart[bf] = part != 0ull;
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
    if (!cpart[bf] && nkeys == 16) {  // every key of the wave attended by every row
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int col = 16 * mt + 4 * g + rr;
          const float p = __builtin_amdgcn_exp2f(x[mt][rr] * a.scale_log2 - clse[bf][col]);
          x[mt][rr] = p;                              // P (columns x keys)
          y[mt][rr] = p * (y[mt][rr] - cds[bf][col]);  // dS
        }
    } else {
      // (the metadata is read before the mask is applied, so that the reads
      // are not each put behind a branch)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int col = 16 * mt + 4 * g + rr;
          const float ls = clse[bf][col], ds = cds[bf][col];
          const int cp = cpos[bf][col];
          const float e = __builtin_amdgcn_exp2f(x[mt][rr] * a.scale_log2 - ls);
          const float p = (n < nkeys && key <= cp) ? e : 0.f;
          x[mt][rr] = p;
          y[mt][rr] = p * (y[mt][rr] - ds);
        }
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

// dQ, ring schedule (groups of 4 or 8 query heads).  A work-group of eight
// waves owns TR = 32 (G = 8) or 64 (G = 4) consecutive rows of one (sequence,
// KV head): 16 row groups of 16/G rows x G heads (the 16 MFMA columns), wave w
// owning groups w and w + 8 with their Q, dO and dQ accumulators in
// registers.  Per window of kDqWin blocks the work-group builds the row and
// row-group bitmasks of every block from the rows' selections and walks the
// union in ascending order; each block's K and V (32 KiB) are fetched once
// into a ring of kDqRing LDS slots by LDS-bound buffer loads.  The ring runs
// the forward's tile-union protocol: only the waves owning a group that wants
// a block wait for its slot's tag, compute and count themselves done; the
// last of them refills the slot with the entry kDqRing ahead, and an LDS-bound
// load of the entry number after the data publishes the tag.  Per block and
// wanting group: S^T = K Q^T, dP^T = V dO^T, P from the saved log-sum-exp
// (0 for a column whose row did not pick the block and for keys after the
// row), dS = P (dP - Dsum), dQ^T += K^T dS^T (pv_tr on the K slot).  A group
// takes its blocks in ascending order, as a row's own list does.  Every tag
// wait is bounded (the library's wait limit): a work-group that gives up
// stores NaN for its rows' dq.
constexpr int kDqWaves = 8;
constexpr int kDqRing = 4;
constexpr int kDqWin = 512;  // blocks per union window
static_assert(kDqWin <= kRingEntries, "ring tags cover a window");

template <int G>
__global__ void __launch_bounds__(kDqWaves * kWave, 1) dq_union_kernel(BwdArgs a) {
  constexpr int RPG = 16 / G;           // rows per group
  constexpr int kNG = 2 * kDqWaves;     // row groups per tile
  constexpr int TR = kNG * RPG;         // rows per tile
  constexpr int NWR = (TR + 31) / 32;   // row-mask words per block
  constexpr int kBlockBytes = kBlock * kHeadDim * 2;
  __shared__ u32x4 ktile[kDqRing][kBlock * 16];
  __shared__ u32x4 vtile[kDqRing][kBlock * 16];
  __shared__ uint32_t rmask[kDqWin][NWR];  // per block: tile rows that picked it
  __shared__ uint32_t gmask[kDqWin];       // per block: row groups that picked it
  __shared__ int32_t ulist[kDqWin];        // union entries: block | (waves wanting it) << 24
  __shared__ int32_t wcount[kDqWaves];
  __shared__ int32_t ready[kDqRing];       // union entry held by each slot
  __shared__ int32_t done[kDqRing];        // waves finished with the slot's entry
  __shared__ int32_t failed;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // scalar (LDS destinations in M0)
  const int n = lane % 16, g = lane / 16;
  const int tile = (int)gridDim.x - 1 - (int)blockIdx.x;  // late (long) tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int t0 = tile * TR;
  const int rows = min(TR, a.Sq - t0);
  const int pos0 = a.q_start + t0;
  const int pos_last = pos0 + rows - 1;
  const int cur_last = pos_last / kBlock;
  const long long hb = (long long)b * a.Hkv + h;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + hb * a.Skv * kHeadDim), (short)0, a.Skv * kHeadDim * 2, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v + hb * a.Skv * kHeadDim), (short)0, a.Skv * kHeadDim * 2, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rtag = __builtin_amdgcn_make_buffer_rsrc(
      (void*)&kEntryIds, (short)0, (int)sizeof(kEntryIds), kRsrcFlags);
  const int32_t* selh = a.sel + (hb * a.Sq + t0) * a.top_k;
  const int rr = n / G, hh = n % G;  // this lane's column: row in group, head

  // owned groups gi = wave + 8j: this lane's column in each
  bf16x8 qf[2][4], gf[2][4];
  float lse2[2], dsv[2];
  int pos[2];
  long long colbase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (wave + kDqWaves * j) * RPG + rr;
    const bool ok = row < rows;
    const int t = t0 + (ok ? row : 0), hq = h * G + hh;
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
  if (tid == 0) failed = 0;

  // Slot fill: instruction j of a block's K (or V) covers key rows 4j..4j+3,
  // lane -> row 4j + lane/16, LDS chunk lane%16, which holds the row's chunk
  // (lane%16) ^ (row & 15) (the swz_slot layout; the lane's offset depends on
  // j mod 4 only).  The diagonal block re-reads its last used row in place of
  // later ones (masked keys, kept finite).
  auto koff = [&](int jm) {
    return (lane / 16) * 256 + 16 * ((lane % 16) ^ kswz(4 * jm + lane / 16));
  };
  auto fetch_rows = [&](int c, int sl, int j0, int j1) {
    const int sb = c * kBlockBytes;
    const int last = min(pos_last - c * kBlock, kBlock - 1);
    for (int j = j0; j < j1; ++j) {
      const int row = 4 * j + lane / 16, srow = min(row, last);
      const int off = srow * 256 + 16 * ((lane % 16) ^ kswz(row));
      load_lds16(rk, &ktile[sl][j * kWave], off, sb);
      load_lds16(rv, &vtile[sl][j * kWave], off, sb);
    }
  };
  auto fetch_full = [&](int c, int sl) {
    const int sb = c * kBlockBytes;
    if (c * kBlock + kBlock - 1 <= pos_last) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int off = koff(j & 3);
        load_lds16(rk, &ktile[sl][j * kWave], off, sb + j * 1024);
        load_lds16(rv, &vtile[sl][j * kWave], off, sb + j * 1024);
      }
    } else {
      fetch_rows(c, sl, 0, 16);
    }
  };

  // block c from slot sl for the wave's groups that want it
  auto compute = [&](int sl, int c, uint32_t gm, const uint32_t* rm) {
    const u32x4* kt = &ktile[sl][0];
    const u32x4* vt = &vtile[sl][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gi = wave + kDqWaves * j;
      if (!((gm >> gi) & 1u)) continue;  // wave-uniform
      const int row = gi * RPG + rr;
      const bool wants = (rm[row / 32] >> (row % 32)) & 1u;
      // the lane's operand bytes in a slot: row 16 mt + n, chunk 4 ks + g at
      // swz_slot, i.e. 4096 mt + kb[ks]
      uint32_t kb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kb[ks] = 256u * n + 16u * ((4 * ks + g) ^ n);
        asm volatile("" : "+v"(kb[ks]));
      }
      f32x4 sv[4], dp[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sv[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = as_bf16x8(lds_u32x4_at(kt, kb[ks] + 4096 * mt));
          const bf16x8 vf = as_bf16x8(lds_u32x4_at(vt, kb[ks] + 4096 * mt));
          sv[mt] = mfma16(kf, qf[j][ks], sv[mt]);
          dp[mt] = mfma16(vf, gf[j][ks], dp[mt]);
        }
      }
      // a column whose row did not pick the block gets P = 0 through an
      // infinite log-sum-exp; the key mask is needed only where the block
      // reaches past a column's row
      const float lsew = wants ? lse2[j] : __builtin_huge_valf();
      if (ballot(c * kBlock + kBlock - 1 <= pos[j]) == ~0ull) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(sv[mt][r] * a.scale_log2 - lsew);
            sv[mt][r] = p * (dp[mt][r] - dsv[j]);
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = c * kBlock + 16 * mt + 4 * g + r;
            const float p = key <= pos[j] ? __builtin_amdgcn_exp2f(sv[mt][r] * a.scale_log2 - lsew) : 0.f;
            sv[mt][r] = p * (dp[mt][r] - dsv[j]);
          }
      }
      pv_tr(sv, kt, acc[j]);  // dQ^T += K^T dS^T
    }
  };

  bool ok_run = true;
  for (int wb = 0; wb <= cur_last && ok_run; wb += kDqWin) {
    const int we = min(wb + kDqWin, cur_last + 1);
    // 1. row and group bitmasks of the window's blocks
    for (int x = tid; x < kDqWin * NWR; x += kDqWaves * kWave) (&rmask[0][0])[x] = 0u;
    for (int x = tid; x < kDqWin; x += kDqWaves * kWave) gmask[x] = 0u;
    if (tid < kDqRing) {
      ready[tid] = -1;
      done[tid] = 0;
    }
    __syncthreads();
    {
      constexpr int parts = kDqWaves * kWave / TR;
      const int row = tid % TR, part = tid / TR;
      if (row < rows) {
        const int cur = (pos0 + row) / kBlock;
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
    // 2. union list of the window, ascending, with the waves that want each entry
    int nu = 0;
    for (int j = 0; j < kDqWin; j += kDqWaves * kWave) {
      const int pidx = j + tid;
      const uint32_t gmv = pidx < we - wb ? gmask[pidx] : 0u;
      const bool nz = gmv != 0u;
      const uint64_t bal = ballot(nz);
      if (lane == 0) wcount[wave] = __popcll(bal);
      __syncthreads();
      int before = nu;
      for (int w = 0; w < wave; ++w) before += wcount[w];
      if (nz) {
        const uint32_t wbits = (gmv | (gmv >> kDqWaves)) & 0xffu;
        ulist[before + prefix_count(bal)] = (wb + pidx) | (int)(wbits << 24);
      }
#pragma unroll
      for (int w = 0; w < kDqWaves; ++w) nu += wcount[w];
      __syncthreads();
    }
    // 3. first kDqRing entries: every wave moves 2 of the 16 instructions of each
    for (int s = 0; s < kDqRing && s < nu; ++s)
      fetch_rows(ulist[s] & 0xffffff, s, 2 * wave, 2 * wave + 2);
    wait_vm(0);
    __syncthreads();
    if (tid < kDqRing && tid < nu) ready[tid] = tid;
    __syncthreads();
    // 4. decoupled sweep over the entries this wave wants
    for (int u0 = 0; u0 < nu && ok_run; u0 += kWave) {
      const int ue = u0 + lane < nu ? ulist[u0 + lane] : 0;
      uint64_t mine = ballot(u0 + lane < nu && ((ue >> (24 + wave)) & 1));
      while (mine != 0ull) {
        const int bit = __builtin_ctzll(mine);
        mine &= mine - 1;
        const int u = u0 + bit;
        const int e = __builtin_amdgcn_readlane(ue, bit);
        const int c = e & 0xffffff;
        const int need = __builtin_popcount((uint32_t)e >> 24);
        const int sl = u % kDqRing;
        // a wave's LDS operations complete in order, so once the tag reads u
        // the slot's data reads below see the block
        if (lds_load_tag(&ready[sl]) != u) {
          int spins = 0;
          while (lds_load_tag(&ready[sl]) != u) {
            if (++spins > a.spin_limit) {
              ok_run = false;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
          if (!ok_run) {
            if (lane == 0) failed = 1;
            break;
          }
        }
        // the wave holding a slot issues ahead of its SIMD's other wave until
        // its refill (if it is the last wanting wave) has gone out
        cbarrier();
        __builtin_amdgcn_s_setprio(2);
        compute(sl, c, gmask[c - wb], rmask[c - wb]);
        cbarrier();
        int prev = 0;
        if (lane == 0) prev = lds_fetch_add_tag(&done[sl], 1);
        prev = __builtin_amdgcn_readfirstlane(prev);
        if (prev == need - 1) {
          // the count is reset before the loads are issued; the tag that lets
          // the next entry's waves in is written after the block's data
          if (lane == 0) lds_store_tag(&done[sl], 0);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (u + kDqRing < nu) {
            fetch_full(ulist[u + kDqRing] & 0xffffff, sl);
            if (lane == 0)
              __builtin_amdgcn_raw_ptr_buffer_load_lds(rtag, (lds_ptr)&ready[sl], 4, 0,
                                                       (u + kDqRing) * 4, 0, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    wait_vm(0);
    __syncthreads();
    if (failed) ok_run = false;
  }
  // a failed sweep (bounded wait exceeded) stores NaN so the caller sees it
  const float mul = ok_run ? a.scale : __builtin_nanf("");
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if ((wave + kDqWaves * j) * RPG + rr < rows) store_tr_f32(acc[j], a.dq + colbase[j] * kHeadDim, mul);
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
  dsum_kernel<<<(unsigned)((nrows + 16 * kDsumCols - 1) / (16 * kDsumCols)), 256, 0, st>>>(a);
  hipError_t e = launch_inverse_lists(s, sel, p, &base, &lists, st);
  if (e != hipSuccess) return e;
  a.base = const_cast<int32_t*>(base);
  a.lists = const_cast<int32_t*>(lists);
  if (s.G == 4 || s.G == 8) {
    // the buffer descriptors address one head's K or V with 32-bit byte offsets
    if ((long long)s.Skv * kHeadDim * 2 > 0x7fffffffLL) return hipErrorInvalidValue;
    a.spin_limit = union_spin_limit();
    const int TR = 2 * kDqWaves * (16 / s.G);
    const dim3 grid(ceil_div(s.Sq, TR), s.Hkv, s.B);
    if (s.G == 8) dq_union_kernel<8><<<grid, kDqWaves * kWave, 0, st>>>(a);
    else dq_union_kernel<4><<<grid, kDqWaves * kWave, 0, st>>>(a);
  } else {
    const long long nw = (long long)s.B * s.Hkv * s.Sq;
    dq_kernel<<<(unsigned)((nw + 3) / 4), 256, 0, st>>>(a);
  }
  dkdv_kernel<<<dim3(s.nblk, s.Hkv, s.B), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
