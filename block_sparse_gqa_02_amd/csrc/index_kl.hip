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
// Every step runs block-stationary: each selected (sequence, KV head, block)
// is read once, by the work-group that owns the block, for every row that
// selected it, and per-row results are gathered from per-(list entry) partials
// in slot order.  Kernels, in launch order:
//   inverse lists        (shared with the main-branch gradient) the ascending
//                        rows that selected each (sequence, KV head, block),
//                        and the list position of every selection entry.
//   kl_lse_kernel        per (list entry, index head), over the block's keys
//                        the row attends: the max of the index scores and the
//                        sum of 2^(s - max).
//   kl_lse_t_kernel      the forward's log-sum-exp in (row, query head) order.
//   kl_lse_merge_kernel  the index log-sum-exp per (row, index head), its
//                        entries combined in a fixed order.
//   kl_entry_kernel      per 16 rows of a block's list: P from the forward's
//                        log-sum-exp, Q from the index log-sum-exp, C = Q - P;
//                        per (list entry, index head) the loss partial, the
//                        diq partial (sums over the block's keys) and C itself
//                        per key.  Long lists are split over work-groups.
//   kl_dik_kernel        per key of the block, dik = the sum of C iq over the
//                        block's (list entry, index head) pairs, long lists
//                        split over work-groups.
//   kl_dik_merge_kernel  dik of split blocks, partials added in split order.
//   kl_merge_kernel      loss and diq per (row, index head), partials added in
//                        slot order.
// Nothing uses floating-point atomics: results are bit-identical from call to
// call.  Products take bf16 operands (C rounded to bf16) with fp32
// accumulation; softmax statistics are fp32.
#include "bwd_tiles.h"
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
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
  const uint16_t* q;       // [B][Sq][Hq][128]
  const uint16_t* k;       // [B][Hkv][Skv][128]
  const uint16_t* iq;      // [B][Sq][4][64]
  const uint16_t* ik;      // [B][Skv][64]
  const int32_t* sel;      // [B][Hkv][Sq][top_k]
  const float* lse;        // [B][Hq][Sq], natural log
  float* loss;             // [B][Sq][4]
  float* diq;              // [B][Sq][4][64]
  float* dik;              // [B][Skv][64]
  float* lse_idx;          // workspace [B][4][Sq]: index log-sum-exp, log2 domain
  float* lse_t;            // workspace [B][Sq][Hq]: the forward's log-sum-exp, log2 domain
  float* dikp;             // workspace [B][nblk][kKeySplits][64][64]: split partials of dik
  const int32_t* slotpos;  // workspace [B][Hkv][Sq][top_k]: list position of an entry, or -1
  f32x2* part_ml;          // workspace [entries][nih]: block max and sum (log2 domain)
  float* part_q;           // workspace [entries][nih][64]: diq partials
  float* part_l;           // workspace [entries][nih]: loss partials
  uint16_t* cbuf;          // workspace [entries][nih][64]: C = Q - P (bf16) per key of the block
  const int32_t* base;     // inverse lists: starts per (sequence, KV head, block), then the total
  const int32_t* lists;    // rows
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
  int tb = r15 * 128 + 8 * (n & 1);  // byte offset in the tile
  asm volatile("" : "+v"(tb));  // opaque: a caller's loop keeps no per-tile address registers
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
      const uint32_t va = (uint32_t)tb + (uint32_t)(32 * kv * 128) + 16 * ch;
      const s16x4 lo = lds_read_tr_at(tile, va);
      const s16x4 hi = lds_read_tr_at(tile, va + 16 * 128);
      const bf16x8 tf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[mt] = mfma16(tf, pb, acc[mt]);
    }
  }
}

__device__ __forceinline__ float max16(const f32x4 (&v)[4]) {
  float m = v[0][0];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmax_nn(m, v[mt][r]);
  return m;
}

// Work-group setup shared by the two block passes: every KV head's list for
// block c (start, length and job count, jobs of `per` rows, in LDS) and the
// block's 64 index keys in LDS (islot layout; rows past the cache repeat the
// last key, masked by position).  Leaves the index-key loads in flight.
__device__ __forceinline__ void block_setup(const KlArgs& a, int b, int c, int per, int* lbeg,
                                            int* llen, int* lnj, u32x4* itile) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  if (tid < 4) {
    const bool hv = tid < a.Hkv;
    const long long e = ((long long)b * a.Hkv + (hv ? tid : 0)) * a.nblk + c;
    const int bg = hv ? a.base[e] : 0;
    const int ln = hv ? a.base[e + 1] - bg : 0;
    lbeg[tid] = bg;
    llen[tid] = ln;
    lnj[tid] = (ln + per - 1) / per;
  }
  for (int inst = wave; inst < 8; inst += 4) {  // 8 loads of 64 lanes cover the 8 KiB
    const int slot = inst * kWave + lane;
    const int key = slot >> 3, ch = (slot & 7) ^ (key & 7);
    const int krow = min(c * kBlock + key, a.Skv - 1);
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const void*>(a.ik + ((long long)b * a.Skv + krow) * kIdxDim + 8 * ch),
        (__attribute__((address_space(3))) void*)(itile + inst * kWave), 16, 0, 0);
  }
}

// (KV head, job) of job j < the block's total, jobs in (head, job) order.
__device__ __forceinline__ int job_head(const int* lnj, int j, int& q) {
  int h = 0;
  while (h < 3 && j >= lnj[h]) {
    j -= lnj[h];
    ++h;
  }
  q = j;
  return h;
}

// Pass A: the index log-sum-exp, block by block.  Work-group (block, sequence,
// split); every wave takes jobs of 16 index columns on its own (no barriers
// after the setup): job q of KV head h is rows q 16/nih .. of h's list, lane
// column n = (row n / nih, index head h + Hkv (n % nih)).  S^T = iK iQ^T over
// the block's 64 keys gives, per column, the max and the sum of 2^(s - max)
// over the keys the row attends, stored per (list entry, index head).
template <int G>
__global__ void __launch_bounds__(256) kl_lse_kernel(KlArgs a) {
  __shared__ u32x4 itile[kBlock * 8];
  __shared__ int lbeg[4], llen[4], lnj[4];
  const int c = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const int nih = a.nih, rpj = 16 / nih;
  block_setup(a, b, c, rpj, lbeg, llen, lnj, itile);
  wait_all_loads();
  __syncthreads();
  const int total = lnj[0] + lnj[1] + lnj[2] + lnj[3];
  const int nsplit = key_splits(total);
  if (split >= nsplit) return;
  const int j0 = (int)((long long)split * total / nsplit);
  const int j1 = (int)((long long)(split + 1) * total / nsplit);
  const int rr = n / nih, m = n % nih;
  if (j0 + wave >= j1) return;  // wave-uniform, and no barrier follows
  // Jobs run as a pipeline: the list entry two jobs ahead and the index query
  // row of the next job are loaded before the current job's products.  Loads
  // of jobs past the split, or of rows past a list's end, read a clamped
  // address; such columns are masked when the scores are formed.
  auto entry = [&](int j) {
    int q;
    const int h = job_head(lnj, min(j, j1 - 1), q);
    return lbeg[h] + min(q * rpj + rr, llen[h] - 1);
  };
  auto query = [&](int t, int h, bf16x8 (&f)[2]) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.iq + (((long long)b * a.Sq + t) * kIdxHeads + h + a.Hkv * m) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) f[ks] = as_bf16x8(src[4 * ks + g]);
  };
  int t_cur = a.lists[entry(j0 + wave)];
  int t_nxt = a.lists[entry(j0 + wave + 4)];
  bf16x8 iqf[2];
  {
    int q;
    query(t_cur, job_head(lnj, j0 + wave, q), iqf);
  }
  for (int j = j0 + wave; j < j1; j += 4) {
    int q;
    const int h = job_head(lnj, j, q);
    const int li = q * rpj + rr;  // the column's row: entry li of h's list
    const bool ok = li < llen[h];
    const int t = t_cur;
    const int t_far = a.lists[entry(j + 8)];
    bf16x8 iqn[2];
    {
      int qn;
      query(t_nxt, job_head(lnj, min(j + 4, j1 - 1), qn), iqn);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the next job's loads ahead of this job's products
    const int pos = a.q_start + t;
    f32x4 si[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      si[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        si[mt] = mfma16(as_bf16x8(itile[islot(16 * mt + n, 4 * ks + g)]), iqf[ks], si[mt]);
    }
    // max and sum over the keys each column attends: the max is taken on
    // the raw scores and then scaled (the scale is positive and rounding is
    // monotone, so this is the max of the scaled scores), each term
    // 2^(s scale - max) with one fused multiply-add.  Jobs whose columns are
    // all real rows attending the whole block skip the masks.
    const bool full = ballot(ok && c * kBlock + kBlock - 1 <= pos) == ~0ull;
    if (!full) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = c * kBlock + 16 * mt + 4 * g + r;
          if (!(ok && key <= pos)) si[mt][r] = -__builtin_huge_valf();
        }
    }
    const float mx = wave_max_xor16_32(max16(si)) * kLog2eB;
    float l = 0.f;
    if (full) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) l += __builtin_amdgcn_exp2f(__builtin_fmaf(si[mt][r], kLog2eB, -mx));
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          l += si[mt][r] != -__builtin_huge_valf()
                   ? __builtin_amdgcn_exp2f(__builtin_fmaf(si[mt][r], kLog2eB, -mx)) : 0.f;
    }
    l = wave_sum_xor16_32(l);
    if (ok && g == 0) a.part_ml[(long long)(lbeg[h] + li) * nih + m] = f32x2{mx, l};
    t_cur = t_nxt;
    t_nxt = t_far;
    iqf[0] = iqn[0];
    iqf[1] = iqn[1];
  }
}

// (max, sum) pairs of the log2-domain softmax: B merged into A.
__device__ __forceinline__ void merge_ml(float& M, float& L, float M2, float L2) {
  if (!(L2 > 0.f)) return;
  if (!(L > 0.f)) {
    M = M2;
    L = L2;
  } else if (M2 > M) {
    L = L * exp2f(M - M2) + L2;
    M = M2;
  } else {
    L += L2 * exp2f(M2 - M);
  }
}

// The index log-sum-exp of every (row, index head): its entries' block
// partials combined in a fixed order.
__global__ void __launch_bounds__(256) kl_lse_merge_kernel(KlArgs a) {
  // 16 lanes per (row, index head): lane l merges slots l, l + 16, l + 32, ...
  // in that order (the slot positions read 16 at a time, every load of a
  // batch issued first), then the 16 lanes' pairs are merged by xor steps 1,
  // 2, 4, 8 (both lanes of a step form the same sum: deterministic)
  const long long x = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;  // (b * 4 + i) * Sq + t
  const int l = threadIdx.x & 15;
  const long long nx = (long long)a.B * kIdxHeads * a.Sq;
  const long long xc = x < nx ? x : nx - 1;
  const int t = (int)(xc % a.Sq);
  const long long bi = xc / a.Sq;
  const int i = (int)(bi % kIdxHeads), b = (int)(bi / kIdxHeads);
  const int h = i % a.Hkv, m = i / a.Hkv;
  const int32_t* sp = a.slotpos + (((long long)b * a.Hkv + h) * a.Sq + t) * a.top_k;
  float M = -__builtin_huge_valf(), L = 0.f;
  for (int s0 = 0; s0 < a.top_k; s0 += 64) {
    int ev[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ev[r] = sp[min(s0 + l + 16 * r, a.top_k - 1)];
    f32x2 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = a.part_ml[(long long)max(ev[r], 0) * a.nih + m];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (s0 + l + 16 * r < a.top_k && ev[r] >= 0) merge_ml(M, L, v[r][0], v[r][1]);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float M2 = __shfl_xor(M, o), L2 = __shfl_xor(L, o);
    merge_ml(M, L, M2, L2);
  }
  if (x < nx && l == 0) a.lse_idx[x] = L > 0.f ? M + __log2f(L) : -__builtin_huge_valf();
}

// The forward's log-sum-exp in (row, query head) order and the log2 domain,
// so that a row's heads are one contiguous read.  One thread per element.
__global__ void __launch_bounds__(256) kl_lse_t_kernel(KlArgs a) {
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;  // (b * Sq + t) * Hq + hq
  if (x >= (long long)a.B * a.Sq * a.Hq) return;
  const int hq = (int)(x % a.Hq);
  const long long bt = x / a.Hq;
  const int t = (int)(bt % a.Sq), b = (int)(bt / a.Sq);
  a.lse_t[x] = a.lse[((long long)b * a.Hq + hq) * a.Sq + t] * kLog2eB;
}

// Pass B1: everything a (list entry, index head) needs from one block.
// Work-group (block, sequence, split); the block's K for one KV head at a time
// and its index keys sit in LDS, and every wave takes jobs of 16 rows of a KV
// head's list on its own, in two phases.
//  1. The rows' main-branch weights, G column groups of 16/G rows x G query
//     heads: S = Q K^T with the query heads on the M side, so a lane holds
//     four heads of one row for one key; P, the mean over the G heads of
//     2^(s scale - lse), is a sum over the lane's registers plus, for G > 4,
//     over the lanes of the other 16-lane rows holding the same row.  P of
//     the 16 rows goes to a wave-private LDS tile.
//  2. Per index head of the KV head, the 16 rows' index scores S^T = iK iQ^T
//     (a row per column): Q = 2^(s - lse), C = Q - P (rounded to bf16), over
//     the block's keys the loss partial sum P (log P - log Q) and the diq
//     partial sum C ik (one MFMA product over the index-key tile).  C itself
//     is stored for the dik pass.
template <int G>
__global__ void __launch_bounds__(256, 2) kl_entry_kernel(KlArgs a) {
  constexpr int RPG = 16 / G;  // rows per main-branch column group
  constexpr int HQ4 = G / 4;   // 16-lane rows that hold the same query row in phase 1
  constexpr int kJob = 16;     // rows per job
  __shared__ u32x4 ktile[kBlock * 16];  // the block's K for the current KV head, swz_slot layout
  __shared__ u32x4 itile[kBlock * 8];   // the block's index keys, islot layout
  __shared__ f32x4 ptile[4][kJob][kBlock / 4 + 1];  // per wave: P of the job's rows, (row, key)
  __shared__ int lbeg[4], llen[4], lnj[4];
  const int c = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const int nih = a.nih;
  block_setup(a, b, c, kJob, lbeg, llen, lnj, itile);
  wait_all_loads();
  __syncthreads();
  const int total = lnj[0] + lnj[1] + lnj[2] + lnj[3];
  const int nsplit = key_splits(total);
  if (split >= nsplit) return;
  const int j0 = (int)((long long)split * total / nsplit);
  const int j1 = (int)((long long)(split + 1) * total / nsplit);
  const float invG = 1.f / (float)G;
  const int key0 = c * kBlock;
  f32x4* pw = &ptile[wave][0][0];
  int hstart = 0;  // first job of KV head h
  for (int h = 0; h < a.Hkv; hstart += lnj[h], ++h) {
    const int hj0 = max(j0, hstart), hj1 = min(j1, hstart + lnj[h]);
    if (hj0 >= hj1) continue;  // uniform over the work-group
    __syncthreads();           // every read of the previous head's K is done
    {
      const long long koff = (((long long)b * a.Hkv + h) * a.Skv + (long long)key0) * kHeadDim;
      for (int inst = wave; inst < 16; inst += 4) {
        const int slot = inst * kWave + lane;
        const int kk = slot >> 4, ch = (slot & 15) ^ (kk & 15);
        const int krow = min(key0 + kk, a.Skv - 1) - key0;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(a.k + koff + (long long)krow * kHeadDim + 8 * ch),
            (__attribute__((address_space(3))) void*)(ktile + inst * kWave), 16, 0, 0);
      }
    }
    wait_all_loads();
    __syncthreads();
    const float* lse_h = a.lse_t + h * G + 4 * (g % HQ4);  // + (b Sq + t) Hq: heads of lane's M rows
    // rows of job j: entries (j - hstart) 16 .. +15 of h's list; lane n < 16
    // holds the row of entry n (-1 past the list)
    auto job_rows = [&](int j) {
      const int li = (j - hstart) * kJob + n;
      return (lane < 16 && li < llen[h]) ? a.lists[lbeg[h] + li] : -1;
    };
    // phase-1 operands of column group u: Q of row u RPG + n / G, head n % G
    // (A operand), and the log2-domain LSE of the lane's four output heads.
    // Two register sets: groups u and u + 1 are in flight while u - 1 is
    // computed.  The loads are unconditional (row 0 stands in for a missing
    // row, whose P the key mask zeroes: lim = -1): a load under a branch, or
    // a value selected right after its load, would make the wave wait for the
    // load at once.
    bf16x8 qa[4], qb[4];
    f32x4 lsea, lseb;
    auto load_group = [&](int tl, int u, bf16x8 (&qn)[4], f32x4& lsen) {
      const int ta = __shfl(tl, u * RPG + n / G);
      const int to = __shfl(tl, u * RPG + (4 * g) / G);
      const long long ba = (long long)b * a.Sq + (ta >= 0 ? ta : 0);
      const u32x4* qs = reinterpret_cast<const u32x4*>(a.q + (ba * a.Hq + h * G + n % G) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qn[ks] = as_bf16x8(qs[4 * ks + g]);
      lsen = *reinterpret_cast<const f32x4*>(lse_h + ((long long)b * a.Sq + (to >= 0 ? to : 0)) * a.Hq);
    };
    int tl = hj0 + wave < hj1 ? job_rows(hj0 + wave) : -1;
    if (hj0 + wave < hj1) {
      load_group(tl, 0, qa, lsea);
      load_group(tl, 1, qb, lseb);
    }
    for (int j = hj0 + wave; j < hj1; j += 4) {
      const int tnext = j + 4 < hj1 ? job_rows(j + 4) : -1;
      const bool more = j + 4 < hj1;
      // ---- phase 1: P of the job's 16 rows into the wave's LDS tile
      // group u from set a (u even) or b (u odd); once its products are
      // issued the set is refilled with group u + 2, of this job or the next
      auto group = [&](int u, bf16x8 (&qn)[4], f32x4& lsen) {
        const int to = __shfl(tl, u * RPG + (4 * g) / G);
        f32x4 sv[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          sv[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            sv[mt] = mfma16(qn[ks], as_bf16x8(ktile[swz_slot(16 * mt + n, 4 * ks + g)]), sv[mt]);
        }
        const f32x4 lse2 = lsen;
        if (u + 2 < G) load_group(tl, u + 2, qn, lsen);
        else if (more) load_group(tnext, u + 2 - G, qn, lsen);
        // lane (n, g): register r of sv[mt] is head 4 (g % HQ4) + r of row
        // u RPG + 4g / G for key 16mt + n
        const int lim = to >= 0 ? a.q_start + to - key0 : -1;  // last attended key of the block
        float ps[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          float s = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) s += __builtin_amdgcn_exp2f(sv[mt][r] * a.scale_log2 - lse2[r]);
          ps[mt] = s;
        }
        if constexpr (HQ4 >= 2) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps[mt]), __float_as_uint(ps[mt]), false, false);
            ps[mt] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          }
        }
        if constexpr (HQ4 >= 4) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps[mt]), __float_as_uint(ps[mt]), false, false);
            ps[mt] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          }
        }
        // the HQ4 lanes of a (row, key) hold the same P: lane g writes the
        // key tiles mt with mt % HQ4 == g % HQ4
        float* prow = reinterpret_cast<float*>(pw + (u * RPG + (4 * g) / G) * (kBlock / 4 + 1));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (mt % HQ4 == g % HQ4) prow[16 * mt + n] = 16 * mt + n <= lim ? ps[mt] * invG : 0.f;
      };
#pragma unroll
      for (int u = 0; u < G; u += 2) {
        group(u, qa, lsea);
        group(u + 1, qb, lseb);
      }
      __builtin_amdgcn_wave_barrier();
      // ---- phase 2: per index head, the rows' index scores, C, loss and diq
      const int tn = __shfl(tl, n);  // row of column n
      const int limn = tn >= 0 ? a.q_start + tn - key0 : -1;
      const long long ebase = (long long)lbeg[h] + (long long)(j - hstart) * kJob + n;  // list entry of column n
      f32x4 pr[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) pr[mt] = pw[n * (kBlock / 4 + 1) + 4 * mt + g];
      for (int m = 0; m < nih; ++m) {
        const int i = h + a.Hkv * m;
        const long long bt = (long long)b * a.Sq + (tn >= 0 ? tn : 0);
        const u32x4* is = reinterpret_cast<const u32x4*>(a.iq + (bt * kIdxHeads + i) * kIdxDim);
        bf16x8 iqf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 v = {0, 0, 0, 0};
          if (tn >= 0) v = is[4 * ks + g];
          iqf[ks] = as_bf16x8(v);
        }
        const float ilse2 = tn >= 0 ? a.lse_idx[((long long)b * kIdxHeads + i) * a.Sq + tn] : 0.f;
        f32x4 si[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          si[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            si[mt] = mfma16(as_bf16x8(itile[islot(16 * mt + n, 4 * ks + g)]), iqf[ks], si[mt]);
        }
        // lane (n, g): register r of si[mt] is key 16mt + 4g + r of row n
        float lsum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool att = 16 * mt + 4 * g + r <= limn;
            const float p = pr[mt][r];  // 0 where not attended
            const float s2 = si[mt][r] * kLog2eB;
            // v_exp_f32 / v_log_f32 directly: results below the normal
            // range flush to zero, and the log term skips P < 1e-30 (each
            // such term is below 1e-28)
            si[mt][r] = att ? __builtin_amdgcn_exp2f(s2 - ilse2) - p : 0.f;  // C = Q - P
            if (p > 1e-30f) lsum += p * (__builtin_amdgcn_logf(p) - s2 + ilse2);
          }
        lsum = wave_sum_xor16_32(lsum);
        f32x4 aq[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) aq[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        pv_idx<2>(si, itile, aq);  // sum over the block's keys of C ik
        if (tn >= 0) {
          const long long pe = ebase * nih + m;
          float* dst = a.part_q + pe * kIdxDim;
          uint16_t* cd = a.cbuf + pe * kBlock;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            *reinterpret_cast<f32x4*>(dst + 16 * mt + 4 * g) = aq[mt];
            u32x2 w2;
            w2[0] = pack_bf16x2(si[mt][0], si[mt][1]);
            w2[1] = pack_bf16x2(si[mt][2], si[mt][3]);
            *reinterpret_cast<u32x2*>(cd + 16 * mt + 4 * g) = w2;  // keys 16mt + 4g .. +3
          }
          if (g == 0) a.part_l[pe] = kLn2 * lsum;
        }
      }
      __builtin_amdgcn_wave_barrier();  // the tile's reads before the next job's writes
      tl = tnext;
    }
  }
}

constexpr int kDikBatch = 32;  // (entry, index head) pairs per step of the dik pass

// Pass B2: dik.  Work-group (block, sequence, split); every wave covers all
// 64 keys of the block and runs on its own over batches of 32 (entry, index
// head) pairs of the block (every KV head's list in order, index heads
// innermost; batch j to wave j mod 4): the pairs' index queries and their C
// rows are staged in wave-private LDS tiles by LDS-bound loads (the next
// batch's while one is computed), and dik^T += iq^T C^T per 16-key tile.
// The four waves' sums are then added in wave order.  Split s of a block with
// n splits takes batches [s nb / n, (s+1) nb / n); with one split it writes
// dik itself, with more each writes its partial and kl_dik_merge_kernel adds
// them in split order (deterministic).
__global__ void __launch_bounds__(256) kl_dik_kernel(KlArgs a) {
  // Per wave, two tile pairs (a batch's index queries and its C rows, islot
  // layout), each tile its own LDS object and the batch loop unrolled by two,
  // so that every access names its tile and the reads of one pair do not wait
  // for the LDS-bound loads into the other.
  __shared__ u32x4 qt0[4 * kDikBatch * 8], qt1[4 * kDikBatch * 8];
  __shared__ u32x4 ct0[4 * kDikBatch * 8], ct1[4 * kDikBatch * 8];
  __shared__ int lbeg[4], lnp[4];
  // the cross-wave sum, 32 keys at a time, in the first query tiles' memory
  // once the batches are done
  float(*red)[kIdxDim + 4] = reinterpret_cast<float(*)[kIdxDim + 4]>(&qt0[0]);
  static_assert(sizeof(float) * (kBlock / 2) * (kIdxDim + 4) <= sizeof(qt0),
                "half the reduction fits in the query tiles");
  const int c = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const int nih = a.nih;
  if (tid < 4) {
    const bool hv = tid < a.Hkv;
    const long long e = ((long long)b * a.Hkv + (hv ? tid : 0)) * a.nblk + c;
    const int bg = hv ? a.base[e] : 0;
    lbeg[tid] = bg;
    lnp[tid] = hv ? (a.base[e + 1] - bg) * nih : 0;
  }
  __syncthreads();
  const int pairs = lnp[0] + lnp[1] + lnp[2] + lnp[3];
  const int nb = (pairs + kDikBatch - 1) / kDikBatch;
  const int nsplit = key_splits(nb);
  if (split >= nsplit) return;  // uniform over the work-group
  const int j0 = (int)((long long)split * nb / nsplit);
  const int j1 = (int)((long long)(split + 1) * nb / nsplit);
  // pair p of the block: its KV head and its row in cbuf (entry e nih + m)
  auto pair_at = [&](int p, int& row, int& m) {
    int h = 0;
    while (h < 3 && p >= lnp[h]) {
      p -= lnp[h];
      ++h;
    }
    row = lbeg[h] * nih + p;
    m = p % nih;
    return h;
  };
  // four loads of 64 lanes per tile: slot = pair x 8 chunks (islot layout).
  // The query rows of a batch's pairs are read from the lists a batch ahead,
  // so that no load address waits for a load.
  int trow[4];
  auto rows_of = [&](int jb) {
#pragma unroll
    for (int inst = 0; inst < 4; ++inst) {
      const int pr = (inst * kWave + lane) >> 3;
      int row, m;
      pair_at(min(jb * kDikBatch + pr, pairs - 1), row, m);
      trow[inst] = a.lists[row / nih];
    }
  };
  auto stage = [&](int jb, u32x4* qdst, u32x4* cdst) {
#pragma unroll
    for (int inst = 0; inst < 4; ++inst) {
      const int slot = inst * kWave + lane;
      const int pr = slot >> 3, ch = (slot & 7) ^ (pr & 7);
      const int p = min(jb * kDikBatch + pr, pairs - 1);
      int row, m;
      const int h = pair_at(p, row, m);
      const int t = trow[inst];
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(a.iq + (((long long)b * a.Sq + t) * kIdxHeads + h + a.Hkv * m) *
                                                   kIdxDim + 8 * ch),
          (__attribute__((address_space(3))) void*)(qdst + inst * kWave), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(a.cbuf + (long long)row * kBlock + 8 * ch),
          (__attribute__((address_space(3))) void*)(cdst + inst * kWave), 16, 0, 0);
    }
  };
  f32x4 dka[4][4];  // [key tile][dim M-tile]
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) dka[kt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wo = wave * kDikBatch * 8;
  if (j0 + wave < j1) {
    rows_of(j0 + wave);
    stage(j0 + wave, qt0 + wo, ct0 + wo);
    rows_of(min(j0 + wave + 4, j1 - 1));
  }
  // Byte offset in a C tile of (pair 16 mt + 4 g + r, key 16 kt + n): the
  // islot address 128 pr + 16 ((kk >> 3) ^ (pr & 7)) + 2 (kk & 7) splits into
  // disjoint bit fields, (A ^ 16 (2 kt ^ r)) + 128 r + 2048 mt with A the
  // lane's part; the eight A ^ 16 c are kept, so every read is one step from
  // the tile pointer plus an immediate.
  uint32_t cbase[8];
  {
    const uint32_t A = 512u * g + 16u * ((n >> 3) | 4u * (g & 1)) + 2u * (n & 7);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      cbase[cc] = A ^ (16u * cc);
      asm volatile("" : "+v"(cbase[cc]));
    }
  }
  // Batch jb from tiles (qcur, ccur); batch jb + 4 staged into (qnext, cnext).
  // The staging is unconditional (the split's last batch once more when jb + 4
  // is past it, never read): with no branch around the LDS-bound loads the
  // compiler keeps the reads of one tile pair from waiting for the other's.
  auto step = [&](int jb, const u32x4* qcur, const u32x4* ccur, u32x4* qnext, u32x4* cnext) {
    wait_all_loads();  // batch jb's tiles and batch jb + 4's query rows
    __builtin_amdgcn_wave_barrier();
    stage(min(jb + 4, j1 - 1), qnext, cnext);
    rows_of(min(jb + 8, j1 - 1));
    const int nvalid = pairs - jb * kDikBatch;  // pairs past this are padding
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      // register r of cw[mt]: pair 16mt + 4g + r, key 16kt + n; padding pairs
      // masked to +0 (a mask, not a branch around the read)
      f32x4 cw[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t keep = 16 * mt + 4 * g + r < nvalid ? 0xffffu : 0u;
          const uint32_t v = lds_u16_at(ccur, cbase[(2 * kt) ^ r] + 128 * r + 2048 * mt);
          cw[mt][r] = __uint_as_float((v & keep) << 16);
        }
      pv_idx<1>(cw, qcur, dka[kt]);
    }
  };
  for (int jb = j0 + wave; jb < j1; jb += 8) {
    step(jb, qt0 + wo, ct0 + wo, qt1 + wo, ct1 + wo);
    if (jb + 4 < j1) step(jb + 4, qt1 + wo, ct1 + wo, qt0 + wo, ct0 + wo);
  }
  wait_all_loads();  // the batch staged past the end has landed
  // the waves' sums, added in wave order, keys 32 hh .. 32 hh + 31 at a time
  // (the first barrier also ends every wave's reads of the tiles); writer
  // thread = (key, 16-dim quarter) of the half, the first 128 threads
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    for (int w = 0; w < 4; ++w) {
      __syncthreads();
      if (wave == w) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float& dst = red[16 * kh + n][16 * mt + 4 * g + r];
              dst = (w == 0 ? 0.f : dst) + dka[2 * hh + kh][mt][r];
            }
      }
    }
    __syncthreads();
    const int kl = tid / 4, d0 = 16 * (tid % 4);
    const int key = c * kBlock + 32 * hh + kl;
    if (tid < 128 && key < a.Skv) {
      float* dst = nsplit == 1
                       ? a.dik + ((long long)b * a.Skv + key) * kIdxDim + d0
                       : a.dikp + ((((long long)b * a.nblk + c) * kKeySplits + split) * kBlock +
                                   32 * hh + kl) * kIdxDim + d0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(dst + 4 * i) = f32x4{red[kl][d0 + 4 * i], red[kl][d0 + 4 * i + 1],
                                                       red[kl][d0 + 4 * i + 2], red[kl][d0 + 4 * i + 3]};
    }
  }
}

// loss and diq of every (row, index head): its entries' block partials added
// in slot order.  One wave per (sequence, row, index head), lane = dim.
__global__ void __launch_bounds__(256) kl_merge_kernel(KlArgs a) {
  const long long w = (long long)blockIdx.x * 4 + threadIdx.x / kWave;  // (b * Sq + t) * 4 + i
  const int lane = threadIdx.x % kWave;
  if (w >= (long long)a.B * a.Sq * kIdxHeads) return;
  const int i = (int)(w % kIdxHeads);
  const long long bt = w / kIdxHeads;
  const int t = (int)(bt % a.Sq), b = (int)(bt / a.Sq);
  const int h = i % a.Hkv, m = i / a.Hkv;
  const int32_t* sp = a.slotpos + (((long long)b * a.Hkv + h) * a.Sq + t) * a.top_k;
  // lane (q, c4): slots q, q + 4, q + 8, ... (16 lanes per slot), dims 4 c4 .. 4 c4 + 3
  const int q = lane >> 4, c4 = lane & 15;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ls = 0.f;
  // eight slots per lane quarter per batch (32 slots), every load issued
  // before any is used; a quarter adds its slots in ascending order, and the
  // quarters are combined in a fixed order below (deterministic)
  for (int s0 = 0; s0 < a.top_k; s0 += 32) {
    int ev[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) ev[x] = sp[min(s0 + 4 * x + q, a.top_k - 1)];
    f32x4 vq[8];
    float vl[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const long long pe = (long long)max(ev[x], 0) * a.nih + m;
      vq[x] = *reinterpret_cast<const f32x4*>(a.part_q + pe * kIdxDim + 4 * c4);
      vl[x] = a.part_l[pe];
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const bool ok = s0 + 4 * x + q < a.top_k && ev[x] >= 0;
      acc += ok ? vq[x] : f32x4{0.f, 0.f, 0.f, 0.f};
      ls += ok ? vl[x] : 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[k] += __shfl_xor(acc[k], 16);
    acc[k] += __shfl_xor(acc[k], 32);
  }
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  // every quarter now holds the total: lane (q, c4) stores dim 4 c4 + q
  a.diq[w * kIdxDim + 4 * c4 + q] = acc[q];
  if (lane == 0) a.loss[w] = ls;
}

// dik of the blocks whose list was split: the splits' partials added in split
// order.  Work-group (block, sequence); thread = (key, 16-dim quarter).
__global__ void __launch_bounds__(256) kl_dik_merge_kernel(KlArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  int pairs = 0;
  for (int h = 0; h < a.Hkv; ++h) {
    const long long e = ((long long)b * a.Hkv + h) * a.nblk + c;
    pairs += (a.base[e + 1] - a.base[e]) * a.nih;
  }
  const int nsplit = key_splits((pairs + kDikBatch - 1) / kDikBatch);
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
  return (s.G == 4 || s.G == 8 || s.G == 16) && s.bs == kBlock;
}

// Workspace: the index log-sum-exp, the forward's log-sum-exp by row, the dik
// split partials, the entries' list positions, the per-entry partials
// (entries <= B Hkv Sq k, and Hkv nih = 4), then the inverse lists.
size_t index_kl_workspace_bytes(const Shape& s) {
  const size_t ent = (size_t)s.B * kIdxHeads * s.Sq * s.top_k;  // (entry, index head) pairs
  return (size_t)s.B * kIdxHeads * s.Sq * 4 + 256 + (size_t)s.B * s.Sq * s.Hq * 4 + 256 +
         (size_t)s.B * s.nblk * kKeySplits * kBlock * kIdxDim * 4 + 256 +
         (size_t)s.B * s.Hkv * s.Sq * s.top_k * 4 + 256 +
         ent * 8 + 256 + ent * kIdxDim * 4 + 256 + ent * 4 + 256 + ent * kBlock * 2 + 256 +
         inverse_lists_bytes(s);
}

namespace {
template <int G>
hipError_t launch_kl(const Shape& s, const KlArgs& a, hipStream_t st) {
  const dim3 blocks(s.nblk, s.B, kKeySplits);
  kl_lse_kernel<G><<<blocks, 256, 0, st>>>(a);
  const long long nlse = (long long)s.B * s.Sq * s.Hq;
  kl_lse_t_kernel<<<(unsigned)((nlse + 255) / 256), 256, 0, st>>>(a);
  const long long rows = (long long)s.B * kIdxHeads * s.Sq;
  kl_lse_merge_kernel<<<(unsigned)((rows * 16 + 255) / 256), 256, 0, st>>>(a);
  kl_entry_kernel<G><<<blocks, 256, 0, st>>>(a);
  kl_dik_kernel<<<blocks, 256, 0, st>>>(a);
  kl_dik_merge_kernel<<<dim3(s.nblk, s.B), 256, 0, st>>>(a);
  kl_merge_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_index_kl_backward(const Shape& s, const void* q, const void* k, const void* iq,
                                    const void* ik, const int32_t* sel, const float* lse,
                                    float* loss, float* diq, float* dik, void* ws,
                                    hipStream_t st) {
  if (!index_kl_supported(s)) return hipErrorInvalidValue;
  const size_t ent = (size_t)s.B * kIdxHeads * s.Sq * s.top_k;
  char* p = align256(static_cast<char*>(ws));
  float* lse_idx = reinterpret_cast<float*>(p);
  p = align256(p + (size_t)s.B * kIdxHeads * s.Sq * 4);
  float* lse_t = reinterpret_cast<float*>(p);
  p = align256(p + (size_t)s.B * s.Sq * s.Hq * 4);
  float* dikp = reinterpret_cast<float*>(p);
  p = align256(p + (size_t)s.B * s.nblk * kKeySplits * kBlock * kIdxDim * 4);
  int32_t* slotpos = reinterpret_cast<int32_t*>(p);
  p = align256(p + (size_t)s.B * s.Hkv * s.Sq * s.top_k * 4);
  f32x2* part_ml = reinterpret_cast<f32x2*>(p);
  p = align256(p + ent * 8);
  float* part_q = reinterpret_cast<float*>(p);
  p = align256(p + ent * kIdxDim * 4);
  float* part_l = reinterpret_cast<float*>(p);
  p = align256(p + ent * 4);
  uint16_t* cbuf = reinterpret_cast<uint16_t*>(p);
  p = align256(p + ent * kBlock * 2);
  const int32_t* base = nullptr;
  const int32_t* lists = nullptr;
  hipError_t e = launch_inverse_lists(s, sel, p, &base, &lists, st, slotpos);
  if (e != hipSuccess) return e;
  KlArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
           static_cast<const uint16_t*>(iq), static_cast<const uint16_t*>(ik), sel, lse, loss,
           diq, dik, lse_idx, lse_t, dikp, slotpos, part_ml, part_q, part_l, cbuf, base, lists, s.B, s.Sq,
           s.Skv, s.q_start, s.Hq, s.Hkv, s.G, s.top_k, s.nblk, kIdxHeads / s.Hkv,
           s.scale * kLog2eB};
  switch (s.G) {
    case 4: return launch_kl<4>(s, a, st);
    case 8: return launch_kl<8>(s, a, st);
    case 16: return launch_kl<16>(s, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
