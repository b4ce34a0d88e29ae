// attn_kvs.hip — sparse GQA prefill attention, KV-block-stationary schedule.
//
// The main branch computes exact softmax attention over the blocks each KV head
// selected (topic page "MiniMax稀疏注意力", summary paragraph).  When a query
// tile's rows share almost none of their blocks — a chunk of a few thousand
// rows choosing 128 of 16384 blocks of a 1M-token context — a tile-union fetch
// buys no reuse, and every row would gather its own blocks.  This schedule
// turns the loop around: each selected (KV head, block) is read from HBM
// once, by one work-group, which attends every row that selected it.  The
// pages' point about contiguous block reads (talk summary "How MiniMax M3 Was
// Built", section "Block-level retrieval makes sparse attention easier to run
// on GPUs") then holds for the whole context: each 16 KiB K block and V block
// is one contiguous read.
//
// Steps (one launch each):
//   1. counts: every valid selection entry (row t, slot x, block c) counts
//      itself on its (sequence, KV head, block) and keeps its rank there;
//   2. scan: exclusive prefix sums of the counts give each block's list offset;
//   3. scatter: entry (t, x) goes to its block's list at offset + rank;
//   4. attention: a work-group per (sequence, KV head, block) stages the
//      block's K and its V, transposed, in LDS and, 16 MFMA columns at a time
//      (16/G rows x G query heads), computes
//      for each listed row the block's scores, a softmax local to the block and
//      the block's output, written as a normalised fp16 partial with its
//      log2-sum-exp in the row's slot x;
//   5. merge: per (row, KV head), the partials of its slots combine by
//      log-sum-exp in slot order, so the result does not depend on the order
//      in which blocks were processed.
// The list order within a block is whatever the counting atomics gave, but
// every partial is computed on its own and lands in its own slot: results are
// bit-identical from call to call.
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKvsWaves = 4;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The fp16 in the low / high half of a 32-bit word, as fp32.
__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

struct KvsArgs {
  const uint16_t* q;      // [B][Sq][Hq][128]
  const uint16_t* k;      // [B][Hkv][Skv][128]
  const uint16_t* v;      // [B][Hkv][Skv][128]
  const int32_t* sel;     // [B][Hkv][Sq][top_k]
  uint16_t* out;          // [B][Sq][Hq][128]
  float* lse;             // [B][Hq][Sq] or null
  int32_t* cnt;           // [B][Hkv][nctx] selections per block
  int32_t* off;           // [B][Hkv][nctx] list offsets (exclusive scan of cnt)
  int32_t* rank;          // [B][Hkv][Sq][top_k] an entry's place in its block's list (-1: none)
  int32_t* list;          // [B * Hkv * Sq * top_k] entries t * 256 + x, grouped by block
  float* part_lse;        // [B][Hkv][Sq][top_k][G] log2-sum-exp of the slot's block
  uint16_t* part_o;       // [B][Hkv][Sq][top_k][G][128] fp16, normalised by its own sum
  int Sq, Skv, q_start, Hq, Hkv, G, top_k, nctx;
  float scale_log2;
  long long nsel;         // B * Hkv * Sq * top_k
  long long nblocks;      // B * Hkv * nctx
  int32_t* status;        // the call's status word (no bounded waits here: cleared only)
};

__global__ void __launch_bounds__(256) kvs_zero_kernel(KvsArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < a.nblocks) a.cnt[i] = 0;
  if (i == 0) *a.status = 0;
}

// One thread per selection entry.
__global__ void __launch_bounds__(256) kvs_count_kernel(KvsArgs a) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.nsel) return;
  const long long row = e / a.top_k;          // (b * Hkv + h) * Sq + t
  const int t = (int)(row % a.Sq);
  const long long bh = row / a.Sq;
  const int cur = (a.q_start + t) / kBlock;
  const int c = a.sel[e];
  int r = -1;
  if (c >= 0 && c <= cur) r = atomicAdd(a.cnt + bh * a.nctx + c, 1);
  a.rank[e] = r;
}

// Exclusive scan of cnt into off, one work-group of 1024 threads: thread i
// sums a contiguous run, the runs' totals are scanned in LDS.
__global__ void __launch_bounds__(1024) kvs_scan_kernel(KvsArgs a) {
  __shared__ long long part[1024];
  const int tid = threadIdx.x;
  const long long per = (a.nblocks + 1023) / 1024;
  const long long lo = tid * per, hi = min(lo + per, a.nblocks);
  long long s = 0;
  for (long long i = lo; i < hi; ++i) s += a.cnt[i];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
    const long long x = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  long long base = part[tid] - s;
  for (long long i = lo; i < hi; ++i) {
    a.off[i] = (int32_t)base;
    base += a.cnt[i];
  }
}

__global__ void __launch_bounds__(256) kvs_scatter_kernel(KvsArgs a) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.nsel) return;
  const int r = a.rank[e];
  if (r < 0) return;
  const long long row = e / a.top_k;
  const int x = (int)(e % a.top_k);
  const int t = (int)(row % a.Sq);
  const long long bh = row / a.Sq;
  const int c = a.sel[e];
  a.list[a.off[bh * a.nctx + c] + r] = t * 256 + x;
}

// Work-group per (block c, KV head h, sequence b), four waves.  LDS: the
// block's K (chunk ch of key r at r * 16 + (ch ^ (r & 15))) and its V
// transposed (dim row d holds the 64 keys in the order the PV product takes
// them: position 32kv + 8g + i is key 32kv + 16(i/4) + 4g + i%4; 16-byte chunk
// ch of row d at d * 8 + (ch ^ ((d >> 1) & 7))), the operand layouts of the
// tile-union kernel.  The work-group transposes V itself: every block is read
// once, so a separate transposing pass would only add traffic.  A wave takes
// one 16-column group at a time, with the next group's list entries and
// queries already loading while the current one is computed.
template <int G>
__global__ void __launch_bounds__(kKvsWaves * kWave) kvs_attn_kernel(KvsArgs a) {
  constexpr int RPG = 16 / G;  // rows per group
  constexpr int NT = kKvsWaves * kWave;
  __shared__ u32x4 ktile[kBlock * 16];
  __shared__ u32x4 vtile[kBlock * 16];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * a.Hkv + h;
  const int n_e = a.cnt[bh * a.nctx + c];
  if (n_e == 0) return;
  const int e0 = a.off[bh * a.nctx + c];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  const int ctx = a.q_start + a.Sq;
  {
    // keys at or past the context end repeat the last context row (zero weight);
    // every load is issued before the first LDS store
    constexpr int PER = kBlock * 16 / NT;  // 16-byte chunks of K (and of V) per thread
    const u32x4* ksrc = reinterpret_cast<const u32x4*>(a.k + bh * a.Skv * kHeadDim);
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(a.v + bh * a.Skv * kHeadDim);
    u32x4 kr[PER], vr[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int i = it * NT + tid, r = i >> 4, ch = i & 15;
      const size_t src = (size_t)min(c * kBlock + r, ctx - 1) * 16 + ch;
      kr[it] = ksrc[src];
      vr[it] = vsrc[src];
    }
    uint16_t* vt16 = reinterpret_cast<uint16_t*>(vtile);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int i = it * NT + tid, r = i >> 4, ch = i & 15;
      ktile[r * 16 + (ch ^ (r & 15))] = kr[it];
      // key r -> position of the PV k-slot order; dims 8ch .. 8ch+7
      const int kv = r >> 5, jj = r & 31;
      const int gg = (jj & 15) >> 2, ii = 4 * (jj >> 4) + (jj & 3);
      const int chunk = 4 * kv + gg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * ch + e;
        const uint32_t word = vr[it][e >> 1];
        vt16[(d * 8 + (chunk ^ ((d >> 1) & 7))) * 8 + ii] = (uint16_t)((e & 1) ? (word >> 16) : word);
      }
    }
  }
  __syncthreads();
  const char* kt = reinterpret_cast<const char*>(ktile);
  const char* vt = reinterpret_cast<const char*>(vtile);
  int kbyte[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kbyte[ks] = n * 256 + (((4 * ks + g) ^ n) << 4);
  const int vlane = n * 128 + 16 * (g ^ (n >> 1));
  const int rr = n / G, hh = n % G;
  const int key0 = c * kBlock + 4 * g;
  const int ngroups = (n_e + RPG - 1) / RPG;
  // group gi's column for this lane: list entry, then its query row
  auto entry = [&](int gi) {
    const int e = gi * RPG + rr;
    return e < n_e ? a.list[e0 + e] : -1;
  };
  auto load_q = [&](int packed, bf16x8 (&qf)[4]) {
    const int t = packed >> 8;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.q + (((size_t)b * a.Sq + (packed < 0 ? 0 : t)) * a.Hq + h * G + hh) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (packed >= 0) v = src[4 * ks + g];
      qf[ks] = as_bf16x8(v);
    }
  };
  int gi = wave;
  if (gi >= ngroups) return;
  int packed = entry(gi);
  int packed_next = entry(gi + kKvsWaves);
  bf16x8 qf[4];
  load_q(packed, qf);
  for (; gi < ngroups; gi += kKvsWaves) {
    // the next group's queries and the one after it's list entries go out now
    bf16x8 qn[4];
    load_q(packed_next, qn);
    const int packed_after = entry(gi + 2 * kKvsWaves);
    // S^T = K Q^T; sc[mt] reg r: key 16mt + 4g + r of the column
    f32x4 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        sc[mt] = mfma16(as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[ks] + mt * 4096)),
                        qf[ks], sc[mt]);
    // softmax local to the block (log2 domain, scale folded into one FMA); the
    // own block masks keys after the row
    const int pos = a.q_start + (packed >> 8);
    if (c * kBlock + kBlock - 1 > pos) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * mt + r > pos) sc[mt][r] = -__builtin_huge_valf();
    }
    float bm = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) bm = fmax_nn(bm, sc[mt][r]);
    const float m = wave_max_xor16_32(bm) * a.scale_log2;
    float ps = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * kv + e / 4][e % 4], a.scale_log2, -m));
        ps += p[e];
      }
      u32x4 pw;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) pw[w2] = pack_bf16x2(p[2 * w2], p[2 * w2 + 1]);
      pb[kv] = as_bf16x8(pw);
    }
    const float lsum = wave_sum_xor16_32(ps);
    // O^T = V^T P^T; o[mt] reg r: dim 16mt + 4g + r of the column
    f32x4 o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kv = st / 8, mt = st % 8;
      o[mt] = mfma16(as_bf16x8(*reinterpret_cast<const u32x4*>(vt + mt * 2048 + (vlane ^ (64 * kv)))),
                     pb[kv], o[mt]);
    }
    // the slot's partial: output normalised by the block's own sum (fp16), and
    // the block's log2-sum-exp
    if (packed >= 0) {
      const long long slot = ((bh * a.Sq + (packed >> 8)) * a.top_k + (packed & 255)) * G + hh;
      const float inv = 1.f / lsum;  // the own key is never masked, so the sum is > 0
      uint16_t* dst = a.part_o + slot * kHeadDim + 4 * g;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const f16x2 lo = __builtin_convertvector(f32x2{o[mt][0] * inv, o[mt][1] * inv}, f16x2);
        const f16x2 hi = __builtin_convertvector(f32x2{o[mt][2] * inv, o[mt][3] * inv}, f16x2);
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, lo);
        w[1] = __builtin_bit_cast(uint32_t, hi);
        *reinterpret_cast<u32x2*>(dst + 16 * mt) = w;
      }
      if (g == 0) a.part_lse[slot] = m + __log2f(lsum);
    }
    packed = packed_next;
    packed_next = packed_after;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qn[ks];
  }
}

// Work-group per (row t, KV head h, sequence b): thread (head hh = tid / 32,
// dims 4 (tid % 32) .. +3).  Slots merge in ascending order; slots whose entry
// is padding or out of causal range hold no partial and are skipped.
template <int G>
__global__ void __launch_bounds__(256) kvs_merge_kernel(KvsArgs a) {
  __shared__ int32_t xs[kMaxTopK];
  __shared__ int nvalid;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * a.Hkv + h;
  const long long row = bh * a.Sq + t;
  const int tid = threadIdx.x;
  const int cur = (a.q_start + t) / kBlock;
  if (tid < kWave) {
    // compact the valid slots, ascending
    int base = 0;
    for (int x0 = 0; x0 < a.top_k; x0 += kWave) {
      const int x = x0 + tid;
      const int cb = x < a.top_k ? a.sel[row * a.top_k + x] : -1;
      const bool v = cb >= 0 && cb <= cur;
      const uint64_t m = ballot(v);
      if (v) xs[base + prefix_count(m)] = x;
      base += __popcll(m);
    }
    if (tid == 0) nvalid = base;
  }
  __syncthreads();
  const int hh = tid / 32, d4 = 4 * (tid % 32);
  if (hh >= G) return;
  const int nv = nvalid;
  const float* pl = a.part_lse + row * a.top_k * G + hh;
  const uint16_t* po = a.part_o + (row * a.top_k * G + hh) * kHeadDim + d4;
  // one pass in batches of U slots (their loads go out together), the running
  // maximum moving once per batch
  constexpr int U = 8;
  float M = -__builtin_huge_valf(), L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nv; i0 += U) {
    float w[U];
    uint32_t ov0[U], ov1[U];  // dims d4, d4+1 and d4+2, d4+3 (fp16 pairs)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = xs[min(i0 + u, nv - 1)];
      w[u] = pl[(size_t)x * G];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(po + (size_t)x * G * kHeadDim);
      ov0[u] = src[0];
      ov1[u] = src[1];
    }
    // straight-line code: slots past the last one repeat it with weight zero
    float Mb = M;
#pragma unroll
    for (int u = 0; u < U; ++u) Mb = fmaxf(Mb, w[u]);
    const float alpha = __builtin_amdgcn_exp2f(M - Mb);  // 0 on the first batch
    L *= alpha;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) acc[q4] *= alpha;
    M = Mb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wt = i0 + u < nv ? __builtin_amdgcn_exp2f(w[u] - M) : 0.f;
      L += wt;
      acc[0] += wt * half_lo(ov0[u]);
      acc[1] += wt * half_hi(ov0[u]);
      acc[2] += wt * half_lo(ov1[u]);
      acc[3] += wt * half_hi(ov1[u]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int hq = h * G + hh;
  u32x2 wv;
  wv[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  wv[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(a.out + (((size_t)b * a.Sq + t) * a.Hq + hq) * kHeadDim + d4) = wv;
  if (a.lse && d4 == 0)
    a.lse[((size_t)b * a.Hq + hq) * a.Sq + t] =
        L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_huge_valf();
}

// Workspace: the status word (256 bytes), counts, offsets, ranks, lists, then
// the partials.
struct KvsLayout {
  size_t cnt, off, rank, list, part_lse, part_o, end;
};

KvsLayout kvs_layout(const Shape& s) {
  const size_t nblocks = (size_t)s.B * s.Hkv * ceil_div(s.q_start + s.Sq, kBlock);
  const size_t nsel = (size_t)s.B * s.Hkv * s.Sq * s.top_k;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  KvsLayout L;
  L.cnt = 256;
  L.off = up(L.cnt + nblocks * 4);
  L.rank = up(L.off + nblocks * 4);
  L.list = up(L.rank + nsel * 4);
  L.part_lse = up(L.list + nsel * 4);
  L.part_o = up(L.part_lse + nsel * s.G * 4);
  L.end = L.part_o + nsel * s.G * kHeadDim * 2;
  return L;
}

}  // namespace

bool kvs_prefill_preferred(const Shape& s) {
  // The tile-union kernel shares a block among the TR rows of a tile; when a
  // tile's rows together select fewer than one block per context block
  // (TR k < context blocks), that sharing is nil and each block is better read
  // once for all the rows that chose it.
  const long long tr = 24LL * 16 / s.G;  // tile rows of the tile-union kernel
  const long long nctx = ceil_div(s.q_start + s.Sq, kBlock);
  return (s.G == 8 || s.G == 4) && s.bs == kBlock && tr * s.top_k < nctx;
}

size_t kvs_prefill_workspace_bytes(const Shape& s) { return kvs_layout(s).end; }

hipError_t launch_kvs_prefill(const Shape& s, const void* q, const void* k, const void* v,
                              const int32_t* sel, void* out, float* lse, void* ws,
                              hipStream_t st) {
  const int nctx = ceil_div(s.q_start + s.Sq, kBlock);
  const long long nsel = (long long)s.B * s.Hkv * s.Sq * s.top_k;
  const long long nblocks = (long long)s.B * s.Hkv * nctx;
  // list entries pack t * 256 + x into an int32, offsets are int32
  if (s.Sq >= (1 << 23) || nsel >= (1LL << 31) || s.top_k > 256 || s.B > 65535 ||
      (s.G != 4 && s.G != 8))
    return hipErrorInvalidValue;
  char* w = static_cast<char*>(ws);
  const KvsLayout L = kvs_layout(s);
  KvsArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
            static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse,
            reinterpret_cast<int32_t*>(w + L.cnt), reinterpret_cast<int32_t*>(w + L.off),
            reinterpret_cast<int32_t*>(w + L.rank), reinterpret_cast<int32_t*>(w + L.list),
            reinterpret_cast<float*>(w + L.part_lse), reinterpret_cast<uint16_t*>(w + L.part_o),
            s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, s.G, s.top_k, nctx, s.scale * kLog2e, nsel,
            nblocks, reinterpret_cast<int32_t*>(w)};
  kvs_zero_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, st>>>(a);
  kvs_count_kernel<<<(unsigned)((nsel + 255) / 256), 256, 0, st>>>(a);
  kvs_scan_kernel<<<1, 1024, 0, st>>>(a);
  kvs_scatter_kernel<<<(unsigned)((nsel + 255) / 256), 256, 0, st>>>(a);
  const dim3 ga(nctx, s.Hkv, s.B), gm(s.Sq, s.Hkv, s.B);
  if (s.G == 8) {
    kvs_attn_kernel<8><<<ga, kKvsWaves * kWave, 0, st>>>(a);
    kvs_merge_kernel<8><<<gm, 256, 0, st>>>(a);
  } else {
    kvs_attn_kernel<4><<<ga, kKvsWaves * kWave, 0, st>>>(a);
    kvs_merge_kernel<4><<<gm, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace msa
