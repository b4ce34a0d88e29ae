// attn_sparse.hip — main branch of MSA: exact GQA attention over each KV
// head's selected 64-token blocks (topic page "MiniMax稀疏注意力", summary
// paragraph), prefill and split-K decode, plus the dense causal decode used as
// the full-attention baseline.
//
// Prefill: one wave per (sequence, KV head, query row); the wave's 16 MFMA
// columns are the row's G query heads (WaveAttn in attn_block.h).  Waves are
// ordered KV-head-major, so the K/V working set of the whole GPU at any moment
// is one head's cache.
//
// Decode: one wave per (sequence, KV head, split) attends a contiguous run of
// the selection (or of all causal blocks for the dense baseline) and writes an
// unnormalised partial (m, l, O); a merge kernel combines the splits by
// log-sum-exp.  Splits keep enough waves in flight to stream K/V at HBM rate
// when only B * Hkv = 128 (sequence, head) pairs exist.  (Merging in the same
// launch, by the last work-group of each (sequence, KV head), measured slower:
// handing the partials over inside a launch takes write-through stores and an
// arrival atomic per work-group, which cost more than the merge launch.)
#include "attn_block.h"
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kAttnWaves = 4;

struct PrefillArgs {
  const uint16_t* q;    // [B][Sq][Hq][128]
  const uint16_t* k;    // [B][Hkv][Skv][128]
  const uint16_t* v;
  const int32_t* sel;   // [B][Hkv][Sq][k]
  uint16_t* out;        // [B][Sq][Hq][128]
  float* lse;           // [B][Hq][Sq] or null
  int Sq, Skv, q_start, Hq, Hkv, G, top_k;
  float scale_log2;
  long long units;      // B * Hkv * Sq
};

__global__ void __launch_bounds__(256) sparse_prefill_kernel(PrefillArgs a) {
  __shared__ u32x4 vtile[kAttnWaves][kBlock * 16];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const long long u = (long long)blockIdx.x * kAttnWaves + wave;
  if (u >= a.units) return;
  const int t = (int)(u % a.Sq);
  const int bh = (int)(u / a.Sq);
  const int h = bh % a.Hkv, b = bh / a.Hkv;
  const int pos = a.q_start + t;
  const int cur = pos / kBlock;
  const int hq0 = h * a.G;

  WaveAttn st;
  st.init();
  st.load_q(a.q + (((size_t)b * a.Sq + t) * a.Hq + hq0) * kHeadDim, a.G);
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  const uint16_t* vh = a.v + ((size_t)b * a.Hkv + h) * a.Skv * kHeadDim;
  // sel == null: dense causal attention over every block 0..cur
  const int32_t* list = a.sel ? a.sel + u * a.top_k : nullptr;
  const int nlist = list ? a.top_k : cur + 1;
  for (int r = 0; r < nlist; ++r) {
    const int c = list ? list[r] : r;
    if (c < 0 || c > cur) continue;  // padding (or an invalid entry): never read
    st.block(kh, vh, c, pos, a.scale_log2, vtile[wave]);
  }
  const float L = st.total_l();
  const int n = lane % 16, g = lane / 16;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (n < a.G) {
    st.store_bf16(a.out + (((size_t)b * a.Sq + t) * a.Hq + hq0 + n) * kHeadDim, inv);
    if (a.lse && g == 0)
      a.lse[((size_t)b * a.Hq + hq0 + n) * a.Sq + t] =
          L > 0.f ? (st.m + __log2f(L)) * kLn2 : -__builtin_huge_valf();
  }
}

struct DecodeArgs {
  const uint16_t* q;     // [B][1][Hq][128]
  const uint16_t* k;     // [B][Hkv][Skv][128]
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* sel;    // [B][Hkv][1][k] or null (dense: every causal block)
  float* part_o;         // [B][Hkv][nsplit][G][128]
  float* part_ml;        // [B][Hkv][nsplit][G][2]
  uint16_t* out;         // [B][1][Hq][128]
  float* lse;            // [B][Hq][1] or null
  int Skv, Hq, Hkv, G, top_k, nsplit, per_split;
  float scale_log2;
  const int32_t* pages;  // paged K/V pools: [B][nblk] page ids, else null
  int num_pages, nblk;
};

// s_waitcnt vmcnt(N) (N in {0, 32}; expcnt and lgkmcnt unconstrained: vmcnt
// bits 3:0 and 15:14), fenced against compiler reordering of memory accesses.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N == 0 || N == 32, "encoded counts");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(N == 0 ? 0xf70 : (0xf70 | (2 << 14)));
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(256) decode_partial_kernel(DecodeArgs a) {
  __shared__ u32x4 vtile[kAttnWaves][2][kBlock * 16];  // 128 KiB
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int split = blockIdx.x * kAttnWaves + wave;
  const int h = blockIdx.y, b = blockIdx.z;
  if (split >= a.nsplit) return;
  const int pos = min(max(a.seq_lens[b], 1), a.Skv) - 1;
  const int cur = pos / kBlock;
  const int hq0 = h * a.G;
  WaveAttn st;
  st.init();
  st.load_q(a.q + ((size_t)b * a.Hq + hq0) * kHeadDim, a.G);
  const int rbeg = split * a.per_split;
  const int rend = a.sel ? min(rbeg + a.per_split, a.top_k) : min(rbeg + a.per_split, cur + 1);
  const int32_t* list = a.sel ? a.sel + ((size_t)b * a.Hkv + h) * a.top_k : nullptr;
  // Lane j < per_split looks up entry rbeg + j: its block c and the element
  // offset of that block's K/V rows.  Ids outside [0, cur] and, with paged
  // caches, pages outside the pool are skipped, never read.
  int c_l = 0;
  long long off_l = 0;
  bool ok_l = false;
  if (lane < a.per_split && rbeg + lane < rend) {
    c_l = list ? list[rbeg + lane] : rbeg + lane;
    ok_l = c_l >= 0 && c_l <= cur;
    if (ok_l && a.pages) {
      // block c of this sequence is page pg of the pools ([page][Hkv][64][128])
      const int pg = a.pages[(size_t)b * a.nblk + c_l];
      ok_l = pg >= 0 && pg < a.num_pages;
      off_l = ((long long)pg * a.Hkv + h) * kBlock * kHeadDim;
    } else if (ok_l) {
      off_l = (((long long)b * a.Hkv + h) * a.Skv + (long long)c_l * kBlock) * kHeadDim;
    }
  }
  uint64_t todo = ballot(ok_l);
  if (todo != 0ull) {
    // Blocks in entry order; block i+1's V loads go out while block i is
    // attended and its K loads right after block i's S products, so one
    // block's loads are always in flight behind the arithmetic.
    auto next = [&](int& c, long long& off) {
      const int j = __builtin_ctzll(todo);
      todo &= todo - 1;
      c = __builtin_amdgcn_readlane(c_l, j);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)off_l, j);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((unsigned long long)off_l >> 32), j);
      off = (long long)(((unsigned long long)hi << 32) | lo);
    };
    // V travels by LDS-bound loads into the wave's two V tiles (alternating),
    // K through registers.  Block i+1's loads (V, then K) are issued right
    // after block i's S products, so they are in flight during block i's
    // softmax and PV.  Loads return in issue order: once block i's K has
    // arrived (the compiler's wait before the S products) its V is in LDS
    // too; the explicit waits before the V reads restate that with block i+1's
    // 32 loads still allowed in flight, and keep the reads below them.
    auto last_row = [&](int c) { return min(pos - c * kBlock, kBlock - 1); };
    u32x4 kr[4][4];
    int c, buf = 0;
    long long off;
    next(c, off);
    WaveAttn::load_v_lds(a.v + off, last_row(c), vtile[wave][0]);
    WaveAttn::load_k<true>(a.k + off, last_row(c), kr);
    while (todo != 0ull) {
      int cn;
      long long offn;
      next(cn, offn);
      st.attend(kr, c, pos, a.scale_log2, vtile[wave][buf],
                [&] {
                  __builtin_amdgcn_sched_barrier(0);  // keep the loads after the S products
                  WaveAttn::load_v_lds(a.v + offn, last_row(cn), vtile[wave][buf ^ 1]);
                  WaveAttn::load_k<true>(a.k + offn, last_row(cn), kr);
                },
                [] { wait_vmcnt<32>(); });
      c = cn;
      buf ^= 1;
    }
    st.attend(kr, c, pos, a.scale_log2, vtile[wave][buf], [] {}, [] { wait_vmcnt<0>(); });
  }
  const float L = st.total_l();
  const int n = lane % 16, g = lane / 16;
  if (n < a.G) {
    const size_t col = (((size_t)b * a.Hkv + h) * a.nsplit + split) * a.G + n;
    st.store_f32(a.part_o + col * kHeadDim);
    if (g == 0) {
      a.part_ml[2 * col] = st.m;  // -inf when the split attended nothing
      a.part_ml[2 * col + 1] = L;
    }
  }
}

// One wave per (sequence, query head): log-sum-exp merge of the splits.  The
// splits are read eight at a time, every load of a batch issued before any is
// used; a batch raises the reference max once and rescales the sums so far
// (with eight or fewer splits the one batch's max is the global one, and the
// sums are those of a two-pass merge).
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  constexpr int kBatch = 8;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int hq = blockIdx.x * kAttnWaves + wave;
  const int b = blockIdx.y;
  if (hq >= a.Hq) return;
  const int h = hq / a.G, n = hq % a.G;
  const size_t col0 = ((size_t)b * a.Hkv + h) * a.nsplit * a.G + n;
  const float ninf = -__builtin_huge_valf();
  float M = ninf, L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += kBatch) {
    f32x2 ml[kBatch], ov[kBatch];
#pragma unroll
    for (int x = 0; x < kBatch; ++x) {
      const bool ok = s0 + x < a.nsplit;
      const size_t col = col0 + (size_t)(ok ? s0 + x : 0) * a.G;
      ml[x] = ok ? reinterpret_cast<const f32x2*>(a.part_ml)[col] : f32x2{ninf, 0.f};
      ov[x] = ok ? reinterpret_cast<const f32x2*>(a.part_o + col * kHeadDim)[lane] : f32x2{0.f, 0.f};
    }
    float bm = M;
#pragma unroll
    for (int x = 0; x < kBatch; ++x) bm = fmaxf(bm, ml[x][0]);  // -inf: the split attended nothing
    if (bm == ninf) continue;
    if (bm > M) {
      const float sc = M == ninf ? 0.f : exp2f(M - bm);
      L *= sc;
      o0 *= sc;
      o1 *= sc;
      M = bm;
    }
#pragma unroll
    for (int x = 0; x < kBatch; ++x) {
      if (ml[x][0] == ninf) continue;
      const float w = exp2f(ml[x][0] - M);
      L += w * ml[x][1];
      o0 += w * ov[x][0];
      o1 += w * ov[x][1];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  reinterpret_cast<uint32_t*>(a.out + ((size_t)b * a.Hq + hq) * kHeadDim)[lane] =
      pack_bf16x2(o0 * inv, o1 * inv);
  if (a.lse && lane == 0)
    a.lse[(size_t)b * a.Hq + hq] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_huge_valf();
}

int decode_per_split(const Shape& s, bool dense) {
  // sparse: 8 selected blocks per wave (measured best at 32 x 256K: shorter runs
  // pay more per-wave set-up and merge than they gain in parallelism);
  // dense: 64 blocks per wave.
  return dense ? 64 : 8;
}
int decode_nsplit(const Shape& s, bool dense) {
  const int n = dense ? s.nblk : s.top_k;
  return ceil_div(n, decode_per_split(s, dense));
}

}  // namespace

size_t sparse_prefill_workspace_bytes(const Shape& s) {
  if (!union_prefill_supported(s)) return 0;
  return kvs_prefill_preferred(s) ? kvs_prefill_workspace_bytes(s)
                                  : union_prefill_workspace_bytes(s);
}

size_t sparse_prefill_status_offset(const Shape& s) {
  return kvs_prefill_preferred(s) ? 0 : union_prefill_status_offset(s);
}

hipError_t launch_sparse_attn_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                      const int32_t* sel, void* out, float* lse, void* ws,
                                      hipStream_t st) {
  PrefillArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse,
                s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, s.G, s.top_k, s.scale * kLog2e,
                (long long)s.B * s.Hkv * s.Sq};
  if (sel && union_prefill_supported(s)) {
    if (kvs_prefill_preferred(s)) return launch_kvs_prefill(s, q, k, v, sel, out, lse, ws, st);
    return launch_union_prefill(s, q, k, v, sel, out, lse, ws, st);
  }
  const long long grid = (a.units + kAttnWaves - 1) / kAttnWaves;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  sparse_prefill_kernel<<<(unsigned)grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_dense_attn_prefill_rowwise(const Shape& s, const void* q, const void* k,
                                             const void* v, void* out, float* lse,
                                             hipStream_t st) {
  return launch_sparse_attn_prefill(s, q, k, v, nullptr, out, lse, nullptr, st);
}

// The decode partials of msa_sparse_attn_decode_static, for callers that
// cannot allocate: one copy per GPU the library runs on, held until the
// process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (dev_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(const Shape& s, bool dense) {
  const size_t cols = (size_t)s.B * s.Hkv * decode_nsplit(s, dense) * s.G;
  return cols * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const Shape& s, const void* q, const void* k, const void* v,
                              const int32_t* seq_lens, const int32_t* sel, void* out, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t st, const Paging* pg) {
  if (ws_bytes < decode_workspace_bytes(s, sel == nullptr)) return hipErrorInvalidValue;
  const bool dense = sel == nullptr;
  const int nsplit = decode_nsplit(s, dense);
  const size_t cols = (size_t)s.B * s.Hkv * nsplit * s.G;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + cols * kHeadDim;
  DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
               static_cast<const uint16_t*>(v), seq_lens, sel, part_o, part_ml,
               static_cast<uint16_t*>(out), lse, s.Skv, s.Hq, s.Hkv, s.G, s.top_k, nsplit,
               decode_per_split(s, dense), s.scale * kLog2e, pg ? pg->table : nullptr,
               pg ? pg->num_pages : 0, s.nblk};
  dim3 g1(ceil_div(nsplit, kAttnWaves), s.Hkv, s.B);
  decode_partial_kernel<<<g1, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(ceil_div(s.Hq, kAttnWaves), s.B);
  decode_merge_kernel<<<g2, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
