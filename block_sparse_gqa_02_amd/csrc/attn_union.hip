// attn_union.hip — sparse GQA prefill attention, tile-union schedule.
//
// The main branch attends only to the blocks each KV head selected (topic page
// "MiniMax稀疏注意力", summary paragraph).  With independent selections per
// row, a tile of rows of one KV head touches most causal blocks, but any one
// block is wanted by only a few of its rows.  Loading each block once per tile
// and reusing it across the rows that picked it cuts K/V traffic several times
// against one gather per (row, block); the pages make the same point about
// contiguous reads and the compute-to-memory ratio (talk summary "How MiniMax
// M3 Was Built", section "Block-level retrieval makes sparse attention easier
// to run on GPUs").
//
// Work-group: eight waves on one (sequence, KV head, tile of 24 row groups); a
// row group is 16/G rows x G query heads, the 16 columns of
// v_mfma_f32_16x16x32_bf16, and wave w owns groups w, w+8, w+16 (queries and
// output accumulators in registers for the whole sweep).  Per window of 512
// blocks the tile builds, in LDS, the row and row-group bitmasks of every block
// from the rows' selections and walks the union of the blocks in ascending
// order; each block's K and V (32 KiB) are fetched once into a ring of LDS
// slots by buffer loads that write LDS directly.
//
// Only the waves that own a row group wanting a block take part in it: they
// wait for the block's slot to carry its ready tag, run their groups, and count
// themselves done.  The last of them refills the slot with the block kRing
// entries ahead.  The new tag is published by the memory system, not by the
// wave: after the 32 data loads the refiller issues one more LDS-bound load
// that copies the entry number from a device table into the slot's tag, and a
// wave's loads return in issue order, so the tag lands after the data.  The
// refiller never waits for its own fetch.  Waves that want none of a block
// skip it without touching the ring.  Every wait is bounded: past the bound
// the kernel stops waiting, stores NaN outputs and sets the call's failure
// word at the end of the workspace (a caller-visible failure, never a hang).
//
// V arrives transposed.  A pre-pass writes, for every context block, a 16 KiB
// V^T tile: 128 dim rows of 64 keys, the keys of each 32-key half permuted so
// that the eight keys one lane feeds to the PV product (k-slots 8g .. 8g+7 of
// a K-step) are adjacent.  The ring then holds V^T, and every V operand is one
// plain 16-byte LDS read instead of two transposing 8-byte reads.
//
// LDS layouts (16-byte chunks).  K (256-byte rows): chunk c of row r sits at
// chunk c ^ (r & 15), so the 16 rows of an S-tile read at one chunk hit 16
// distinct chunks.  V^T (128-byte rows): chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7); the 16 dim rows of one operand read then cover all 16
// chunk positions of a 256-byte bank line.
#include "common.h"
#include "kernels.h"
#include "lds_ring.h"

#include <atomic>

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWin = 512;          // blocks per union window
constexpr float kRescale = 8.0f;   // lazy-rescale threshold (log2 units)
constexpr int kWaves = 8;          // waves per work-group (2 per SIMD)
constexpr int kGPW = 3;            // row groups owned per wave
constexpr int kNG = kWaves * kGPW; // row groups per tile
constexpr int kRing = 4;           // K/V slots in the LDS ring
constexpr int kDefaultSpinLimit = 1 << 22;  // tag polls before a wave gives up
constexpr int kStatusBytes = 256;           // failure word at the end of the workspace
constexpr int kBlockBytes = kBlock * kHeadDim * 2;  // one K or V block

struct UnionArgs {
  const uint16_t* q;    // [B][Sq][Hq][128]
  const uint16_t* k;    // [B][Hkv][Skv][128]
  const uint16_t* vt;   // [B][Hkv][nblk_ctx] V^T tiles of 16 KiB
  const int32_t* sel;   // [B][Hkv][Sq][k]
  uint16_t* out;        // [B][Sq][Hq][128]
  float* lse;           // [B][Hq][Sq] or null
  int32_t* status;      // failure word: set to 1 when a bounded wait gives up
  int Sq, Skv, q_start, Hq, Hkv, top_k, ntiles, nblk_ctx;
  float scale_log2;
  int spin_limit;
};

// V^T tile of block c: position 32kv + 8g + i of dim row d holds V[64c + 32kv +
// 16(i/4) + 4g + i%4][d], the key of k-slot 8g + i of K-step kv in the PV
// product.  Keys at or past the context end (q_start + Sq) repeat the last
// context row: their probabilities are exactly zero, and the copy keeps them
// finite whatever the cache holds beyond the context.
struct VtArgs {
  const uint16_t* v;    // [B][Hkv][Skv][128]
  uint16_t* vt;         // [B][Hkv][nblk_ctx][128][64]
  int32_t* status;      // the call's failure word, cleared here (runs before the sweep)
  int Skv, ctx, nblk_ctx;
};

__global__ void __launch_bounds__(256) vt_kernel(VtArgs a) {
  // V block in LDS: chunk ch (dims 8ch .. 8ch+7) of key k at slot k*16 + (ch ^ (k & 15))
  __shared__ u32x4 blk[kBlock * 16];
  const long long tl = blockIdx.x;  // (b * Hkv + h) * nblk_ctx + c
  const int c = (int)(tl % a.nblk_ctx);
  const long long head = tl / a.nblk_ctx;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.v + head * a.Skv * kHeadDim);
  const int tid = threadIdx.x;
  if (tl == 0 && tid == 0) *a.status = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = i * 256 + tid;  // chunk q of the block: key q / 16, dim chunk q % 16
    const int key = q >> 4, ch = q & 15;
    const int row = min(c * kBlock + key, a.ctx - 1);
    blk[key * 16 + (ch ^ (key & 15))] = src[(size_t)row * 16 + ch];
  }
  __syncthreads();
  const uint16_t* b16 = reinterpret_cast<const uint16_t*>(blk);
  u32x4* dst = reinterpret_cast<u32x4*>(a.vt + tl * (kBlock * kHeadDim));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = i * 256 + tid;  // chunk q of the tile: dim q / 8, positions 8(q % 8) .. +7
    const int d = q >> 3, kv = (q >> 2) & 1, g = q & 3;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int k0 = 32 * kv + 16 * (e / 4) + 4 * g + (e % 4);  // position e; e + 1 is k0 + 1
      const uint32_t x0 = b16[(k0 * 16 + ((d >> 3) ^ (k0 & 15))) * 8 + (d & 7)];
      const uint32_t x1 = b16[((k0 + 1) * 16 + ((d >> 3) ^ ((k0 + 1) & 15))) * 8 + (d & 7)];
      w[e / 2] = x0 | (x1 << 16);
    }
    dst[q] = w;
  }
}

static_assert(kWin <= kRingEntries, "ring tags cover a window");

template <int G>
__global__ void __launch_bounds__(kWaves * kWave, 1) union_prefill_kernel(UnionArgs a) {
  constexpr int RPG = 16 / G;               // rows per group
  constexpr int TR = kNG * RPG;             // rows per tile
  constexpr int NWR = (TR + 31) / 32;       // row-mask words per block
  __shared__ u32x4 ktile[kRing][1024];
  __shared__ u32x4 vtile[kRing][1024];
  __shared__ uint32_t rmask[kWin][NWR];     // per block: tile rows that picked it
  __shared__ uint32_t gmask[kWin];          // per block: row groups that picked it
  __shared__ int32_t ulist[kWin];           // union entries: block | (waves wanting it) << 24
  __shared__ int32_t wcount[kWaves];
  __shared__ int32_t ready[kRing];          // union entry held by each slot
  __shared__ int32_t done[kRing];           // waves finished with the slot's entry
  __shared__ int32_t failed;

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, g = lane / 16;
  // work-groups: (b, h) major, tiles late-first (longest sweeps start first)
  const int tile = a.ntiles - 1 - (int)(blockIdx.x % a.ntiles);
  const int bh = (int)(blockIdx.x / a.ntiles);
  const int h = bh % a.Hkv, b = bh / a.Hkv;
  const int t0 = tile * TR;
  const int rows = min(TR, a.Sq - t0);
  const int pos0 = a.q_start + t0;
  const int pos_last = pos0 + rows - 1;
  const int cur_last = pos_last / kBlock;
  const size_t head = (size_t)b * a.Hkv + h;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + head * a.Skv * kHeadDim), (short)0, a.Skv * kHeadDim * 2, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.vt + head * a.nblk_ctx * (kBlock * kHeadDim)), (short)0,
      a.nblk_ctx * kBlockBytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rtag = __builtin_amdgcn_make_buffer_rsrc(
      (void*)&kEntryIds, (short)0, (int)sizeof(kEntryIds), kRsrcFlags);
  const int32_t* selh = a.sel + (head * a.Sq + t0) * a.top_k;
  const int rr = n / G, hh = n % G;  // this lane's column: row in group, head

  // owned groups gi = wave + 8j
  bf16x8 qf[kGPW][4];
  float mref[kGPW], lsum[kGPW];
  f32x4 o[kGPW][8];
#pragma unroll
  for (int j = 0; j < kGPW; ++j) {
    const int row = (wave + kWaves * j) * RPG + rr;
    const bool ok = row < rows;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.q + (((size_t)b * a.Sq + t0 + (ok ? row : 0)) * a.Hq + h * G + hh) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = src[4 * ks + g];
      qf[j][ks] = as_bf16x8(v);
    }
    mref[j] = -__builtin_huge_valf();
    lsum[j] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[j][x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid == 0) failed = 0;

  // Ring fill.  K instruction j of a block (64 lanes x 16 B) covers rows
  // 4j..4j+3: lane -> row 4j + lane/16, LDS chunk lane%16, which holds the
  // row's chunk (lane%16) ^ kswz(row).  Blocks wholly at or before every tile
  // row's position take precomputed per-lane offsets (the swizzle depends on
  // j mod 4); the diagonal block re-reads its last used row in place of later
  // ones.  V^T instruction j covers dim rows 8j..8j+7: lane -> row
  // 8j + lane/8, LDS chunk lane%8, which holds chunk (lane%8) ^ ((row >> 1) & 7)
  // (depends on j mod 2).
  int koff[4];
#pragma unroll
  for (int jm = 0; jm < 4; ++jm) {
    const int row = 4 * jm + lane / 16;
    koff[jm] = (lane / 16) * 256 + 16 * ((lane % 16) ^ kswz(row));
  }
  auto vtoff = [&](int j) { return (lane / 8) * 128 + 16 * ((lane % 8) ^ ((4 * j + lane / 16) & 7)); };
  const int voff[2] = {vtoff(0), vtoff(1)};
  auto fetch_full = [&](int c, int sl) {
    const int sb = c * kBlockBytes;
    if (c * kBlock + kBlock - 1 <= pos_last) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        load_lds16(rk, &ktile[sl][j * kWave], koff[j & 3], sb + j * 1024);
        load_lds16(rv, &vtile[sl][j * kWave], voff[j & 1], sb + j * 1024);
      }
    } else {
      const int last = pos_last - c * kBlock;
      for (int j = 0; j < 16; ++j) {
        const int row = 4 * j + lane / 16, srow = min(row, last);
        load_lds16(rk, &ktile[sl][j * kWave], srow * 256 + 16 * ((lane % 16) ^ kswz(row)), sb);
        load_lds16(rv, &vtile[sl][j * kWave], vtoff(j), sb + j * 1024);
      }
    }
  };
  auto fetch_part = [&](int c, int sl, int j0, int j1) {
    const int sb = c * kBlockBytes;
    const int last = min(pos_last - c * kBlock, kBlock - 1);
    for (int j = j0; j < j1; ++j) {
      const int row = 4 * j + lane / 16, srow = min(row, last);
      load_lds16(rk, &ktile[sl][j * kWave], srow * 256 + 16 * ((lane % 16) ^ kswz(row)), sb);
      load_lds16(rv, &vtile[sl][j * kWave], vtoff(j), sb + j * 1024);
    }
  };

  // K operand: lane reads row 16mt + n, dims 32ks + 8g .. +7
  int kbyte[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kbyte[ks] = n * 256 + (((4 * ks + g) ^ n) << 4);
  // V^T operand: lane (g, n) of M-tile mt, K-step kv reads dim row 16mt + n,
  // chunk 4kv + g (k-slots 8g .. 8g+7), stored at chunk (4kv + g) ^ (n >> 1):
  // byte 2048 mt + (vlane ^ 64 kv).
  const int vlane = n * 128 + 16 * (g ^ (n >> 1));

  auto compute = [&](int sl, int c, uint32_t gm, const uint32_t* rm) {
    const char* kt = reinterpret_cast<const char*>(&ktile[sl][0]);
    const char* vt = reinterpret_cast<const char*>(&vtile[sl][0]);
    const int key0 = c * kBlock + 4 * g;
#pragma unroll
    for (int j = 0; j < kGPW; ++j) {
      const int gi = wave + kWaves * j;
      if (!((gm >> gi) & 1u)) continue;
      // S^T = K Q^T: sc[mt][r] is the score of key 16mt + 4g + r for this column.
      // K-step outer, M-tile inner: the four accumulators are independent, and
      // the fragments of K-step ks + 1 are read while K-step ks multiplies.
      f32x4 sc[4];
      bf16x8 kf[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        kf[0][mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[0] + mt * 4096));
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < 3) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            kf[(ks + 1) & 1][mt] =
                as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kbyte[ks + 1] + mt * 4096));
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sc[mt] = mfma16(kf[ks & 1][mt], qf[j][ks], sc[mt]);
      }
      const int row = gi * RPG + rr;
      const bool act = (rm[row / 32] >> (row % 32)) & 1u;
      if (c * kBlock + kBlock - 1 > pos0 + gi * RPG) {
        // the block reaches past the group's first row: mask keys after each row
        const int pc = pos0 + row;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + 16 * mt + r > pc) sc[mt][r] = -__builtin_huge_valf();
      }
      float bm = fmax_nn(fmax_nn(fmax_nn(sc[0][0], sc[0][1]), fmax_nn(sc[0][2], sc[0][3])),
                       fmax_nn(fmax_nn(sc[1][0], sc[1][1]), fmax_nn(sc[1][2], sc[1][3])));
      bm = fmax_nn(bm, fmax_nn(fmax_nn(fmax_nn(sc[2][0], sc[2][1]), fmax_nn(sc[2][2], sc[2][3])),
                           fmax_nn(fmax_nn(sc[3][0], sc[3][1]), fmax_nn(sc[3][2], sc[3][3]))));
      bm = act ? bm : -__builtin_huge_valf();
      bm = wave_max_xor16_32(bm) * a.scale_log2;
      // lazy rescale: move the reference max only when a block exceeds it by > 2^8
      const bool grow = bm > mref[j] + kRescale;
      if (ballot(grow) != 0ull) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(mref[j] - bm) : 1.f;  // 0 from -inf
#pragma unroll
        for (int x = 0; x < 8; ++x) o[j][x] *= alpha;
        lsum[j] *= alpha;
        mref[j] = grow ? bm : mref[j];
      }
      // rows that did not pick the block get P = 0 (exp2 of -inf)
      const float msub = act ? mref[j] : __builtin_huge_valf();
      float ps = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * kv + e / 4][e % 4], a.scale_log2, -msub));
          ps += p[e];
        }
        u32x4 pw;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) pw[w2] = pack_bf16x2(p[2 * w2], p[2 * w2 + 1]);
        pb[kv] = as_bf16x8(pw);
      }
      lsum[j] += ps;
      // O^T += V^T P^T over two K-steps of 32 keys; k-slot e of K-step kv is key
      // 32kv + 16(e/4) + 4g + e%4, matching this lane's own P registers.  V
      // fragments are read three (K-step, M-tile) steps ahead of their multiply.
      auto vfrag = [&](int kv, int mt) {
        return as_bf16x8(*reinterpret_cast<const u32x4*>(vt + mt * 2048 + (vlane ^ (64 * kv))));
      };
      bf16x8 vf[4];
      vf[0] = vfrag(0, 0);
      vf[1] = vfrag(0, 1);
      vf[2] = vfrag(0, 2);
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int kv = st / 8, mt = st % 8;
        if (st < 13) vf[(st + 3) & 3] = vfrag((st + 3) / 8, (st + 3) % 8);
        o[j][mt] = mfma16(vf[st & 3], pb[kv], o[j][mt]);
      }
    }
  };

  bool ok_run = true;
  for (int wb = 0; wb <= cur_last && ok_run; wb += kWin) {
    const int we = min(wb + kWin, cur_last + 1);
    // 1. row and group bitmasks of the window's blocks
    for (int x = tid; x < kWin * NWR; x += kWaves * kWave) (&rmask[0][0])[x] = 0u;
    for (int x = tid; x < kWin; x += kWaves * kWave) gmask[x] = 0u;
    if (tid < kRing) {
      ready[tid] = -1;
      done[tid] = 0;
    }
    __syncthreads();
    {
      constexpr int parts = kWaves * kWave / TR;
      const int row = tid % TR, part = tid / TR;
      if (row < rows && part < parts) {
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
    for (int j = 0; j < kWin; j += kWaves * kWave) {
      const int pidx = j + tid;
      const uint32_t gmv = pidx < we - wb ? gmask[pidx] : 0u;
      const bool nz = gmv != 0u;
      const uint64_t bal = ballot(nz);
      if (lane == 0) wcount[wave] = __popcll(bal);
      __syncthreads();
      int before = nu;
      for (int w = 0; w < wave; ++w) before += wcount[w];
      if (nz) {
        const uint32_t wbits = (gmv | (gmv >> 8) | (gmv >> 16)) & 0xffu;
        ulist[before + prefix_count(bal)] = (wb + pidx) | (int)(wbits << 24);
      }
#pragma unroll
      for (int w = 0; w < kWaves; ++w) nu += wcount[w];
      __syncthreads();
    }
    // 3. first kRing entries: every wave moves 2 of the 16 instructions of each
    for (int s = 0; s < kRing && s < nu; ++s)
      fetch_part(ulist[s] & 0xffffff, s, 2 * wave, 2 * wave + 2);
    wait_vm(0);
    __syncthreads();
    if (tid < kRing && tid < nu) ready[tid] = tid;
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
        const int sl = u % kRing;
        // a wave's LDS operations complete in order, so once the tag reads u the
        // slot's data reads below see the block
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
        // A wave that holds a slot issues ahead of its SIMD's other wave from
        // here until its refill has gone out, so slots turn over sooner.
        cbarrier();
        __builtin_amdgcn_s_setprio(2);
        compute(sl, c, gmask[c - wb], rmask[c - wb]);
        cbarrier();
        // count this wave done (its slot reads precede the increment in the
        // wave's in-order LDS stream); the last wanting wave refills the slot
        // with entry u + kRing
        int prev = 0;
        if (lane == 0) prev = lds_fetch_add_tag(&done[sl], 1);
        prev = __builtin_amdgcn_readfirstlane(prev);
        if (prev == need - 1) {
          // the count is reset before the loads are issued; the tag that lets
          // the next entry's waves in is written after the block's data
          if (lane == 0) lds_store_tag(&done[sl], 0);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (u + kRing < nu) {
            fetch_full(ulist[u + kRing] & 0xffffff, sl);
            if (lane == 0)
              __builtin_amdgcn_raw_ptr_buffer_load_lds(rtag, (lds_ptr)&ready[sl], 4, 0,
                                                       (u + kRing) * 4, 0, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    wait_vm(0);
    __syncthreads();
    if (failed) ok_run = false;
  }
  if (!ok_run && tid == 0) *a.status = 1;  // a vector store: visible to the caller after the call

  // epilogue: normalise and store this wave's groups; register r of o[j][mt] is
  // dim 16mt + 4g + r of this lane's column
#pragma unroll
  for (int j = 0; j < kGPW; ++j) {
    const int row = (wave + kWaves * j) * RPG + rr;
    const float L = wave_sum_xor16_32(lsum[j]);
    if (row < rows) {
      // a failed sweep (bounded wait exceeded) stores NaN so the caller sees it
      const float inv = !ok_run ? __builtin_nanf("") : (L > 0.f ? 1.f / L : 0.f);
      uint16_t* dst = a.out + (((size_t)b * a.Sq + t0 + row) * a.Hq + h * G + hh) * kHeadDim;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        u32x2 w;
        w[0] = pack_bf16x2(o[j][mt][0] * inv, o[j][mt][1] * inv);
        w[1] = pack_bf16x2(o[j][mt][2] * inv, o[j][mt][3] * inv);
        *reinterpret_cast<u32x2*>(dst + 16 * mt + 4 * g) = w;
      }
      if (a.lse && g == 0)
        a.lse[((size_t)b * a.Hq + h * G + hh) * a.Sq + t0 + row] =
            L > 0.f ? (mref[j] + __log2f(L)) * kLn2 : -__builtin_huge_valf();
    }
  }
}

}  // namespace

bool union_prefill_supported(const Shape& s) { return s.G == 8 || s.G == 4; }

static int context_blocks(const Shape& s) { return ceil_div(s.q_start + s.Sq, kBlock); }

static size_t vt_bytes(const Shape& s) {
  return (size_t)s.B * s.Hkv * context_blocks(s) * kBlockBytes;
}

size_t union_prefill_workspace_bytes(const Shape& s) { return vt_bytes(s) + kStatusBytes; }

size_t union_prefill_status_offset(const Shape& s) { return vt_bytes(s); }

static std::atomic<int> g_spin_limit{kDefaultSpinLimit};

void set_union_spin_limit(int spins) { g_spin_limit.store(spins > 0 ? spins : kDefaultSpinLimit); }

int union_spin_limit() { return g_spin_limit.load(); }

hipError_t launch_vt_tiles(const Shape& s, const void* v, void* ws, hipStream_t st) {
  const int nblk_ctx = context_blocks(s);
  const long long tiles_vt = (long long)s.B * s.Hkv * nblk_ctx;
  if (tiles_vt > 0x7fffffffLL) return hipErrorInvalidValue;
  int32_t* status = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + vt_bytes(s));
  VtArgs t{static_cast<const uint16_t*>(v), static_cast<uint16_t*>(ws), status, s.Skv,
           s.q_start + s.Sq, nblk_ctx};
  vt_kernel<<<(unsigned)tiles_vt, 256, 0, st>>>(t);
  return hipGetLastError();
}

hipError_t launch_union_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                const int32_t* sel, void* out, float* lse, void* ws,
                                hipStream_t st) {
  const int TR = kNG * 16 / s.G;
  const int ntiles = ceil_div(s.Sq, TR);
  const int nblk_ctx = context_blocks(s);
  // the buffer descriptors address one head's K or V^T with 32-bit byte offsets
  if ((long long)s.Skv * kHeadDim * 2 > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long tiles_vt = (long long)s.B * s.Hkv * nblk_ctx;
  const long long grid = (long long)ntiles * s.Hkv * s.B;
  if (grid > 0x7fffffffLL || tiles_vt > 0x7fffffffLL) return hipErrorInvalidValue;
  int32_t* status = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + vt_bytes(s));
  hipError_t e = launch_vt_tiles(s, v, ws, st);
  if (e != hipSuccess) return e;
  UnionArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
              static_cast<const uint16_t*>(ws), sel, static_cast<uint16_t*>(out), lse, status,
              s.Sq, s.Skv, s.q_start, s.Hq, s.Hkv, s.top_k, ntiles, nblk_ctx, s.scale * kLog2e,
              g_spin_limit.load()};
  if (s.G == 8) union_prefill_kernel<8><<<(unsigned)grid, kWaves * kWave, 0, st>>>(a);
  else if (s.G == 4) union_prefill_kernel<4><<<(unsigned)grid, kWaves * kWave, 0, st>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
