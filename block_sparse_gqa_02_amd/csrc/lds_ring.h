// lds_ring.h — helpers shared by the attention kernels that stage K/V blocks
// in LDS with direct global->LDS loads.
#pragma once

#include "common.h"

namespace msa {

typedef __attribute__((address_space(3))) void* lds_ptr;

// 16-byte chunk swizzles of a 256-byte K or V row in LDS.  K: the 16 rows
// 16mt+n read at one chunk hit 16 distinct chunks.  V: the 16 rows of one
// transposed read (ds_read_b64_tr_b16, rows 16hf + 4g + n/4 of a K-step) hit
// each 32-byte pair of chunks exactly twice.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
__device__ __forceinline__ int vswz(int row) { return (row & 7) << 1; }

// Compiler-only memory barrier (no instruction).
__device__ __forceinline__ void cbarrier() { asm volatile("" ::: "memory"); }

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Ring-tag accesses as plain LDS instructions.  The compiler would otherwise
// put a wait for every outstanding LDS-bound buffer load in front of them; the
// ring kernels order them against those loads with their own vmcnt waits.
__device__ __forceinline__ int lds_load_tag(const int32_t* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ void lds_store_tag(int32_t* p, int v) {
  asm volatile("ds_write_b32 %0, %1" :: "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_fetch_add_tag(int32_t* p, int v) {
  int old;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(old) : "v"(lds_addr(p)), "v"(v) : "memory");
  return old;
}

// s_waitcnt vmcnt(n) for n in {0, 32}, expcnt and lgkmcnt unconstrained
// (vmcnt bits 3:0 and 15:14).
__device__ __forceinline__ void wait_vm(int n) {
  cbarrier();
  if (n == 0) __builtin_amdgcn_s_waitcnt(0xf70);
  else __builtin_amdgcn_s_waitcnt(0xf70 | (2 << 14));  // vmcnt = 32
  cbarrier();
}

constexpr int kRsrcFlags = 0x00020000;  // raw buffer descriptor word 3

// One 16-byte LDS-bound buffer load per lane: LDS bytes dst + 16 * lane
// receive bytes voff + soff of the descriptor's range (reads past the range
// return zero).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, const void* dst, int voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)dst, 16, voff, soff, 0, 0);
}

// Entry numbers 0..kRingEntries-1, the source of the ring tags written by
// LDS-bound loads (a union window holds at most this many entries).
constexpr int kRingEntries = 512;
struct RingEntryIds {
  int32_t v[kRingEntries];
  constexpr RingEntryIds() : v() {
    for (int i = 0; i < kRingEntries; ++i) v[i] = i;
  }
};
namespace {
__device__ const RingEntryIds kEntryIds{};
}  // namespace

// s_barrier without the memory fences of __syncthreads: the kernels order
// their global->LDS loads with explicit vmcnt waits instead.
__device__ __forceinline__ void raw_barrier() {
  cbarrier();
  __builtin_amdgcn_s_barrier();
  cbarrier();
}

// Copies rows [4*j0, 4*j1) of a 64-row K or V block (16 instructions cover the
// block) into an LDS tile with the given swizzle; rows past `last` re-read row
// `last` (they are masked by the caller).
template <int (*SWZ)(int)>
__device__ __forceinline__ void load_block_rows(const uint16_t* blk, int last, u32x4* tile, int j0,
                                                int j1) {
  const int lane = lane_id();
  for (int j = j0; j < j1; ++j) {
    const int row = 4 * j + lane / 16, ph = lane % 16;
    const int srow = min(row, last);
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const void*>(blk + srow * kHeadDim + 8 * (ph ^ SWZ(row))),
        (lds_ptr)(tile + j * kWave), 16, 0, 0);
  }
}

}  // namespace msa
