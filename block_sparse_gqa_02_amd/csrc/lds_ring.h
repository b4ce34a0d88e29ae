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
