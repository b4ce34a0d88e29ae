// bwd_tiles.h — LDS tile helpers shared by the gradient kernels (main branch
// and index branch): the 256-byte-row tile swizzle, transposed LDS reads, and
// the load wait that orders LDS-bound global loads.
#pragma once

#include "common.h"

namespace msa {

constexpr float kLog2eB = 1.4426950408889634f;

// LDS tiles of 64 rows x 128 bf16: chunk c (16 bytes) of row r at chunk
// c ^ (r & 15), so the 16 rows of a 16-byte operand read (one chunk column)
// hit 16 distinct chunks.
__device__ __forceinline__ int swz_slot(int row, int ch) { return row * 16 + (ch ^ (row & 15)); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// ds_read_b64_tr_b16 at LDS byte address `addr`.
__device__ __forceinline__ s16x4 lds_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(uintptr_t)addr);
}

// ds_read_b64_tr_b16 at byte `off` of the LDS tile `tile`.  Unlike an address
// rebuilt from an integer, the pointer keeps the tile's LDS object in view of
// the compiler, so the read waits only for LDS-bound loads into that object.
__device__ __forceinline__ s16x4 lds_read_tr_at(const void* tile, uint32_t off) {
  typedef __attribute__((address_space(3))) const char* lds_cchar_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)((lds_cchar_ptr)tile + off));
}

// The 16 bytes at byte `off` of the LDS tile `tile` (one step from the tile
// pointer, like lds_read_tr_at).
__device__ __forceinline__ u32x4 lds_u32x4_at(const void* tile, uint32_t off) {
  typedef __attribute__((address_space(3))) const char* lds_cchar_ptr;
  typedef __attribute__((address_space(3))) const u32x4* lds_u32x4_ptr;
  return *(lds_u32x4_ptr)((lds_cchar_ptr)tile + off);
}

// The 16-bit word at byte `off` of the LDS tile `tile`, addressed like
// lds_read_tr_at (one step from the tile pointer).
__device__ __forceinline__ uint32_t lds_u16_at(const void* tile, uint32_t off) {
  typedef __attribute__((address_space(3))) const char* lds_cchar_ptr;
  typedef __attribute__((address_space(3))) const uint16_t* lds_u16_ptr;
  return *(lds_u16_ptr)((lds_cchar_ptr)tile + off);
}

// s_waitcnt vmcnt(0) with a compiler fence: the LDS-bound loads of the
// staged columns are complete (for this wave) before anything below.
__device__ __forceinline__ void wait_all_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xf70);  // vmcnt 0; expcnt, lgkmcnt unconstrained
  asm volatile("" ::: "memory");
}

}  // namespace msa
