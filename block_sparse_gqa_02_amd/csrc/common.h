// common.h — device-side building blocks shared by the gfx950 kernels of
// libmsa: vector types, the two bf16 MFMA shapes used, order-preserving key
// encodings for exact top-k, and small wave-level helpers.
//
// Wave64 MFMA operand layouts (checked on the device):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[m = l%16][k = 8*(l/16) + i] and
//     B[k = 8*(l/16) + i][n = l%16] (i = 0..7); result reg r of lane l is
//     C[m = 4*(l/16) + r][n = l%16].
//   v_mfma_f32_32x32x16_bf16: lane l holds A[m = l%32][k = 8*(l/32) + i] and
//     B[k = 8*(l/32) + i][n = l%32]; result reg r of lane l is
//     C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32].
// Because a contraction sums over k, A and B may use any common permutation
// of k; the kernels pick permutations that make every operand load a single
// contiguous 16-byte read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 64;       // tokens per selection block
constexpr int kHeadDim = 128;    // main-branch head dim
constexpr int kIdxDim = 64;      // index-branch head dim
constexpr int kIdxHeads = 4;     // index-query heads
constexpr int kMaxTopK = 256;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Two fp32 -> packed bf16x2 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Order-preserving map of an fp32 score to uint32: a < b as reals <=>
// key(a) < key(b); -0 and +0 map to the same key.  -inf maps to 0x007fffff,
// so the key 0 lies below every real score.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` held by lanes below the calling lane.
__device__ __forceinline__ int prefix_count(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Cache-policy operand of the LDS-bound load builtins: the non-temporal bit.
constexpr int kCachePolicyNT = 2;

// The value of lane l ^ 1 (DPP quad permutation 1, 0, 3, 2).
__device__ __forceinline__ float swap_lane_pairs(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false));
}

// max(a, b) of values that are never NaN (scores, -inf for masked ones).
// It is the IEEE maximum (a NaN would propagate; -0 orders below +0), which
// the compiler issues as is: fmaxf on values it cannot prove canonical (MFMA
// results, lane-swap results) first quiets each operand with one more
// v_max_f32.  gfx950 fuses chains of it into v_maximum3_f32.
__device__ __forceinline__ float fmax_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Reductions over the four lanes l, l^16, l^32, l^48 (the same MFMA column
// in every 16-lane row), with lane swaps instead of LDS permutes:
// v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap the two halves.
__device__ __forceinline__ float wave_max_xor16_32(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane l < 32 receives max(a[l], a[l+32]); lane l >= 32 receives
// max(b[l-32], b[l]) (one v_permlane32_swap).
__device__ __forceinline__ float halves_max(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmax_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Hand-over of data between the work-groups of one launch (the last one to
// finish a unit of work consumes what the others wrote).  The data travels
// through agent-scope coherent stores and loads, which write through / read
// past the non-coherent copy in an XCD's L2, so the producer needs no L2
// write-back (an agent-scope release fence writes back the whole L2, which
// costs far more than the data when thousands of work-groups do it); a wait
// for the producer's stores to complete orders them before its arrival count.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained), fenced against compiler
// reordering: every store this wave issued has completed.
__device__ __forceinline__ void wait_stores_done() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xf70);
  asm volatile("" ::: "memory");
}

// Counts the calling work-group in on `counter` once every thread's
// store_agent() data has completed; true, in every thread, for the work-group
// that arrives last of `total`, which also puts the counter back to zero for
// the next launch.  Nothing waits for another work-group.  flag: one int of LDS.
__device__ __forceinline__ bool arrive_last(int32_t* counter, int total, int* flag) {
  wait_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int before = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    const int last = before == total - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

}  // namespace msa
