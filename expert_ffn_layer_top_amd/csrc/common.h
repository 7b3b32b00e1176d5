// Internal helpers shared by the library's translation units: status reporting, argument
// checks, bf16 / fp32 bit helpers and wave-level primitives for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe_mi355x.h"

namespace moe {

// ---------------------------------------------------------------- status / errors

// Records `msg` as the calling thread's last error and returns `st`.
int set_error(int st, const char* fmt, ...);

#define MOE_REQUIRE(cond, st, ...)                 \
  do {                                             \
    if (!(cond)) return ::moe::set_error((st), __VA_ARGS__); \
  } while (0)

#define MOE_CHECK_PTR(p) MOE_REQUIRE((p) != nullptr, MOE_ERR_INVALID_ARG, "null pointer: %s", #p)
#define MOE_CHECK_ALIGN(p) \
  MOE_REQUIRE((reinterpret_cast<uintptr_t>(p) & 15u) == 0, MOE_ERR_INVALID_ARG, "pointer not 16-byte aligned: %s", #p)

// Returns MOE_OK, or MOE_ERR_HIP with the launch error recorded.
int check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device (cached per device; 256 if the query fails).
int cu_count();

// Workgroups of a persistent grouped-GEMM launch: the tile upper bound rounded up to a multiple
// of 8 (one per XCD slot), at most one per compute unit.  The environment variable
// MOE_GG_WORKGROUPS lowers the cap (a multiple of 8, at least 8): tests use it to run many
// tiles per workgroup at small shapes.
int gemm_workgroups(long long tiles_upper);

// Shared shape rules of the ABI.
int check_layer_shape(int T, int E, int k);

// ---------------------------------------------------------------- numeric helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed pair of bf16 (low half = a), round-to-nearest-even, in one instruction
// (v_cvt_pk_bf16_f32).  Finite values and infinities convert exactly as f32_to_bf16 does; a NaN
// stays a NaN (its payload may differ).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- wave64 primitives

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

}  // namespace moe
