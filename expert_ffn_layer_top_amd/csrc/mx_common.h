// MXFP8 block-format helpers (device): the shared E8M0 exponent of a block of bf16 values and
// saturating round-to-nearest-even E4M3 encoding.
//
// Format facts (the OCP Microscaling formats definition, which MXFP8 on the [news] page
// "MXFP8 reduces compute and memory costs" refers to): E4M3 has 1 sign, 4 exponent (bias 7)
// and 3 mantissa bits, subnormals m * 2^-9, largest finite 448 (0x7E), no infinity; an E8M0
// byte s means 2^(s - 127).  Block rule: shared = clamp(floor(log2 amax) - 8, -127, 127)
// (8 is the exponent of 448), scale byte = shared + 127, q = E4M3(v / 2^shared).
#pragma once

#include "common.h"

namespace moe {

// Layout of the block scales the MXFP8 grouped GEMMs read for their forward and dgrad operands
// (a K step of a 256-row tile needs 4 scale bytes of every row): a matrix of R rows quantised
// along K (K/32 scale bytes per row) stores the byte of row r, block b at ((b / G) R + r) G + b % G
// with G = 16 when K is a multiple of 512, 4 when of 128, else 1, i.e. [K/32G][R][G]: the scales
// of G consecutive blocks of consecutive rows are one contiguous run, one cache line per 128 / G
// rows, where row-major scales take a line per row.  Batched matrices lay out each one alone.
__host__ __device__ __forceinline__ int mx_gemm_group(long long K) { return K % 512 == 0 ? 16 : (K % 128 == 0 ? 4 : 1); }
__host__ __device__ __forceinline__ long long mx_gemm_scale_index(long long r, long long b, long long R, long long K) {
  const int G = mx_gemm_group(K);
  return ((b / G) * R + r) * G + (b % G);
}

// floor(log2(amax)) - 8 clamped to [-127, 127], from the magnitude bits of a bf16 amax
// (amax_bits = max over the block of (bits & 0x7fff)).  Returns -127 for an all-zero block.
// mode 1 (the rounded-up scale): the smallest power of two X with amax / X <= 448, i.e. one more
// when amax's significand exceeds 1.75 (448 = 1.75 * 2^8), so that no element saturates.
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits, int mode = 0) {
  if (amax_bits == 0) return -127;
  const int eb = static_cast<int>(amax_bits >> 7);
  const int man = static_cast<int>(amax_bits & 0x7f);
  int e;
  if (eb > 0) {
    e = eb - 127;
    if (mode == 1 && man > 96) ++e;          // significand 1 + man/128 > 1.75
  } else {                                   // bf16 subnormal: man * 2^-133, man in [1, 127]
    const int top = 31 - __clz(man);
    e = top - 133;
    if (mode == 1 && 4 * man > (7 << top)) ++e;   // significand man / 2^top > 1.75
  }
  int s = e - 8;
  s = s < -127 ? -127 : s;
  s = s > 127 ? 127 : s;
  return s;
}

// bf16 value `b` divided by 2^shared, as a signed fp32 clamped to [-448, 448] (the largest E4M3
// magnitude: larger ones saturate).  The bf16 bits in the top half of a word are the fp32 value
// exactly (subnormals included), and 2^-shared is a normal fp32 (a bf16 amax puts shared in
// [-127, 120]), so the product is exact whenever it is at least 2^-126; a smaller one (rounded,
// possibly to a signed zero) is far below half the smallest E4M3 subnormal, 2^-10, and encodes as
// a zero of its sign either way.  Needs fp32 denormals preserved (the compiler's default here).
__device__ __forceinline__ float mx_scaled(uint32_t b, int shared) {
  const float a = __uint_as_float(b << 16) * __uint_as_float(static_cast<uint32_t>(127 - shared) << 23);
  return __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
}

// E4M3 codes of bf16 values b0..b3 divided by 2^shared, in bytes 0..3 of one word: the hardware
// conversion to the OCP E4M3 format, rounding to nearest even (inputs are within +-448, so
// nothing overflows; values below the smallest subnormal give a zero of their sign).  The second
// conversion writes the high half of the first one's result.
__device__ __forceinline__ uint32_t mx_encode4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, int shared) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(b0, shared), mx_scaled(b1, shared), 0, false);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(b2, shared), mx_scaled(b3, shared), lo, true));
}

}  // namespace moe
