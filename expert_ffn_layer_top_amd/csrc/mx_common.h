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

// floor(log2(amax)) - 8 clamped to [-127, 127], from the magnitude bits of a bf16 amax
// (amax_bits = max over the block of (bits & 0x7fff)).  Returns -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  const int eb = static_cast<int>(amax_bits >> 7);
  int e;
  if (eb > 0) {
    e = eb - 127;
  } else {                                   // bf16 subnormal: m * 2^-133, m in [1, 127]
    e = (31 - __clz(static_cast<int>(amax_bits & 0x7f))) - 133;
  }
  int s = e - 8;
  s = s < -127 ? -127 : s;
  s = s > 127 ? 127 : s;
  return s;
}

// E4M3 code of bf16 value `b` divided by 2^shared (round-to-nearest-even, saturating).
__device__ __forceinline__ uint32_t mx_encode(uint32_t b, int shared) {
  const uint32_t sign = (b & 0x8000u) ? 0x80u : 0u;
  const uint32_t mag = b & 0x7fffu;
  float a;
  if ((mag >> 7) != 0) {
    // normal bf16: scale by 2^-shared (a normal fp32 power of two); exact unless the result
    // is below 2^-126, where the E4M3 code is a signed zero either way
    a = __uint_as_float(mag << 16) * __uint_as_float(static_cast<uint32_t>(127 - shared) << 23);
  } else {
    // bf16 subnormal m * 2^-133: build m * 2^(-133 - shared) without touching fp32 denormals
    const int ex = -133 - shared;
    a = (ex < -126) ? 0.f : static_cast<float>(mag) * __uint_as_float(static_cast<uint32_t>(ex + 127) << 23);
  }
  a = fminf(a, 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: E4M3 subnormal spacing 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));   // 0..8 (8 = smallest normal)
  } else {
    const uint32_t u = __float_as_uint(a);
    const uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;  // exponent|3-bit mantissa, RNE
    code = r - (120u << 3);                  // rebias 127 -> 7
  }
  return code | sign;
}

}  // namespace moe
