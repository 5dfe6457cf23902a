// UE8M0 block codes and E4M3FN rounding on gfx950, shared by the fp8/UE8M0
// cache writer and the fp8 QK of the decode (which quantises q_nope the way
// the writer quantises a latent row's NoPE).
//
// The block rule follows the vLLM page "[ROCm][DSV4][Perf] Optimize Triton
// sparse-MLA decode on gfx950", Design (UE8M0 codes capped at 254 on gfx950):
// for each 64-dim NoPE block, c = clamp(ceil(log2(amax / 448)) + 127, 0, 254)
// (amax the largest |x|, NaN ignored; c = 0 for an empty block), and a value
// x is stored as the E4M3FN byte nearest to x * 2^(127 - c), ties to the even
// mantissa, non-saturating.
#pragma once

#include "smd_internal.h"

#include <math.h>

namespace smd {

// ceil(log2(amax / 448)) + 127 clamped to [0, 254] for amax > 0 (finite or
// infinite), from the float's fields: amax = (1 + f) 2^E, 448 = 1.75 * 2^8,
// so the ceiling is E - 8, plus one when the mantissa exceeds 1.75.
__device__ __forceinline__ uint32_t ue8m0_code(float amax) {
  if (!(amax > 0.f)) return 0u;       // zero, or every value NaN
  if (isinf(amax)) return 254u;
  int bias = 0;
  if (amax < 1.17549435e-38f) {       // fp32 subnormal: scale into the normal range (exact)
    amax *= 18446744073709551616.f;   // 2^64
    bias = 64;
  }
  const uint32_t u = __float_as_uint(amax);
  const int e = (int)(u >> 23) - 127 - bias;
  const int up = (u & 0x7FFFFFu) > 0x600000u;  // mantissa above 1.75
  const int c = e - 8 + up + 127;
  return (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
}

// OCP E4M3FN byte of y, round to nearest even, non-saturating, branch-free:
// below 2^-6 the result is a multiple of 2^-9, which the fp32 add to 2^14
// rounds to (its ulp is 2^-9); above, the mantissa is rounded to 3 bits with
// the carry into the exponent, and anything that lands past 0x7E (values
// beyond 464, infinities, NaN) saturates at the NaN code 0x7F.
__device__ __forceinline__ uint32_t e4m3fn_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t sub = __float_as_uint(fabsf(y) + 16384.0f) - 0x46800000u;
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t nrm = (r >> 20) - 960u;  // ((biased exponent - 120) << 3) | mantissa
  const uint32_t b = a < 0x3C800000u ? sub : nrm;
  return (b < 0x7Fu ? b : 0x7Fu) | ((u >> 24) & 0x80u);
}

}  // namespace smd
