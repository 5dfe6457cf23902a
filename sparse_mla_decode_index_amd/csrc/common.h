// Device helpers shared by every decode kernel of libsmd (gfx950, MI355X):
// vector types, the zero row read in place of masked rows, the XOR swizzles
// of the LDS tiles, cross-lane reductions, fp32 -> bf16 rounding, UE8M0
// scales and the output scaling of the softmax epilogues.
//
// The softmax epilogue follows the vLLM page "[ROCm][DSV4][Perf] Optimize
// Triton sparse-MLA decode on gfx950", section Design (attention sinks in the
// denominator), and the aiter page "[ASM][HIP][MLA v4 nm] Split plan helper
// and persistent decode kernel", Summary part 1 (split partials carry their
// own log-sum-exp; the merge folds the sink in once).
#pragma once

#include "smd_internal.h"

#include <math.h>

namespace smd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define SMD_LDS __attribute__((address_space(3)))
#define SMD_GLOBAL __attribute__((address_space(1)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// A row's reference max is fixed at its first tile with a valid entry; a later
// score more than this far above it (log2 domain) sends the work through an
// exact-max second pass, so every weight 2^(x - m_ref) stays <= 2^32 and the
// accumulators are never rescaled.
constexpr float kRefSlackLog2 = 32.f;

enum Pass { kPassMain = 0, kPassMax = 1, kPassFixed = 2 };

// A zero row read in place of every masked row (1 KiB of zero bytes: bf16
// zeros, e4m3 zeros and UE8M0 code 0).
static __device__ __attribute__((aligned(256))) uint8_t g_zero_row[1024];

// XOR permutation of the 16-byte chunks of row r of a 16-row tile (rows r and
// r+16 share it).  A bijection on 0..15 that maps rows 0..7 / 8..15 to even /
// odd values: the 16-byte reads of one chunk column of 16 consecutive rows and
// the 8-byte transposed reads of 8 rows x 32 bytes both touch distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// XOR permutation of the 16-byte chunks of row r of a 32-row tile read by
// 32x32 MFMA operands: f(r) = 4 (r mod 4) + (floor(r/4) mod 4).  A bijection
// on each 16 consecutive rows (one chunk column of rows 0..15 or 16..31 is
// conflict-free), and four consecutive rows r = 4k..4k+3 put any aligned
// 64-byte group of chunks into four distinct 64-byte bank groups (the
// transposed V reads, 4 rows x 64 bytes per half wave).
__device__ __forceinline__ int swz32(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four 16-lane groups (lanes j, j+16, j+32, j+48) with the
// gfx950 permlane swaps (VALU, no LDS round trip).
__device__ __forceinline__ float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max / sum of lanes l and l ^ 32 (the two halves of a 32x32 MFMA column).
__device__ __forceinline__ float half_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values -> two bf16 packed low-first, rounded to nearest even by
// v_cvt_pk_bf16_f32 (the same result as f32_to_bf16_rne for every non-NaN
// fp32 bit pattern, checked exhaustively on gfx950; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two packed bf16 (pack_bf16x2 order) back to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Four fp32 values x scale -> four bf16 (round to nearest even), 8 bytes.
__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 v, float scale) {
  u32x2 r;
  r[0] = pack_bf16x2(v[0] * scale, v[1] * scale);
  r[1] = pack_bf16x2(v[2] * scale, v[3] * scale);
  return r;
}

// UE8M0 code -> fp32 scale 2^(code-127).  Code 0 is the subnormal 2^-127.
__device__ __forceinline__ float ue8m0_scale(uint32_t code) {
  return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
}

// Scale of an accumulated row and its log-sum-exp.
struct OutScale {
  float inv;  // multiplies the unnormalised accumulator
  float lse;  // natural log
};

// Final output of a row whose weights were taken relative to m (log2 domain)
// and sum to l, with the sink logit sink_ln (natural domain, -inf for none)
// folded in: out = O / (l + e^(sink - m)), lse = m + ln(l + e^(sink - m)).
// Nothing and no sink gives out = 0, lse = -inf.
__device__ __forceinline__ OutScale direct_scale(float m, float l, float sink_ln) {
  const float sink2 = sink_ln * kLog2e;
  const float mf = fmaxf(m, sink2);
  OutScale s{0.f, -INFINITY};
  if (mf != -INFINITY) {
    const float e = exp2_fast(m - mf);
    const float z = l * e + exp2_fast(sink2 - mf);
    s.inv = e / z;
    s.lse = (mf + __log2f(z)) * kLn2;
  }
  return s;
}

// A split partial (no sink): o = O / l, lse = m + ln l; empty: o = 0, lse = -inf.
__device__ __forceinline__ OutScale partial_scale(float m, float l) {
  OutScale s{0.f, -INFINITY};
  if (l > 0.f) {
    s.inv = 1.f / l;
    s.lse = (m + __log2f(l)) * kLn2;
  }
  return s;
}

}  // namespace smd
