// fp8/UE8M0 KV-cache writer for gfx950: bf16 latent rows -> the fp8 pool the
// decode reads (448 OCP E4M3FN bytes + 7 UE8M0 codes + 1 pad byte + 64 bf16
// RoPE dims per row).
//
// The vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on
// gfx950", Design, says that on gfx950 both cache writers cap the UE8M0 codes
// at 254 and canonicalise RoPE NaNs.  The block rule: for each 64-dim NoPE
// block, code c = clamp(ceil(log2(amax / 448)) + 127, 0, 254) (amax the
// largest |x|, NaN ignored; c = 0 for an empty block), and each value is
// stored as the E4M3FN byte nearest to x * 2^(127 - c), ties to the even
// mantissa, non-saturating (overflow and infinities give NaN with the sign).
//
// One wave per row, 8 values (16 bytes) per lane: lanes 0..55 the NoPE dims
// (lanes 8b..8b+7 = block b), lanes 56..63 the RoPE dims.  HBM-bound: 1 KiB
// read and 584 bytes written per row, coalesced.
#include "smd_internal.h"

#include <math.h>

namespace smd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// OCP E4M3FN byte of y, round to nearest even, non-saturating.
__device__ __forceinline__ uint32_t e4m3fn_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a < 0x3C800000u) {                       // below 2^-6: multiples of 2^-9 (and zero)
    const float q = rintf(__uint_as_float(a) * 512.f);  // exact scaling; 0..8
    return sign | (uint32_t)q;                 // 8 is 2^-6, the smallest normal
  }
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);  // round the mantissa to 3 bits
  const int e = (int)(r >> 23) - 127;
  if (e > 8) return sign | 0x7Fu;              // past 464 (and infinity): NaN
  return sign | ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);  // e = 8, mantissa 7 is NaN too
}

__global__ __launch_bounds__(256) void write_kv_fp8_kernel(WriterArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.num_rows) return;
  const int64_t dst = a.slots ? (int64_t)a.slots[r] : (int64_t)r;
  if (dst < 0 || dst >= a.pool_rows) return;  // wave-uniform
  const u32x4 v = *(const u32x4 *)(a.kv + (int64_t)r * a.kv_stride + 8 * lane);
  if (lane >= kNope / 8) {  // RoPE: copied, every NaN made canonical
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = v[i] & 0xFFFFu, hi = v[i] >> 16;
      if ((lo & 0x7F80u) == 0x7F80u && (lo & 0x7Fu)) lo = 0x7FC0u;
      if ((hi & 0x7F80u) == 0x7F80u && (hi & 0x7Fu)) hi = 0x7FC0u;
      o[i] = lo | (hi << 16);
    }
    *(u32x4 *)(a.rope + dst * a.rope_stride + 8 * (lane - kNope / 8)) = o;
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));  // fmaxf ignores NaN
  // block maximum over the 8 lanes of the block (the RoPE lanes reduce among themselves, unused)
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const uint32_t c = ue8m0_code(m);
  if (lane < kNope / 8) {
    u32x2 bytes = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) bytes[i >> 2] |= e4m3fn_rne(ldexpf(x[i], 127 - (int)c)) << (8 * (i & 3));
    *(u32x2 *)(a.nope + dst * a.nope_stride + 8 * lane) = bytes;
    if ((lane & 7) == 0) a.scale[dst * a.scale_stride + (lane >> 3)] = (uint8_t)c;
  } else if (lane == kNope / 8) {
    a.scale[dst * a.scale_stride + 7] = 0;  // pad byte
  }
}

hipError_t launch_write_kv_fp8(const WriterArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.num_rows + 3) / 4));
  hipLaunchKernelGGL(write_kv_fp8_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smd
