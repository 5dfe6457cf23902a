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
// A wave per row (two rows, loaded together, for large writes), 8 values
// (16 bytes) per lane: lanes 0..55 the NoPE dims (lanes 8b..8b+7 = block b),
// lanes 56..63 the RoPE dims.  HBM-bound: 1 KiB read and 584 bytes written
// per row, coalesced.
#include "quant.h"

namespace smd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Largest value over each group of 8 lanes: swaps within quads (lane ^ 1,
// lane ^ 2), then lane i with lane 7 - i of its half-row.
__device__ __forceinline__ float max_over8(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));
  return m;
}

// Each wave writes RPW rows, their loads issued together.
template <int RPW>
__global__ __launch_bounds__(256) void write_kv_fp8_kernel(WriterArgs a) {
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
  int64_t dst[RPW];
  u32x4 v[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = r0 + k;
    dst[k] = r < a.num_rows ? (a.slots ? (int64_t)a.slots[r] : (int64_t)r) : -1;
    if (dst[k] >= a.pool_rows) dst[k] = -1;  // past the pool: skipped like -1
  }
#pragma unroll
  for (int k = 0; k < RPW; ++k)
    if (dst[k] >= 0) v[k] = *(const u32x4 *)(a.kv + (int64_t)(r0 + k) * a.kv_stride + 8 * lane);
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    if (dst[k] < 0) continue;  // wave-uniform
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[k][i] << 16);
      x[2 * i + 1] = __uint_as_float(v[k][i] & 0xFFFF0000u);
    }
    bool nan = false;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      nan |= x[i] != x[i];
      m = fmaxf(m, fabsf(x[i]));  // fmaxf ignores NaN
    }
    // block maximum (the RoPE lanes reduce among themselves, unused)
    const uint32_t c = ue8m0_code(max_over8(m));
    if (lane >= kNope / 8) {  // RoPE: copied, every NaN made canonical
      u32x4 o = v[k];
      if (nan) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t lo = o[i] & 0xFFFFu, hi = o[i] >> 16;
          if ((lo & 0x7F80u) == 0x7F80u && (lo & 0x7Fu)) lo = 0x7FC0u;
          if ((hi & 0x7F80u) == 0x7F80u && (hi & 0x7Fu)) hi = 0x7FC0u;
          o[i] = lo | (hi << 16);
        }
      }
      *(u32x4 *)(a.rope + dst[k] * a.rope_stride + 8 * (lane - kNope / 8)) = o;
      if (lane == kNope / 8) a.scale[dst[k] * a.scale_stride + 7] = 0;  // pad byte
    } else {
      const int e = 127 - (int)c;
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ldexpf(x[i], e);  // exact: powers of two
      // the hardware conversion rounds to nearest even like e4m3fn_rne on every
      // finite and infinite input; a NaN loses its sign there, so a lane holding
      // one converts in software
      u32x2 bytes;
      bytes[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      bytes[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)bytes[0], true);
      bytes[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      bytes[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)bytes[1], true);
      if (nan) {
        bytes[0] = bytes[1] = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) bytes[i >> 2] |= e4m3fn_rne(y[i]) << (8 * (i & 3));
      }
      *(u32x2 *)(a.nope + dst[k] * a.nope_stride + 8 * lane) = bytes;
      if ((lane & 7) == 0) a.scale[dst[k] * a.scale_stride + (lane >> 3)] = (uint8_t)c;
    }
  }
}

hipError_t launch_write_kv_fp8(const WriterArgs &a, hipStream_t stream) {
  // two rows per wave once the grid holds several waves per SIMD anyway
  // (more bytes in flight per wave); one row per wave for small writes
  if (a.num_rows >= 65536) {
    hipLaunchKernelGGL(write_kv_fp8_kernel<2>, dim3((unsigned)((a.num_rows + 7) / 8)), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(write_kv_fp8_kernel<1>, dim3((unsigned)((a.num_rows + 3) / 4)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace smd
