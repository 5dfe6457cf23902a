// Split-KV sparse MLA decode and stage-2 merge kernels for gfx950 (MI355X).
//
// Split partials and their merge follow the aiter page "[ASM][HIP][MLA v4 nm]
// Split plan helper and persistent decode kernel", Summary part 1: split r of
// an index row covers a contiguous range of its positions and writes an FP32
// partial (o_r, lse_r); the merge reweights the partials by their log-sum-exps
// and folds in the sink.  One split writes the bf16 output directly.
#include "decode_core.h"

namespace smd {

// Work decomposition: a workgroup (4 waves) owns one index row b, one group g
// of 16*RB query rows and one split r.
template <int RB, bool FP8, bool PACKED, bool P_HILO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 2 : 1, RB == 1 ? 2 : 1))) void decode_kernel(DecodeArgs a) {
  constexpr int DS = 4 / RB;
  constexpr int NC = 16 / DS, ND = 32 / DS;
  __shared__ __attribute__((aligned(1024))) Smem<DS> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rb = wave % RB, ds = wave / RB;
  const int j = lane & 15;   // query row within the wave's block / column
  const int grp = lane >> 4; // 16-lane group

  // Workgroup -> (work unit u = b*S + r, row group g).  The G row groups of a
  // unit read the same KV rows; consecutive workgroups land on consecutive
  // XCDs, so the groups of one unit are spaced 8 apart to share one XCD's L2.
  const int per = 8 * a.G;
  const int g = (int)(blockIdx.x % per) / 8;
  const int u = (int)(blockIdx.x / per) * 8 + (int)(blockIdx.x % 8);
  if (u >= a.num_units) return;
  const int b = u / a.S;
  const int r = u % a.S;
  const int p0 = min(r * a.chunk, a.topk);
  const int p1 = min(p0 + a.chunk, a.topk);
  const int32_t *row_idx = a.indices + (int64_t)b * a.indices_stride;

  // This lane's query row m -> (token, head).
  const int m = g * (RB * 16) + rb * 16 + j;
  const int tok = b * a.qps + m / a.H;
  const int head = m % a.H;
  const int64_t qrow = (int64_t)tok * a.H + head;  // [T, H] row

  bf16x8 qreg[NC];
  load_q<DS>(a, qrow, ds, grp, qreg);
  int qk_base[4], pv_base[8];
  lds_bases(j, grp, qk_base, pv_base);

  WaveState<ND> w;
  attend_range<RB, FP8, PACKED, P_HILO>(a, sm, row_idx, p0, p1, wave, lane, grp, ds, qreg, qk_base, pv_base, w);

  const float l_tot = row_total(w.l_run);
  const int dcol = 16 * (ds * ND) + 4 * grp;
  const bool lse_lane = grp == 0 && ds == 0;
  if (a.S == 1 && a.out != nullptr) {
    write_direct(w, l_tot, a.sink ? a.sink[head] : -INFINITY, a.out + qrow * kDim + dcol,
                 (a.lse != nullptr && lse_lane) ? a.lse + qrow : nullptr);
  } else {
    write_partial(w, l_tot, a.part_o + (qrow * a.S + r) * kDim + dcol,
                  lse_lane ? a.part_lse + qrow * a.S + r : nullptr);
  }
}

// Stage-2 merge: one wave per [T,H] row, 8 dims per lane.
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ po,
                                                    const float *__restrict__ plse, int rows, int H,
                                                    int S, const float *__restrict__ sink,
                                                    uint16_t *__restrict__ out, float *__restrict__ lse) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int head = row % H;
  const float *ls = plse + (int64_t)row * S;
  float mx = sink ? sink[head] : -INFINITY;
  for (int r = 0; r < S; ++r) mx = fmaxf(mx, ls[r]);
  uint16_t *dst = out + (int64_t)row * kDim + lane * 8;
  if (mx == -INFINITY) {
    *(u32x4 *)dst = u32x4{0u, 0u, 0u, 0u};
    if (lse && lane == 0) lse[row] = -INFINITY;
    return;
  }
  float z = sink ? exp2_fast((sink[head] - mx) * kLog2e) : 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float *src = po + (int64_t)row * S * kDim + lane * 8;
  for (int r = 0; r < S; ++r) {
    const float w = exp2_fast((ls[r] - mx) * kLog2e);
    z += w;
    const f32x4 v0 = *(const f32x4 *)(src + (int64_t)r * kDim);
    const f32x4 v1 = *(const f32x4 *)(src + (int64_t)r * kDim + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] += w * v0[i];
      o[4 + i] += w * v1[i];
    }
  }
  const float inv = 1.f / z;
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (uint32_t)f32_to_bf16_rne(o[2 * i] * inv) | ((uint32_t)f32_to_bf16_rne(o[2 * i + 1] * inv) << 16);
  *(u32x4 *)dst = v;
  if (lse && lane == 0) lse[row] = mx + logf(z);
}

template <int RB, bool FP8, bool PACKED, bool P_HILO>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_kernel<RB, FP8, PACKED, P_HILO>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int RB, bool P_HILO>
static hipError_t launch_decode_rb(const DecodeArgs &a, bool fp8, hipStream_t stream) {
  if (fp8) return launch_decode_t<RB, true, false, P_HILO>(a, stream);
  return a.packed ? launch_decode_t<RB, false, true, P_HILO>(a, stream)
                  : launch_decode_t<RB, false, false, P_HILO>(a, stream);
}

template <bool P_HILO>
static hipError_t launch_decode_p(const DecodeArgs &a, int rb, bool fp8, hipStream_t stream) {
  switch (rb) {
    case 1: return launch_decode_rb<1, P_HILO>(a, fp8, stream);
    case 2: return launch_decode_rb<2, P_HILO>(a, fp8, stream);
    case 4: return launch_decode_rb<4, P_HILO>(a, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

// Partials the caller reads are written with the two-part P (FP32-partial
// precision); partials that only feed the merge into bf16, and the direct
// bf16 output, use a single bf16 P.
hipError_t launch_decode(const DecodeArgs &a, int rb, bool fp8, hipStream_t stream) {
  return a.hilo ? launch_decode_p<true>(a, rb, fp8, stream) : launch_decode_p<false>(a, rb, fp8, stream);
}

hipError_t launch_merge(const float *part_o, const float *part_lse, int32_t rows, int32_t H,
                        int32_t S, const float *sink, uint16_t *out, float *lse,
                        hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, stream, part_o, part_lse, rows, H, S, sink,
                     out, lse);
  return hipGetLastError();
}

}  // namespace smd
