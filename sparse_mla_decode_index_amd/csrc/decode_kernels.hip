// Split-KV sparse MLA decode and stage-2 merge kernels for gfx950 (MI355X).
//
// Split partials and their merge follow the aiter page "[ASM][HIP][MLA v4 nm]
// Split plan helper and persistent decode kernel", Summary part 1: split r of
// an index row covers a contiguous range of its positions and writes an FP32
// partial (o_r, lse_r); the merge reweights the partials by their log-sum-exps
// and folds in the sink.  One split writes the bf16 output directly.
#include "ks8_core.h"

namespace smd {

using namespace ks;

// Work decomposition: a workgroup (8 waves, two per SIMD) owns one index row
// b, one block g of 16 query rows and one split r; its waves share the split's
// positions (interleaved half-tiles of 16) and merge their states at the end.
template <bool PACKED, bool P_HILO>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) ks8::Smem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform

  // Workgroup -> (work unit u = b*S + r, row block g).  The G blocks of a unit
  // read the same KV rows; consecutive workgroups land on consecutive XCDs,
  // so the blocks of one unit are spaced 8 apart to share one XCD's L2.
  const int per = 8 * a.G;
  const int g = (int)(blockIdx.x % per) / 8;
  const int u = (int)(blockIdx.x / per) * 8 + (int)(blockIdx.x % 8);
  if (u >= a.num_units) return;
  const int b = u / a.S;
  const int r = u % a.S;
  const int p0 = min(r * a.chunk, a.topk);
  const int p1 = min(p0 + a.chunk, a.topk);
  const int32_t *row_idx = a.indices + (int64_t)b * a.indices_stride;

  const ks::Lane L = ks::make_lane(lane);
  // This lane's query row m -> (token, head).
  const int m = g * 16 + L.j;
  const int tok = b * a.qps + m / a.H;
  const int head = m % a.H;
  const int64_t qrow = (int64_t)tok * a.H + head;  // [T, H] row

  // the first indices and rows are in flight while Q^T is staged
  ks8::Pipe pipe;
  ks8::prime<PACKED>(a, row_idx, p0, p1, wave, L, pipe);
  ks8::stage_q(a, qrow, wave, L, sm);
  __syncthreads();
  ks::State st;
  ks8::attend<PACKED, P_HILO>(a, row_idx, p0, p1, wave, L, (const uint8_t SMD_LDS *)&sm.q[0],
                              (uint8_t SMD_LDS *)&sm.buf[wave][0], st, pipe);
  ks::f32x4 o[8];
  float mm, ll;
  if (!ks8::merge_waves(sm, wave, L, st, o, mm, ll)) return;
  const int dcol = 128 * wave + 4 * L.g;
  const bool lse_lane = L.g == 0 && wave == 0;
  if (a.S == 1 && a.out != nullptr) {
    ks::write_direct(o, mm, ll, a.sink ? a.sink[head] : -INFINITY, a.out + qrow * kDim + dcol,
                     (a.lse != nullptr && lse_lane) ? a.lse + qrow : nullptr);
  } else {
    ks::write_partial(o, mm, ll, a.part_o + (qrow * a.S + r) * kDim + dcol,
                      lse_lane ? a.part_lse + qrow * a.S + r : nullptr);
  }
}

// Stage-2 merge: one wave per [T,H] row, 8 dims per lane.  The partials are
// read four at a time (their lse and o in one round trip) and folded into a
// running max / sum, so a plan of up to four splits costs one round trip.
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ po,
                                                    const float *__restrict__ plse, int rows, int H,
                                                    int S, const float *__restrict__ sink,
                                                    uint16_t *__restrict__ out, float *__restrict__ lse) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int head = row % H;
  const float *ls = plse + (int64_t)row * S;
  const float *src = po + (int64_t)row * S * kDim + lane * 8;
  const float sk = sink ? sink[head] : -INFINITY;
  float mx = sk;   // running max of the lse terms (natural log)
  float z = 1.f;   // sum of e^(term - mx) (the sink, or nothing yet)
  if (mx == -INFINITY) z = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < S; r0 += 4) {
    float l[4];
    f32x4 v[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = min(r0 + c, S - 1);  // clamped: every chunk issues the same loads
      l[c] = r0 + c < S ? ls[r] : -INFINITY;
      v[c][0] = *(const f32x4 *)(src + (int64_t)r * kDim);
      v[c][1] = *(const f32x4 *)(src + (int64_t)r * kDim + 4);
    }
    const float cm = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
    if (cm == -INFINITY) continue;
    const float nm = fmaxf(mx, cm);
    const float rescale = mx == -INFINITY ? 0.f : exp2_fast((mx - nm) * kLog2e);
    z *= rescale;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= rescale;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float w = l[c] == -INFINITY ? 0.f : exp2_fast((l[c] - nm) * kLog2e);
      z += w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] += w * v[c][0][i];
        o[4 + i] += w * v[c][1][i];
      }
    }
    mx = nm;
  }
  uint16_t *dst = out + (int64_t)row * kDim + lane * 8;
  if (mx == -INFINITY) {
    *(u32x4 *)dst = u32x4{0u, 0u, 0u, 0u};
    if (lse && lane == 0) lse[row] = -INFINITY;
    return;
  }
  const float inv = 1.f / z;
  u32x4 vo;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    vo[i] = (uint32_t)f32_to_bf16_rne(o[2 * i] * inv) | ((uint32_t)f32_to_bf16_rne(o[2 * i + 1] * inv) << 16);
  *(u32x4 *)dst = vo;
  if (lse && lane == 0) lse[row] = mx + logf(z);
}

template <bool PACKED, bool P_HILO>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_kernel<PACKED, P_HILO>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

// bf16 pools (fp8 pools go to launch_decode_rb).  Partials the caller reads
// are written with the two-part P (FP32-partial precision); partials that only
// feed the merge into bf16, and the direct bf16 output, use a single bf16 P.
// a.G must be M / 16.
hipError_t launch_decode(const DecodeArgs &a, bool fp8, hipStream_t stream) {
  if (fp8) return hipErrorInvalidValue;
  if (a.hilo) return a.packed ? launch_decode_t<true, true>(a, stream) : launch_decode_t<false, true>(a, stream);
  return a.packed ? launch_decode_t<true, false>(a, stream) : launch_decode_t<false, false>(a, stream);
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
