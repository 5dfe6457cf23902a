// Split-KV sparse MLA decode and stage-2 merge kernels for gfx950 (MI355X).
//
// Split partials and their merge follow the aiter page "[ASM][HIP][MLA v4 nm]
// Split plan helper and persistent decode kernel", Summary part 1: split r of
// an index row covers a contiguous range of its positions and writes an FP32
// partial (o_r, lse_r); the merge reweights the partials by their log-sum-exps
// and folds in the sink.  One split writes the bf16 output directly.
#include "kp_core.h"
#include "ks8_core.h"

namespace smd {

using namespace ks;

// Work decomposition: a workgroup (8 waves, two per SIMD) owns one index row
// b, one block g of 16 query rows and one split r; its waves share the split's
// positions (interleaved half-tiles of 16) and merge their states at the end.
template <int FMT, bool P_HILO, bool TWO>
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
  const ks::Src<TWO> src{a.indices + (int64_t)b * a.indices_stride,
                         TWO ? a.indices2 + (int64_t)b * a.indices2_stride : nullptr, a.k_main};

  const ks::Lane L = ks::make_lane(lane);
  // This lane's query row m -> (token, head).
  const int m = g * 16 + L.j;
  const int tok = b * a.qps + m / a.H;
  const int head = m % a.H;
  const int64_t qrow = (int64_t)tok * a.H + head;  // [T, H] row

  // the first indices and rows are in flight while Q^T is staged
  ks8::Pipe<FMT> pipe;
  ks8::prime<FMT>(a, src, p0, p1, wave, L, pipe);
  ks8::stage_q(a, qrow, wave, L, sm);
  __syncthreads();
  ks::State st;
  ks8::attend<FMT, P_HILO>(a, src, p0, p1, wave, L, (const uint8_t SMD_LDS *)&sm.q[0],
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
    ks::write_partial_any(a.hilo != 0, o, mm, ll, a.part_o, (qrow * a.S + r) * kDim + dcol,
                          lse_lane ? a.part_lse + qrow * a.S + r : nullptr);
  }
}

// Work decomposition of the dim-split variant: a workgroup (8 waves = 4 pairs
// of dim halves) owns one index row b, one block g of 32 query rows and one
// split r; a.G = M / 32.  Mapping to the grid as in decode_kernel.
template <int FMT, bool P_HILO, bool TWO>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_kp_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) kp::Smem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int per = 8 * a.G;
  const int g = (int)(blockIdx.x % per) / 8;
  const int u = (int)(blockIdx.x / per) * 8 + (int)(blockIdx.x % 8);
  if (u >= a.num_units) return;
  const int b = u / a.S;
  const int r = u % a.S;
  const int p0 = min(r * a.chunk, a.topk);
  const int p1 = min(p0 + a.chunk, a.topk);
  const ks::Src<TWO> src{a.indices + (int64_t)b * a.indices_stride,
                         TWO ? a.indices2 + (int64_t)b * a.indices2_stride : nullptr, a.k_main};

  const ks::Lane L = ks::make_lane(lane);
  const kp::PLane P = kp::make_plane(L);
  int64_t qrow[2];
  int head[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int m = g * kp::kRows + 16 * qb + L.j;
    head[qb] = m % a.H;
    qrow[qb] = (int64_t)(b * a.qps + m / a.H) * a.H + head[qb];
  }
  const int k = wave >> 1, h = wave & 1;

  kp::Pipe<FMT> pipe;
  if (p1 > p0) kp::prime<FMT>(a, src, p0, p1, k, h, L, pipe);  // workgroup-uniform
  kp::stage_q(a, qrow, wave, L, sm);
  if (lane == 0) sm.flag[wave] = 0;
  __syncthreads();
  kp::State st;
  kp::attend<FMT, P_HILO>(a, src, p0, p1, wave, L, P, sm, st, pipe);
  if (!kp::merge_pairs(sm, wave, L, st)) return;
  // waves 0 and 1: dims [256h, 256h + 256) of both blocks
  const int dcol = 256 * h + 4 * L.g;
  const bool lse_lane = L.g == 0 && h == 0;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = ks::group_sum(st.l_run[qb]);
    ks::f32x4 lo[8], hi[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      lo[d] = st.acc[2 * d + qb];
      hi[d] = st.acc[2 * (8 + d) + qb];
    }
    if (a.S == 1 && a.out != nullptr) {
      uint16_t *dst = a.out + qrow[qb] * kDim + dcol;
      const float sk = a.sink ? a.sink[head[qb]] : -INFINITY;
      ks::write_direct(lo, st.m_ref[qb], l, sk, dst, (a.lse != nullptr && lse_lane) ? a.lse + qrow[qb] : nullptr);
      ks::write_direct(hi, st.m_ref[qb], l, sk, dst + 128, nullptr);
    } else {
      const int64_t off = (qrow[qb] * a.S + r) * kDim + dcol;
      ks::write_partial_any(a.hilo != 0, lo, st.m_ref[qb], l, a.part_o, off,
                            lse_lane ? a.part_lse + qrow[qb] * a.S + r : nullptr);
      ks::write_partial_any(a.hilo != 0, hi, st.m_ref[qb], l, a.part_o, off + 128, nullptr);
    }
  }
}

// Stage-2 merge.  WPR waves share one [T,H] row (8 dims per lane); wave w of
// the row folds the partials r = w, w + WPR, ... into a running max / sum,
// reading CH of them (their lse and o) per round trip, so a plan of up to
// CH * WPR splits costs one round trip.  The row's waves then combine
// their states through LDS and the row's first wave writes the result.
// A workgroup has max(4, WPR) waves, so 4 / WPR rows or one.
// BF16: the partials' o values are bf16 (in the FP32 buffer's first half),
// the form of partials that only feed this merge.
template <int WPR>
constexpr int merge_waves() {
  return WPR > 4 ? WPR : 4;
}

template <int WPR, int CH, bool BF16>
__global__ __launch_bounds__(64 * merge_waves<WPR>()) void merge_kernel(const float *__restrict__ po,
                                                                        const float *__restrict__ plse, int rows,
                                                                        int H, int S, const float *__restrict__ sink,
                                                                        uint16_t *__restrict__ out,
                                                                        float *__restrict__ lse) {
  constexpr int NW = merge_waves<WPR>();
  __shared__ float xo[NW][8][64];  // [wave][dim][lane]: bank-conflict-free
  __shared__ float xs[NW][2];      // [wave] {max, sum}
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int w = wave % WPR;
  const int row = blockIdx.x * (NW / WPR) + wave / WPR;
  const bool live = row < rows;
  float mx = -INFINITY;  // running max of the lse terms (natural log)
  float z = 0.f;         // sum of e^(term - mx)
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float *ls = plse + (int64_t)row * S;
    const float *src = po + (int64_t)row * S * kDim + lane * 8;
    const uint16_t *srcb = (const uint16_t *)po + (int64_t)row * S * kDim + lane * 8;
    if (w == 0 && sink) {
      mx = sink[row % H];
      z = mx == -INFINITY ? 0.f : 1.f;
    }
    for (int r0 = w; r0 < S; r0 += CH * WPR) {
      float l[CH];
      f32x4 v[CH][2];
      u32x4 vb[CH];  // BF16: the raw values, widened where they are used (all loads issue first)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int rr = r0 + c * WPR;
        const int r = rr < S ? rr : r0;  // clamped: every chunk issues the same loads
        l[c] = rr < S ? ls[r] : -INFINITY;
        if constexpr (BF16) {
          vb[c] = *(const u32x4 *)(srcb + (int64_t)r * kDim);
        } else {
          v[c][0] = *(const f32x4 *)(src + (int64_t)r * kDim);
          v[c][1] = *(const f32x4 *)(src + (int64_t)r * kDim + 4);
        }
      }
      float cm = l[0];
#pragma unroll
      for (int c = 1; c < CH; ++c) cm = fmaxf(cm, l[c]);
      if (cm == -INFINITY) continue;
      const float nm = fmaxf(mx, cm);
      const float rescale = mx == -INFINITY ? 0.f : exp2_fast((mx - nm) * kLog2e);
      z *= rescale;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= rescale;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const float e = l[c] == -INFINITY ? 0.f : exp2_fast((l[c] - nm) * kLog2e);
        z += e;
        if constexpr (BF16) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            v[c][i][0] = __uint_as_float(vb[c][2 * i] << 16);
            v[c][i][1] = __uint_as_float(vb[c][2 * i] & 0xffff0000u);
            v[c][i][2] = __uint_as_float(vb[c][2 * i + 1] << 16);
            v[c][i][3] = __uint_as_float(vb[c][2 * i + 1] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] += e * v[c][0][i];
          o[4 + i] += e * v[c][1][i];
        }
      }
      mx = nm;
    }
  }
  if constexpr (WPR > 1) {
    if (w != 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) xo[wave][i][lane] = o[i];
      if (lane == 0) {
        xs[wave][0] = mx;
        xs[wave][1] = z;
      }
    }
    __syncthreads();
    if (w != 0 || !live) return;
    float m2[WPR], z2[WPR];
    float nm = mx;
#pragma unroll
    for (int k = 1; k < WPR; ++k) {
      m2[k] = xs[wave + k][0];
      z2[k] = xs[wave + k][1];
      nm = fmaxf(nm, m2[k]);
    }
    if (nm != -INFINITY) {
      const float e0 = mx == -INFINITY ? 0.f : exp2_fast((mx - nm) * kLog2e);
      z *= e0;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= e0;
#pragma unroll
      for (int k = 1; k < WPR; ++k) {
        const float e = m2[k] == -INFINITY ? 0.f : exp2_fast((m2[k] - nm) * kLog2e);
        z += e * z2[k];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] += e * xo[wave + k][i][lane];
      }
    }
    mx = nm;
  }
  if (!live) return;
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
    vo[i] = pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
  *(u32x4 *)dst = vo;
  if (lse && lane == 0) lse[row] = mx + logf(z);
}

template <int FMT, bool P_HILO, bool TWO>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_kernel<FMT, P_HILO, TWO>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int FMT, bool P_HILO, bool TWO>
static hipError_t launch_decode_kp_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_kp_kernel<FMT, P_HILO, TWO>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int FMT, bool TWO>
static hipError_t launch_decode_s(const DecodeArgs &a, bool pairs, hipStream_t stream) {
  if (pairs)
    return a.hilo ? launch_decode_kp_t<FMT, true, TWO>(a, stream) : launch_decode_kp_t<FMT, false, TWO>(a, stream);
  return a.hilo ? launch_decode_t<FMT, true, TWO>(a, stream) : launch_decode_t<FMT, false, TWO>(a, stream);
}

template <int FMT>
static hipError_t launch_decode_f(const DecodeArgs &a, bool pairs, hipStream_t stream) {
  return a.indices2 ? launch_decode_s<FMT, true>(a, pairs, stream) : launch_decode_s<FMT, false>(a, pairs, stream);
}

// Partials the caller reads are written with the two-part P (FP32-partial
// precision); partials that only feed the merge into bf16, and the direct
// bf16 output, use a single bf16 P.  a.G must be M / 32 with pairs (the
// dim-split kernel), M / 16 without.  a.indices2 non-null: two sources.
hipError_t launch_decode(const DecodeArgs &a, bool fp8, bool pairs, hipStream_t stream) {
  static_assert((int)kp::kBf16Packed == (int)ks8::kBf16Packed && (int)kp::kFp8 == (int)ks8::kFp8, "formats");
  if (fp8) return launch_decode_f<ks8::kFp8>(a, pairs, stream);
  return a.packed ? launch_decode_f<ks8::kBf16Packed>(a, pairs, stream)
                  : launch_decode_f<ks8::kBf16Split>(a, pairs, stream);
}

template <int WPR, int CH, bool BF16>
static hipError_t launch_merge_t(const float *part_o, const float *part_lse, int32_t rows, int32_t H,
                                 int32_t S, const float *sink, uint16_t *out, float *lse,
                                 hipStream_t stream) {
  constexpr int NW = merge_waves<WPR>();
  const int rpb = NW / WPR;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  hipLaunchKernelGGL((merge_kernel<WPR, CH, BF16>), grid, dim3(64 * NW), 0, stream, part_o, part_lse, rows, H,
                     S, sink, out, lse);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_merge_f(const float *part_o, const float *part_lse, int32_t rows, int32_t H,
                                 int32_t S, const float *sink, uint16_t *out, float *lse,
                                 hipStream_t stream) {
  if (S <= 4) return launch_merge_t<1, 4, BF16>(part_o, part_lse, rows, H, S, sink, out, lse, stream);
  if (S <= 8) return launch_merge_t<2, 4, BF16>(part_o, part_lse, rows, H, S, sink, out, lse, stream);
  if (S <= 16) return launch_merge_t<4, 4, BF16>(part_o, part_lse, rows, H, S, sink, out, lse, stream);
  if (S <= 64) return launch_merge_t<4, 8, BF16>(part_o, part_lse, rows, H, S, sink, out, lse, stream);
  // long plans: 16 waves per row, so up to 128 splits cost one round trip
  return launch_merge_t<16, 8, BF16>(part_o, part_lse, rows, H, S, sink, out, lse, stream);
}

hipError_t launch_merge(const float *part_o, const float *part_lse, int32_t rows, int32_t H,
                        int32_t S, const float *sink, uint16_t *out, float *lse,
                        hipStream_t stream, bool bf16_parts) {
  return bf16_parts ? launch_merge_f<true>(part_o, part_lse, rows, H, S, sink, out, lse, stream)
                    : launch_merge_f<false>(part_o, part_lse, rows, H, S, sink, out, lse, stream);
}

}  // namespace smd
