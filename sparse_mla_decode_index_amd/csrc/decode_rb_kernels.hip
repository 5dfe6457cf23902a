// Split-KV sparse MLA decode with row-block workgroups (used for fp8 pools).
//
// A workgroup of 4 waves shares each 32-row KV tile through LDS: wave w owns
// the 16 query rows of block w % RB and the 512/DS dims of slice w / RB
// (RB * DS = 4), so every gathered row enters the compute unit once and is
// read by all the query blocks.  The device core is in decode_core.h.
#include "decode_core.h"

namespace smd {

// Work decomposition: a workgroup (4 waves) owns one index row b, one group g
// of 16*RB query rows and one split r.
template <int RB, bool FP8, bool PACKED, bool P_HILO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 2 : 1, RB == 1 ? 2 : 1))) void decode_rb_kernel(DecodeArgs a) {
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

template <int RB, bool FP8, bool PACKED, bool P_HILO>
static hipError_t launch_rb_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_rb_kernel<RB, FP8, PACKED, P_HILO>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int RB, bool P_HILO>
static hipError_t launch_rb_rb(const DecodeArgs &a, bool fp8, hipStream_t stream) {
  if (!fp8) return hipErrorInvalidValue;  // bf16 pools use the wave-independent kernel
  return launch_rb_t<RB, true, false, P_HILO>(a, stream);
}

template <bool P_HILO>
static hipError_t launch_rb_p(const DecodeArgs &a, int rb, bool fp8, hipStream_t stream) {
  switch (rb) {
    case 1: return launch_rb_rb<1, P_HILO>(a, fp8, stream);
    case 2: return launch_rb_rb<2, P_HILO>(a, fp8, stream);
    case 4: return launch_rb_rb<4, P_HILO>(a, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

// Partials the caller reads are written with the two-part P (FP32-partial
// precision); otherwise a single bf16 P.  a.G must be M / (16 rb).
hipError_t launch_decode_rb(const DecodeArgs &a, int rb, bool fp8, hipStream_t stream) {
  return a.hilo ? launch_rb_p<true>(a, rb, fp8, stream) : launch_rb_p<false>(a, rb, fp8, stream);
}

}  // namespace smd
