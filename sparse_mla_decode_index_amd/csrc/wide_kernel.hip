// Split-KV sparse MLA decode on the wide waves (gfx950), for M = heads x MTP
// positions a multiple of 128: a workgroup of 4 waves owns one index row b,
// one split r and one group of 128 query rows, and every gathered 32-row tile
// serves all 128 of them (wide_core.h: 32x32x16 MFMAs, one wave per SIMD).
//
// Split partials and their merge follow the aiter page "[ASM][HIP][MLA v4 nm]
// Split plan helper and persistent decode kernel", Summary part 1: split r of
// an index row covers a contiguous range of its positions and writes an FP32
// partial (o_r, lse_r); one split writes the bf16 output with the sink
// folded in (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode
// on gfx950", Design: attention sinks, direct bf16 output when unsplit).
#include "wide_core.h"

namespace smd {

// QF8: the fp8 QK of wide_core.h (fp8 pools; options qk = SMD_QK_FP8).
template <bool FP8, bool PACKED, bool P_HILO, bool QF8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_wide_kernel(DecodeArgs a) {
  static_assert(!QF8 || FP8, "the fp8 QK reads an fp8 pool");
  constexpr bool RING = wide_ring<FP8>();
  constexpr bool RINGB = !FP8 && kWideBf16Ring;  // bf16 pools on the bf16 ring
  __shared__ __attribute__((aligned(1024)))
  std::conditional_t<QF8, SmemWideQ<7>, std::conditional_t<RINGB, SmemWideB, SmemWide<RING>>> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Workgroup -> (work unit u = b*S + r, row group g).  The G groups of a unit
  // read the same KV rows; consecutive workgroups land on consecutive XCDs,
  // so the groups of one unit are spaced 8 apart to share one XCD's L2.
  const int per = 8 * a.G;
  const int g = (int)(blockIdx.x % per) / 8;
  const int u = (int)(blockIdx.x / per) * 8 + (int)(blockIdx.x % 8);
  if (u >= a.num_units) return;
  const int b = u / a.S;
  const int r = u % a.S;
  const int p0 = min(r * a.chunk, a.topk);
  const int p1 = min(p0 + a.chunk, a.topk);

  // wave w owns query rows 32w .. 32w+31 of the group: the consecutive rows
  // qbase .. qbase + 31 of the queries (row b*M + m for query row m of index
  // row b); this lane's row is qbase + lane % 32
  const int64_t qbase = (int64_t)b * a.M + g * kWideRows + 32 * wave;
  const int64_t qrow = qbase + (lane & 31);
  const int head = (int)(qrow % a.H);

  WideDma dm = {nullptr, nullptr};
  if constexpr (RING) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_raw[raw_slots<QF8>() * raw_slot<QF8>()];
    __shared__ __attribute__((aligned(16))) int32_t s_ibuf[2 * kIdxBlock];
    dm = WideDma{(uint8_t SMD_LDS *)s_raw, (int32_t SMD_LDS *)s_ibuf};
  } else if constexpr (RINGB) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_rawb[kRingBSlots * kTileBytes];
    __shared__ __attribute__((aligned(16))) int32_t s_ibufb[2 * kIdxBlock];
    dm = WideDma{(uint8_t SMD_LDS *)s_rawb, (int32_t SMD_LDS *)s_ibufb};
  }
  WideState w;
  const WideLanes L = wide_lanes(lane);
  uint8_t SMD_LDS *stage;
  if constexpr (QF8) {
    QF8Regs<7> q;  // loaded by attend_range_wide_qf8
    attend_range_wide_qf8<P_HILO, true, 7>(a, sm, dm, a.indices + (int64_t)b * a.indices_stride, p0, p1, wave, lane,
                                        qbase, q, L, w);
    static_assert(raw_slots<true>() * raw_slot<true>() >= 4 * kStageWave, "staging slices fit the raw ring");
    stage = dm.raw + wave * kStageWave;
  } else if constexpr (RINGB) {
    bf16x8 qreg[kQRegDma];  // loaded by attend_range_wide_b
    attend_range_wide_b<PACKED, P_HILO>(a, sm, dm, a.indices + (int64_t)b * a.indices_stride, p0, p1, wave, lane,
                                        qbase, qreg, L, w);
    stage = dm.raw + wave * kStageWave;
  } else {
    bf16x8 qreg[wide_qreg<wide_ring<FP8>()>()];  // loaded by attend_range_wide
    attend_range_wide<FP8, PACKED, P_HILO>(a, sm, dm, a.indices + (int64_t)b * a.indices_stride, p0, p1, wave,
                                           lane, qbase, qreg, L, w);
    stage = wide_stage<wide_ring<FP8>()>(sm, dm, wave);
  }
  const float l_tot = half_sum(w.l_run);
  const bool lse_lane = lane < 32;
  const bool direct = a.S == 1 && a.out != nullptr;
  const OutScale sc = direct ? direct_scale(w.m_ref, l_tot, a.sink ? a.sink[head] : -INFINITY)
                             : partial_scale(w.m_ref, l_tot);
  if (direct)
    store_rows_wide<false>(w, sc.inv, false, a.out + qbase * kDim, kDim, stage);
  else if (a.hilo)  // FP32 partials, returned to the caller
    store_rows_wide<false>(w, sc.inv, true, a.part_o + (qbase * a.S + r) * kDim, (int64_t)a.S * kDim, stage);
  else  // bf16 partials in the same buffer: they only feed the merge
    store_rows_wide<false>(w, sc.inv, false, (uint16_t *)a.part_o + (qbase * a.S + r) * kDim, (int64_t)a.S * kDim,
                           stage);
  float *lse_dst = direct ? (a.lse != nullptr && lse_lane ? a.lse + qrow : nullptr)
                          : (lse_lane ? a.part_lse + qrow * a.S + r : nullptr);
  if (lse_dst != nullptr) *lse_dst = sc.lse;
}

template <bool FP8, bool PACKED, bool P_HILO, bool QF8>
static hipError_t launch_wide_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_wide_kernel<FP8, PACKED, P_HILO, QF8>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool FP8, bool PACKED, bool QF8 = false>
static hipError_t launch_wide_f(const DecodeArgs &a, hipStream_t stream) {
  return a.hilo ? launch_wide_t<FP8, PACKED, true, QF8>(a, stream) : launch_wide_t<FP8, PACKED, false, QF8>(a, stream);
}

// a.G = M / 128; one source only (a.indices2 null); a.qk_fp8 needs an fp8 pool.
hipError_t launch_decode_wide(const DecodeArgs &a, bool fp8, hipStream_t stream) {
  if (a.indices2 != nullptr || a.M % kWideRows != 0 || (a.qk_fp8 && !fp8)) return hipErrorInvalidValue;
  if (fp8) return a.qk_fp8 ? launch_wide_f<true, false, true>(a, stream) : launch_wide_f<true, false>(a, stream);
  return a.packed ? launch_wide_f<false, true>(a, stream) : launch_wide_f<false, false>(a, stream);
}

}  // namespace smd
