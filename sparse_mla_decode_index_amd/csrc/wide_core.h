// Wide waves for the persistent sparse MLA decode (gfx950): each of a
// workgroup's 4 waves owns NQ = 2 blocks of 16 query rows and all 512 dims,
// so one gathered 32-row tile serves 128 query rows and every K fragment and
// every transposed V fragment read from LDS feeds two MFMAs.  The O
// accumulators fill all 256 AGPRs; Q^T k-steps below KQ sit in VGPRs and the
// rest in LDS (each wave reads only its own region).
//
// The row gather is the long pole (a random row's latency under load), so its
// depth matters most.  Two walks over a range's tiles:
//   - bf16 pools: rows staged through one VGPR set, the rows of tile t+1 in
//     flight while tile t is computed (a second set would spill);
//   - fp8 pools: direct-to-LDS loads (global_load_lds) fill a ring of three
//     raw tiles with no VGPRs held, so tiles t+1..t+3 are in flight while t is
//     computed; each wave dequantises its own rows of the next raw tile into
//     the shared bf16 tile (e4m3 x 2^(code-127), exact in bf16).  The index
//     blocks arrive the same way, so no vector load's wait drains the ring.
// Softmax and PASS semantics are those of decode_core.h (a reference max per
// row fixed at its first valid tile, exact-max redo on overflow).
#pragma once

#include "decode_core.h"

#include <type_traits>

namespace smd {

#ifndef SMD_WIDE_KPRE
#define SMD_WIDE_KPRE 2
#endif
#ifndef SMD_WIDE_KPV
#define SMD_WIDE_KPV 8
#endif

constexpr int kWideNQ = 2;
constexpr int kQRegStaged = 6;  // Q^T k-steps in VGPRs next to a staged row set
#ifndef SMD_WIDE_QREG_DMA
#define SMD_WIDE_QREG_DMA 9
#endif
#ifndef SMD_WIDE_RAW_SLOTS
#define SMD_WIDE_RAW_SLOTS 3
#endif
constexpr int kQRegDma = SMD_WIDE_QREG_DMA;  // ... when the gather holds no VGPRs

// Raw fp8 rows of one tile as the direct-to-LDS loads leave them, per wave
// (rows 8w..8w+7 of the tile): NoPE [8][32][16 B] at 0 (chunks 28..31 of a
// row are padding), RoPE [8][8][16 B] at 4096, UE8M0 codes [8][8 B] at 5120
// (then 192 bytes of padding).
constexpr int kRawNope = 0, kRawRope = 4096, kRawCode = 5120;
constexpr int kRawWave = 5120 + 256;
constexpr int kRawSlot = 4 * kRawWave;
constexpr int kRawSlots = SMD_WIDE_RAW_SLOTS;

template <bool FP8>
struct SmemWide;

template <>
struct SmemWide<false> {
  uint8_t tile[2][kTileBytes];                      // double-buffered bf16 tiles
  int32_t ibuf[2][kIdxBlock];                       // index blocks
  uint8_t qs[4][kWideNQ][16 - kQRegStaged][64 * 16];  // [wave][block][k-step - KQ][lane]
};

// The direct-to-LDS targets (the raw ring and the index blocks) are separate
// __shared__ objects (WideDma): the compiler orders any read of a possible
// target after every load in flight (a full vmcnt wait), so those two are
// read only through inline asm with the waits issued by hand, and everything
// the MFMA path reads lives in this other object.
template <>
struct SmemWide<true> {
  uint8_t tile[1][kTileBytes];                      // the bf16 tile being computed
  uint8_t qs[4][kWideNQ][16 - kQRegDma][64 * 16];
};

struct WideDma {
  uint8_t SMD_LDS *raw;   // [kRawSlots][kRawSlot]: ring of raw fp8 tiles
  int32_t SMD_LDS *ibuf;  // [2][kIdxBlock]: index blocks
};

template <bool FP8>
constexpr int wide_qreg() {
  return FP8 ? kQRegDma : kQRegStaged;
}

template <int NQ>
struct WideState {
  f32x4 acc[NQ][32];  // acc[q][d][i] = sum_j 2^(x_j - m_ref[q]) V[j][16d + 4grp + i], block q
  float m_ref[NQ];    // reference max per block (log2 domain), same in the four 16-lane groups
  float l_run[NQ];    // this lane's share of sum_j 2^(x_j - m_ref[q])
  bool overflow;      // some score exceeded its m_ref + kRefSlackLog2 (this lane)
};

// QK, softmax weights and PV of one 32-row tile for a wide wave.  The two kv
// halves of the tile (rows 0..15, 16..31) make the 32-deep contraction of the
// PV MFMA: lane group grp supplies P of kv rows 4grp..4grp+3 and
// 16+4grp..16+4grp+3, and the two transposed V reads give the same rows.
// PASS as in compute_tile.
template <int NQ, int KQ, int PASS, bool P_HILO>
__device__ __forceinline__ void compute_tile_wide(const uint8_t SMD_LDS *tile, const bf16x8 (&qreg)[NQ][KQ],
                                                  const uint8_t SMD_LDS *qs, const int (&qk_base)[4],
                                                  const int (&pv_base)[8], uint32_t vbits, int lane, int grp,
                                                  float scale_log2, WideState<NQ> &w) {
  // ---- QK: S^T tiles of kv rows 0..15 / 16..31 for each block
  constexpr int kPre = SMD_WIDE_KPRE;  // LDS reads in flight ahead of their MFMAs
  f32x4 s[NQ][2];
#pragma unroll
  for (int q = 0; q < NQ; ++q) s[q][0] = s[q][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 k0[kPre], k1[kPre], ql[kPre][NQ];
  auto qk_load = [&](int c) {
    const uint8_t SMD_LDS *p = tile + qk_base[c & 3] + 256 * (c >> 2);
    k0[c % kPre] = *(const bf16x8 SMD_LDS *)(p);
    k1[c % kPre] = *(const bf16x8 SMD_LDS *)(p + 16 * kLdsRow);
    if (c >= KQ) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        ql[c % kPre][q] = *(const bf16x8 SMD_LDS *)(qs + ((q * (16 - KQ) + c - KQ) * 64 + lane) * 16);
    }
  };
#pragma unroll
  for (int c = 0; c < kPre; ++c) qk_load(c);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const bf16x8 a0 = k0[c % kPre], a1 = k1[c % kPre];
    bf16x8 b[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) b[q] = c < KQ ? qreg[q][c < KQ ? c : 0] : ql[c % kPre][q];
    if (c + kPre < 16) qk_load(c + kPre);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      s[q][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b[q], s[q][0], 0, 0, 0);
      s[q][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b[q], s[q][1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads kPre steps ahead of their MFMAs
  }

  // ---- softmax weights per block; this lane holds kv rows 4grp+i and 16+4grp+i
  bf16x8 pb[NQ], pl[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = ((vbits >> (4 * grp + i)) & 1) ? s[q][0][i] * scale_log2 : -INFINITY;
      x[4 + i] = ((vbits >> (16 + 4 * grp + i)) & 1) ? s[q][1][i] * scale_log2 : -INFINITY;
    }
    float tmax =
        fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    tmax = group_max(tmax);
    if constexpr (PASS == kPassMax) {
      w.m_ref[q] = fmaxf(w.m_ref[q], tmax);
      continue;
    }
    if constexpr (PASS == kPassMain) {
      if (w.m_ref[q] == -INFINITY) w.m_ref[q] = tmax;  // nothing accumulated yet for this row
      w.overflow |= tmax > w.m_ref[q] + kRefSlackLog2;
    }
    const float m_use = (w.m_ref[q] == -INFINITY) ? 0.f : w.m_ref[q];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = exp2_fast(x[i] - m_use);
      psum += p;
      pb[q][i] = (__bf16)p;
      if constexpr (P_HILO) pl[q][i] = (__bf16)(p - (float)pb[q][i]);
    }
    w.l_run[q] += psum;
  }
  if constexpr (PASS == kPassMax) return;

  // ---- PV: O^T[16d.., m] += V^T . P^T, each V^T fragment shared by the NQ blocks
  constexpr int kPv = SMD_WIDE_KPV;
  bf16x4 vlo[kPv], vhi[kPv];
  auto pv_load = [&](int d) {
    const uint8_t SMD_LDS *p = tile + pv_base[d & 7] + 256 * (d >> 3);
    vlo[d % kPv] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(p));
    vhi[d % kPv] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(p + 16 * kLdsRow));
  };
#pragma unroll
  for (int d = 0; d < kPv; ++d) pv_load(d);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const bf16x8 av = __builtin_shufflevector(vlo[d % kPv], vhi[d % kPv], 0, 1, 2, 3, 4, 5, 6, 7);
    if (d + kPv < 32) pv_load(d + kPv);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      w.acc[q][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[q], w.acc[q][d], 0, 0, 0);
      if constexpr (P_HILO) w.acc[q][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl[q], w.acc[q][d], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Walk the range's tiles once with one staged register set (bf16 pools).
// Step t: store the rows of tile t+1 (in flight since step t-1) to the free
// LDS buffer, issue the loads of tile t+2, compute tile t, one barrier.
// Indices come from the LDS index blocks as in run_split.
template <int NQ, bool PACKED, bool P_HILO, int PASS>
__device__ __forceinline__ void run_split_wide(const DecodeArgs &a, SmemWide<false> &sm, const int32_t *row_idx,
                                               int p0, int p1, int wave, int lane, int grp,
                                               const bf16x8 (&qreg)[NQ][kQRegStaged], const int (&qk_base)[4],
                                               const int (&pv_base)[8], WideState<NQ> &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  uint8_t SMD_LDS *tile0 = (uint8_t SMD_LDS *)&sm.tile[0][0];
  int32_t SMD_LDS *ib0 = (int32_t SMD_LDS *)&sm.ibuf[0][0];
  const uint8_t SMD_LDS *qs = (const uint8_t SMD_LDS *)&sm.qs[wave][0][0][0];
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  Staged<false> sa;
  const uint8_t *zrow = g_zero_row;
  const GatherLanes gl = make_gather_lanes(wave, lane);
  const int blk0 = load_idx_block(row_idx, p0, p1, 0);
  __syncthreads();  // the buffers may still be read by a previous pass
  ib0[threadIdx.x] = blk0;
  __syncthreads();
  load_rows<false, PACKED>(a, zrow, gl, tidx(0), p0, p1, wave, lane, sa);
  store_rows<false>(tile0, wave, lane, sa);
  load_rows<false, PACKED>(a, zrow, gl, tidx(1), p0 + kBK, p1, wave, lane, sa);
  __syncthreads();
  uint32_t v_cur = tile_valid_bits(tidx(0), p0, p1, lane, a.num_rows32);
  for (int t = 0; t < ntiles; ++t) {
    const int nb = t / kTilesPerIdxBlock + 1;  // the next index block
    const int blk = load_idx_block(row_idx, p0, p1, nb);
    store_rows<false>(tile0 + ((t + 1) & 1) * kTileBytes, wave, lane, sa);
    load_rows<false, PACKED>(a, zrow, gl, tidx(t + 2), p0 + (t + 2) * kBK, p1, wave, lane, sa);
    compute_tile_wide<NQ, kQRegStaged, PASS, P_HILO>(tile0 + (t & 1) * kTileBytes, qreg, qs, qk_base, pv_base,
                                                     v_cur, lane, grp, a.scale_log2, w);
    if (t % kTilesPerIdxBlock == kTilesPerIdxBlock - 3) ib0[(nb & 1) * kIdxBlock + threadIdx.x] = blk;
    __syncthreads();
    v_cur = tile_valid_bits(tidx(t + 1), p0 + (t + 1) * kBK, p1, lane, a.num_rows32);
  }
}

// One direct-to-LDS load: lane i's SIZE bytes at src land at dst + SIZE * i
// (dst wave-uniform, passed in M0).  Issued through inline asm so that the
// compiler does not order every later LDS read after it (it cannot tell which
// LDS bytes such a load writes); the walk below waits for these loads itself.
template <int SIZE>
__device__ __forceinline__ void lds_dma(const void *src, uint8_t SMD_LDS *dst) {
  const uint64_t va = (uint64_t)(uintptr_t)src;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  static_assert(SIZE == 16 || SIZE == 4, "load size");
  if constexpr (SIZE == 16)
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(va), "{m0}"(m0) : "memory");
  else
    asm volatile("global_load_lds_dword %0, off" ::"v"(va), "{m0}"(m0) : "memory");
}

// Direct-to-LDS loads of this wave's 8 rows of a tile (indices at tidx) into
// its raw region `dst` (layout above): loads 0..3 bring the NoPE of rows
// 2k + (lane >> 5), load 4 the RoPE of row lane >> 3, load 5 the codes, 4
// bytes per lane (lanes 0..15: row lane / 2, half lane % 2).  Invalid rows and positions past p1 read the
// zero row, as in load_rows.
// The 8 indices at p (the same for every lane), read behind the compiler's back.
__device__ __forceinline__ void lds_read_idx8(const int32_t SMD_LDS *p, uint32_t (&w)[8]) {
  u32x4 lo, hi;
  const uint32_t addr = (uint32_t)(uintptr_t)p;
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi)
      : "v"(addr)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = __builtin_amdgcn_readfirstlane(lo[i]);
    w[4 + i] = __builtin_amdgcn_readfirstlane(hi[i]);
  }
}

// One index per lane (lane i reads p[i & 31]), read behind the compiler's back.
__device__ __forceinline__ int32_t lds_read_idx_lane(const int32_t SMD_LDS *p, int lane) {
  int32_t v;
  const uint32_t addr = (uint32_t)(uintptr_t)(p + (lane & (kBK - 1)));
  asm volatile(
      "ds_read_b32 %0, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v)
      : "v"(addr)
      : "memory");
  return v;
}

// Select w[r] for a lane-dependent r in 0..7.
__device__ __forceinline__ uint32_t pick8(const uint32_t (&w)[8], int r) {
  const uint32_t a = (r & 1) ? w[1] : w[0], b = (r & 1) ? w[3] : w[2];
  const uint32_t c = (r & 1) ? w[5] : w[4], d = (r & 1) ? w[7] : w[6];
  const uint32_t e = (r & 2) ? b : a, f = (r & 2) ? d : c;
  return (r & 4) ? f : e;
}

__device__ __forceinline__ void dma_rows_fp8(const DecodeArgs &a, const int32_t SMD_LDS *tidx, int first_pos, int p1,
                                             int wave, int lane, uint8_t SMD_LDS *dst) {
  uint32_t widx[8];
  lds_read_idx8(tidx + wave * (kBK / 4), widx);
  const int rows_left = p1 - first_pos - wave * (kBK / 4);
  const uint8_t *z = g_zero_row;
  // Padding lanes re-read a chunk of their own row (lanes 28..31 of a half
  // read chunk 27, code lanes 16..63 repeat lanes 0..15): the zero row is one
  // cache line that every wave would hit at once.
  const int c = min(lane & 31, 27);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 2 * k + (lane >> 5);
    const uint32_t idx = (lane >> 5) ? widx[2 * k + 1] : widx[2 * k];
    const bool v = r < rows_left && idx < a.num_rows32;
    const uint8_t *src = v ? a.kv_nope + (uint64_t)idx * (uint64_t)a.nope_stride_b + 16 * c : z + 16 * c;
    lds_dma<16>(src, dst + kRawNope + 1024 * k);
  }
  {
    const int r = lane >> 3;
    const uint32_t idx = pick8(widx, r);
    const bool v = r < rows_left && idx < a.num_rows32;
    const uint8_t *src = (v ? a.kv_rope + (uint64_t)idx * (uint64_t)a.rope_stride_b : z) + 16 * (lane & 7);
    lds_dma<16>(src, dst + kRawRope);
  }
  const int r = (lane >> 1) & 7;
  const uint32_t idx = pick8(widx, r);
  const bool v = r < rows_left && idx < a.num_rows32;
  const uint8_t *src = (v ? a.kv_scale + (uint64_t)idx * (uint64_t)a.scale_stride_b : z) + 4 * (lane & 1);
  lds_dma<4>(src, dst + kRawCode);
}

// Index block k straight into LDS: wave w's lanes load positions
// p0 + 256k + 64w + lane (clamped into [p0, p1), as load_idx_block).
__device__ __forceinline__ void dma_idx_block(const int32_t *row_idx, int p0, int p1, int k, int wave, int lane,
                                              int32_t SMD_LDS *dst) {
  const int pos = min(p0 + k * kIdxBlock + 64 * wave + lane, p1 - 1);
  lds_dma<4>(row_idx + pos, (uint8_t SMD_LDS *)(dst + 64 * wave));
}

// This wave's raw rows (its own region, landed) in the register layout of
// Staged<true>, ready for store_rows<true>; read behind the compiler's back.
__device__ __forceinline__ void raw_to_staged(const uint8_t SMD_LDS *src, Staged<true> &st) {
  // The lane id comes from an opaque asm so that the lane offsets below are
  // recomputed in the loop rather than hoisted: hoisted, they get spilled,
  // and the wait for their reload would land in the loop and drain the ring.
  int lane;
  asm volatile(
      "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
      "v_mbcnt_hi_u32_b32 %0, -1, %0"
      : "=v"(lane));
  const int c = min(lane & 31, 27);
  const uint32_t a1 = (uint32_t)(uintptr_t)(src + kRawNope + ((lane >> 5) * 32 + c) * 16);
  const uint32_t a2 = (uint32_t)(uintptr_t)(src + kRawCode + (lane >> 5) * 8 + (c >> 2));
  const uint32_t a3 = (uint32_t)(uintptr_t)(src + kRawRope + lane * 16);
  // row 2j + (lane >> 5): NoPE at a1 + 1024 j, code at a2 + 16 j
  static_assert(kRawCode <= 65535 - 48 && kRawNope + 3072 <= 65535, "ds offsets");
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %9 offset:1024\n\t"
      "ds_read_b128 %2, %9 offset:2048\n\t"
      "ds_read_b128 %3, %9 offset:3072\n\t"
      "ds_read_u8 %4, %10\n\t"
      "ds_read_u8 %5, %10 offset:16\n\t"
      "ds_read_u8 %6, %10 offset:32\n\t"
      "ds_read_u8 %7, %10 offset:48\n\t"
      "ds_read_b128 %8, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(st.v[0]), "=&v"(st.v[1]), "=&v"(st.v[2]), "=&v"(st.v[3]), "=&v"(st.code[0]), "=&v"(st.code[1]),
        "=&v"(st.code[2]), "=&v"(st.code[3]), "=&v"(st.rope)
      : "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// Valid-row bits of a tile whose indices sit in a direct-to-LDS target.
__device__ __forceinline__ uint32_t tile_valid_bits_dma(const int32_t SMD_LDS *tidx, int first_pos, int p1, int lane,
                                                        uint32_t num_rows) {
  const int idx_v = lds_read_idx_lane(tidx, lane);
  return (uint32_t)__ballot(lane < kBK && first_pos + lane < p1 && (uint32_t)idx_v < num_rows);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every vector-memory operation in flight (the direct-to-LDS loads count as
// stores to be released), which would drain the ring at every barrier.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Q^T of block q of a wide wave (query row qrow[q]) as QK B operands: k-steps
// below KQ into VGPRs, the rest into the wave's LDS region (only this wave
// reads it, after its own stores).
template <int NQ, int KQ>
__device__ __forceinline__ void load_q_wide(const DecodeArgs &a, const int64_t (&qrow)[NQ], int lane, int grp,
                                            uint8_t SMD_LDS *qs, bf16x8 (&qreg)[NQ][KQ]) {
  // Every load is issued before the first LDS store: interleaved, each store
  // would wait for its own load and the k-steps would arrive one latency at
  // a time.
  bf16x8 tmp[NQ][16 - KQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint16_t *src = (c < 14) ? a.q_nope + qrow[q] * kNope + 32 * c + 8 * grp
                                     : a.q_rope + qrow[q] * kRope + 32 * (c - 14) + 8 * grp;
      const bf16x8 v = *(const bf16x8 *)src;
      if (c < KQ)
        qreg[q][c < KQ ? c : 0] = v;
      else
        tmp[q][c < KQ ? 0 : c - KQ] = v;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int c = KQ; c < 16; ++c)
      *(bf16x8 SMD_LDS *)(qs + ((q * (16 - KQ) + c - KQ) * 64 + lane) * 16) = tmp[q][c - KQ];
  }
}

// Walk the range's tiles once (fp8 pools) with the raw ring.  Tile k's loads
// go to slot k % 3 at step k - 3.  Step t:
//   wait for this wave's loads of tile t (12 younger loads are allowed: the
//   six of each of tiles t+1 and t+2; an index block load among them only
//   makes the wait longer), read its raw rows into registers;
//   barrier A (everyone is done with the bf16 tile of t-1 and has read its
//   raw rows of t: slot t % 3 is free);
//   issue the loads of tile t+3 into slot t % 3 (and, at t % 8 == 0, index
//   block t/8 + 1);
//   dequantise into the bf16 tile, barrier B, compute.
// Index block k is read from step 8k - 3 on; issued at step 8(k-1), it has
// landed by the wait of step 8k - 4 (four tiles' loads later) and barrier A
// of that step publishes it.  The block it replaces was last read at step
// 8(k-1) - 1.
template <int NQ, bool P_HILO, int PASS>
__device__ __forceinline__ void run_split_wide_dma(const DecodeArgs &a, SmemWide<true> &sm, const WideDma &dm,
                                                   const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                   int grp, const bf16x8 (&qreg)[NQ][kQRegDma],
                                                   const int (&qk_base)[4], const int (&pv_base)[8],
                                                   WideState<NQ> &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  uint8_t SMD_LDS *tile = (uint8_t SMD_LDS *)&sm.tile[0][0];
  uint8_t SMD_LDS *raw = dm.raw;
  int32_t SMD_LDS *ib0 = dm.ibuf;
  const uint8_t SMD_LDS *qs = (const uint8_t SMD_LDS *)&sm.qs[wave][0][0][0];
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  auto slot = [&](int k) { return raw + (k % kRawSlots) * kRawSlot + wave * kRawWave; };
  // A real vmcnt(0) (not inline asm) so that the compiler's wait bookkeeping
  // starts the walk with nothing in flight: the loads it cannot see are
  // counted by the hardware too, and a wait it would otherwise keep for an
  // earlier load (of Q^T, say) would drain the ring at every step.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
  if constexpr (PASS != kPassMain) {  // the main pass's caller has done this, with the Q^T load
    __syncthreads();  // the buffers may still be read by a previous pass
    dma_idx_block(row_idx, p0, p1, 0, wave, lane, ib0);
    wait_vm<0>();
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kRawSlots; ++k) dma_rows_fp8(a, tidx(k), p0 + k * kBK, p1, wave, lane, slot(k));
  for (int t = 0; t < ntiles; ++t) {
    wait_vm<6 * (kRawSlots - 1)>();
    Staged<true> st;
    raw_to_staged(slot(t), st);
    const uint32_t v_cur = tile_valid_bits_dma(tidx(t), p0 + t * kBK, p1, lane, a.num_rows32);
    barrier_lds();  // A (this wave's raw reads of slot t % 3 are done too)
    dma_rows_fp8(a, tidx(t + kRawSlots), p0 + (t + kRawSlots) * kBK, p1, wave, lane, slot(t));
    if (t % kTilesPerIdxBlock == 0) {
      const int nb = t / kTilesPerIdxBlock + 1;
      dma_idx_block(row_idx, p0, p1, nb, wave, lane, ib0 + (nb & 1) * kIdxBlock);
    }
    store_rows<true>(tile, wave, lane, st);
    barrier_lds();  // B
    compute_tile_wide<NQ, kQRegDma, PASS, P_HILO>(tile, qreg, qs, qk_base, pv_base, v_cur, lane, grp,
                                                  a.scale_log2, w);
  }
  wait_vm<0>();  // no load may land in LDS after the walk
}

// Attend the wide wave's query rows over positions [p0, p1) of row_idx: the
// main pass, and the exact-max two-pass redo when some score overflowed its
// reference max anywhere in the workgroup.
template <int NQ, bool FP8, bool PACKED, bool P_HILO>
__device__ __forceinline__ void attend_range_wide(const DecodeArgs &a, SmemWide<FP8> &sm, const WideDma &dm,
                                                  const int32_t *row_idx,
                                                  int p0, int p1, int wave, int lane, int grp,
                                                  const int64_t (&qrow)[NQ], bf16x8 (&qreg)[NQ][wide_qreg<FP8>()],
                                                  const int (&qk_base)[4], const int (&pv_base)[8],
                                                  WideState<NQ> &w) {
  auto reset = [&]() {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int d = 0; d < 32; ++d) w.acc[q][d] = f32x4{0.f, 0.f, 0.f, 0.f};
      w.m_ref[q] = -INFINITY;
      w.l_run[q] = 0.f;
    }
  };
  auto walk = [&](auto pass) {
    constexpr int PASS = decltype(pass)::value;
    if constexpr (FP8)
      run_split_wide_dma<NQ, P_HILO, PASS>(a, sm, dm, row_idx, p0, p1, wave, lane, grp, qreg, qk_base, pv_base,
                                           w);
    else
      run_split_wide<NQ, PACKED, P_HILO, PASS>(a, sm, row_idx, p0, p1, wave, lane, grp, qreg, qk_base, pv_base,
                                               w);
  };
  if constexpr (FP8) {
    // The first index block of the main pass goes out ahead of the Q^T
    // loads: the two round trips overlap instead of following each other.
    __syncthreads();  // the buffers may still be read by a previous piece
    if (p1 > p0) dma_idx_block(row_idx, p0, p1, 0, wave, lane, dm.ibuf);
  }
  load_q_wide<NQ, wide_qreg<FP8>()>(a, qrow, lane, grp, (uint8_t SMD_LDS *)&sm.qs[wave][0][0][0], qreg);
  reset();
  w.overflow = false;
  walk(std::integral_constant<int, kPassMain>{});
  if (__syncthreads_or(w.overflow)) {
    reset();
    walk(std::integral_constant<int, kPassMax>{});
    walk(std::integral_constant<int, kPassFixed>{});
  }
}

// Outputs of block q of a wide wave: bf16 with the sink folded in, or the
// FP32 partial; dst points at dim 4*grp of the row.
template <int NQ>
__device__ __forceinline__ void write_direct_wide(const WideState<NQ> &w, int q, float l_tot, float sink_ln,
                                                  uint16_t *dst, float *lse_dst) {
  const float sink2 = sink_ln * kLog2e;
  const float mf = fmaxf(w.m_ref[q], sink2);
  float inv = 0.f, lse_v = -INFINITY;
  if (mf != -INFINITY) {
    const float e = exp2_fast(w.m_ref[q] - mf);
    const float z = l_tot * e + exp2_fast(sink2 - mf);
    inv = e / z;
    lse_v = (mf + __log2f(z)) * kLn2;
  }
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    u32x2 v;
    v[0] = (uint32_t)f32_to_bf16_rne(w.acc[q][d][0] * inv) | ((uint32_t)f32_to_bf16_rne(w.acc[q][d][1] * inv) << 16);
    v[1] = (uint32_t)f32_to_bf16_rne(w.acc[q][d][2] * inv) | ((uint32_t)f32_to_bf16_rne(w.acc[q][d][3] * inv) << 16);
    *(u32x2 *)(dst + 16 * d) = v;
  }
  if (lse_dst != nullptr) *lse_dst = lse_v;
}

template <int NQ>
__device__ __forceinline__ void write_partial_wide(const WideState<NQ> &w, int q, float l_tot, float *dst,
                                                   float *lse_dst) {
  float inv = 0.f, lse_v = -INFINITY;
  if (l_tot > 0.f) {
    inv = 1.f / l_tot;
    lse_v = (w.m_ref[q] + __log2f(l_tot)) * kLn2;
  }
#pragma unroll
  for (int d = 0; d < 32; ++d) *(f32x4 *)(dst + 16 * d) = w.acc[q][d] * inv;
  if (lse_dst != nullptr) *lse_dst = lse_v;
}

}  // namespace smd
