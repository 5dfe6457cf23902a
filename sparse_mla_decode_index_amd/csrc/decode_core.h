// Row-block device core of the persistent sparse MLA decode for gfx950
// (MI355X).
//
// What is computed (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
// decode on gfx950", Design): per query row, a 512-wide dot product (448 NoPE
// + 64 RoPE dims) with every selected latent row, an online softmax that also
// counts a per-head sink logit, and a PV product over the same 512-wide rows.
// Split partials and their merge follow the aiter page "[ASM][HIP][MLA v4 nm]
// Split plan helper and persistent decode kernel", Summary part 1.
//
// A workgroup of 4 waves attends one group of 16*RB query rows (heads x MTP
// positions sharing one index list) over a range [p0, p1) of index positions.
// Wave w owns the 16 query rows of block w % RB and the 512/DS dims of slice
// w / RB (RB * DS = 4).
//
// Per 32-row KV tile:
//   gather   each wave loads 8 of the tile's rows into VGPRs (16 bytes per
//            lane per load; fp8 rows are dequantised in registers,
//            e4m3 x 2^(code-127) -> bf16, exact) and stores them to an LDS
//            tile.  Two tiles are in flight while a third is computed.  Rows
//            of invalid indices (outside [0, N)) and positions past p1 load a
//            zero row, so every tile issues the same loads and stale LDS
//            contents never reach the MFMAs.
//   QK       S^T[32 kv x 16 q] = K[32 x 512] . Q^T[512 x 16] with
//            v_mfma_f32_16x16x32_bf16; K from LDS, Q resident in VGPRs.  In
//            this orientation each lane holds scores of one query row, so the
//            softmax statistics are per-lane values.  With DS > 1 the waves
//            that share query rows add their partial scores through LDS.
//   softmax  a reference max per query row fixed at its first valid tile
//            (exp2 domain, scale pre-multiplied by log2(e)); a score more than
//            2^32 above it sends the workgroup through an exact-max second
//            pass, so the accumulators are never rescaled.
//   PV       O^T[512 x 16] += V^T[512 x 32] . P^T[32 x 16]; P^T is the score
//            tile converted to bf16 in registers, V^T comes from LDS with
//            ds_read_b64_tr_b16 transposed reads.
// The LDS tile is row-major, 1 KiB per row, with the 16-byte chunks of row r
// permuted by an XOR of swz(r) so that both the 16-byte QK reads (16 rows, one
// column) and the 8-byte transposed reads (8 rows, 32 bytes each) touch
// distinct banks.
#pragma once

#include "common.h"

namespace smd {

constexpr int kBK = 32;                      // KV rows per tile
constexpr int kLdsRow = 1024;                // bytes per bf16 row in LDS
constexpr int kTileBytes = kBK * kLdsRow;    // 32 KiB

// Index lists are staged through LDS in blocks of kIdxBlock positions (8 tiles),
// double-buffered and refilled kIdxBlock/32 - 3 tiles before first use, so no
// per-tile global read sits on the critical path of the row gather.
constexpr int kIdxBlock = 256;
constexpr int kTilesPerIdxBlock = kIdxBlock / kBK;  // 8

template <int DS>
struct Smem {
  uint8_t tile[2][kTileBytes];          // double-buffered bf16 tiles
  float sx[DS > 1 ? 4 * 64 * 8 : 4];    // partial S^T tiles of the dim-split waves
  int32_t ibuf[2][kIdxBlock];           // index blocks (tiles 8k .. 8k+7 in ibuf[k & 1])
};

// Index block k (positions p0 + 256k + tid, tid < 256), clamped into [p0, p1)
// (p1 > p0) so that the load is unconditional: every step issues the same
// memory operations and the compiler's wait counts stay exact.  Positions at
// or beyond p1 are masked where the indices are used.
__device__ __forceinline__ int load_idx_block(const int32_t *row_idx, int p0, int p1, int k) {
  return row_idx[min(p0 + k * kIdxBlock + (int)threadIdx.x, p1 - 1)];
}

// Row data of one tile held in registers between its global loads and its
// LDS stores.  Wave w handles tile rows 8w .. 8w+7.
//   bf16: v[i] = logical 16-byte chunk lane ^ tile_swz(rr) of row rr = 8w + i.
//   fp8:  v[j] (j < 4) = 16 e4m3 bytes of chunk (lane & 31) (clamped to 27) of
//         row 8w + 2j + (lane >> 5) and code[j] = the UE8M0 code of that
//         chunk's 64-dim block; rope = 16 RoPE bytes, chunk lane & 7 of row
//         8w + (lane >> 3).
template <bool FP8>
struct Staged {
  u32x4 v[FP8 ? 4 : kBK / 4];
  u32x4 rope;
  uint32_t code[FP8 ? 4 : 1];
};

// Per-wave constants of the gather, computed once.
struct GatherLanes {
  uint32_t voff[kBK / 4];  // bf16: byte offset of this lane's chunk in row 8w+i
  uint32_t sel_rope;       // bf16, split layout: bit i set when that chunk is RoPE
};

// Chunk permutation of tile row r: swz (16x16 MFMA operands) or swz32 (32x32).
enum TileLayout { kLay16 = 0, kLay32 = 1 };
template <int LAY>
__device__ __forceinline__ int tile_swz(int r) {
  return LAY == kLay32 ? swz32(r) : swz(r);
}

template <int LAY = kLay16>
__device__ __forceinline__ GatherLanes make_gather_lanes(int wave, int lane) {
  GatherLanes g;
  g.sel_rope = 0;
#pragma unroll
  for (int i = 0; i < kBK / 4; ++i) {
    const int c = lane ^ tile_swz<LAY>(wave * (kBK / 4) + i);
    g.voff[i] = (uint32_t)c * 16u;
    g.sel_rope |= (c >= kNope / 8 ? 1u : 0u) << i;
  }
  return g;
}

// Global loads of this wave's 8 rows of a tile (indices at tidx in LDS).
// Invalid rows (index outside [0, N), or past the split) read the zero row, so
// stale LDS contents (even NaN) never reach the MFMAs and every tile issues
// the same loads.  bf16 rows whose RoPE part follows the NoPE part (the packed
// [N, 512] layout) need one scalar row base per row; other layouts select the
// NoPE or RoPE base per lane.
template <bool FP8, bool PACKED>
__device__ __forceinline__ void load_rows(const DecodeArgs &a, const uint8_t *zrow, const GatherLanes &gl,
                                          const int32_t SMD_LDS *tidx, int first_pos, int p1, int wave,
                                          int lane, Staged<FP8> &st) {
  const int32_t SMD_LDS *widx = tidx + wave * (kBK / 4);  // this wave's 8 indices
  const int rows_left = p1 - first_pos - wave * (kBK / 4);  // rows of this wave below p1
  if constexpr (!FP8) {
    const u32x4 ia = *(const u32x4 SMD_LDS *)(widx);
    const u32x4 ib = *(const u32x4 SMD_LDS *)(widx + 4);
    // byte offsets from the NoPE base; the zero row as an offset from it
    const uint64_t zoff = (uint64_t)(zrow - a.kv_nope);
#pragma unroll
    for (int i = 0; i < kBK / 4; ++i) {
      const uint32_t idx = __builtin_amdgcn_readfirstlane(i < 4 ? ia[i & 3] : ib[i & 3]);
      const bool v = (i < rows_left) & (idx < a.num_rows32);  // idx < 0 wraps to a huge value
      if constexpr (PACKED) {
        const uint64_t off = v ? (uint64_t)idx * a.row_stride32 : zoff;
        st.v[i] = *(const u32x4 *)(a.kv_nope + off + gl.voff[i]);
      } else {
        const uint64_t zr = (uint64_t)(zrow - a.kv_rope) + kNope * 2;
        const uint64_t noff = v ? (uint64_t)idx * (uint64_t)a.nope_stride_b : zoff;
        const uint64_t roff = v ? (uint64_t)idx * (uint64_t)a.rope_stride_b : zr;
        const uint8_t *nb = a.kv_nope + noff;
        const uint8_t *rb = a.kv_rope + roff - kNope * 2;
        st.v[i] = *(const u32x4 *)((((gl.sel_rope >> i) & 1) ? rb : nb) + gl.voff[i]);
      }
    }
  } else {
    const u32x4 ia = *(const u32x4 SMD_LDS *)(widx);
    const u32x4 ib = *(const u32x4 SMD_LDS *)(widx + 4);
    const int c = min(lane & 31, 27);
    const uint64_t zoff = (uint64_t)(zrow - a.kv_nope);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ia_ = __builtin_amdgcn_readfirstlane(j < 2 ? ia[(2 * j) & 3] : ib[(2 * j) & 3]);
      const uint32_t ib_ = __builtin_amdgcn_readfirstlane(j < 2 ? ia[(2 * j + 1) & 3] : ib[(2 * j + 1) & 3]);
      const bool va = (2 * j < rows_left) & (ia_ < a.num_rows32);
      const bool vb = (2 * j + 1 < rows_left) & (ib_ < a.num_rows32);
      const uint64_t oa = va ? (uint64_t)ia_ * (uint64_t)a.nope_stride_b : zoff;
      const uint64_t ob = vb ? (uint64_t)ib_ * (uint64_t)a.nope_stride_b : zoff;
      st.v[j] = *(const u32x4 *)(a.kv_nope + (lane < 32 ? oa : ob) + c * 16);
      const uint8_t *sa = va ? a.kv_scale + (uint64_t)ia_ * (uint64_t)a.scale_stride_b : zrow;
      const uint8_t *sb = vb ? a.kv_scale + (uint64_t)ib_ * (uint64_t)a.scale_stride_b : zrow;
      st.code[j] = (lane < 32 ? sa : sb)[c >> 2];
    }
    // RoPE and codes of the 8 rows: lane l serves row l >> 3
    const uint32_t il = (uint32_t)widx[lane >> 3];
    const bool vl = ((lane >> 3) < rows_left) & (il < a.num_rows32);
    const uint8_t *rp = vl ? a.kv_rope + (uint64_t)il * (uint64_t)a.rope_stride_b : zrow;
    st.rope = *(const u32x4 *)(rp + (lane & 7) * 16);
  }
}

// LDS stores of the staged rows into `tile` (bf16 layout, chunks swizzled);
// fp8 rows are dequantised on the way: e4m3 x 2^(code-127) is exact in bf16.
// The stores come in kStorePieces<FP8> independent pieces (bf16: one row
// each; fp8: one row pair each, then the RoPE dims of the 8 rows), so that a
// caller can spread them between other work.
template <bool FP8>
constexpr int kStorePieces = FP8 ? 5 : kBK / 4;

template <bool FP8, int LAY = kLay16>
__device__ __forceinline__ void store_row_piece(uint8_t SMD_LDS *tile, int wave, int lane, const Staged<FP8> &st,
                                                int i) {
  if constexpr (!FP8) {
    *(u32x4 SMD_LDS *)(tile + (wave * (kBK / 4) + i) * kLdsRow + lane * 16) = st.v[i];
  } else if (i < 4) {
    const int c = lane & 31;
    const int rl = 2 * i + (lane >> 5);  // row within the wave's 8
    const uint32_t code = st.code[i];
    if (c < 28) {
      const int rr = wave * (kBK / 4) + rl;
      const int f = tile_swz<LAY>(rr);
      uint8_t SMD_LDS *row = tile + rr * kLdsRow;
      const float sc = ue8m0_scale(code);
      u32x4 lo, hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t u0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)st.v[i][q], sc, false));
        const uint32_t u1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)st.v[i][q], sc, true));
        if (q < 2) { lo[2 * q] = u0; lo[2 * q + 1] = u1; }
        else { hi[2 * q - 4] = u0; hi[2 * q - 3] = u1; }
      }
      *(u32x4 SMD_LDS *)(row + (((2 * c) ^ f) << 4)) = lo;
      *(u32x4 SMD_LDS *)(row + (((2 * c + 1) ^ f) << 4)) = hi;
    }
  } else {
    const int rr = wave * (kBK / 4) + (lane >> 3);
    *(u32x4 SMD_LDS *)(tile + rr * kLdsRow + (((kNope / 8 + (lane & 7)) ^ tile_swz<LAY>(rr)) << 4)) = st.rope;
  }
}

template <bool FP8, int LAY = kLay16>
__device__ __forceinline__ void store_rows(uint8_t SMD_LDS *tile, int wave, int lane, const Staged<FP8> &st) {
#pragma unroll
  for (int i = 0; i < kStorePieces<FP8>; ++i) store_row_piece<FP8, LAY>(tile, wave, lane, st, i);
}

// Valid-row bits of a tile (first position first_pos, indices at tidx).
__device__ __forceinline__ uint32_t tile_valid_bits(const int32_t SMD_LDS *tidx, int first_pos, int p1, int lane,
                                                    uint32_t num_rows) {
  const int idx_v = tidx[lane & (kBK - 1)];
  return (uint32_t)__ballot(lane < kBK && first_pos + lane < p1 && (uint32_t)idx_v < (uint32_t)num_rows);
}

// Per-wave state of the softmax and the O^T accumulator (ND 16-dim blocks).
template <int ND>
struct WaveState {
  f32x4 acc[ND];  // acc[d][i] = sum_j 2^(x_j - m_ref) V[j][16(d0+d) + 4grp + i]
  float m_ref;    // reference max (log2 domain), same in the four 16-lane groups
  float l_run;    // this lane's share of sum_j 2^(x_j - m_ref)
  bool overflow;  // some score exceeded m_ref + kRefSlackLog2 (this lane)
};

// QK, softmax weights and PV over one 32-row tile for one wave: 16 query rows
// and the 512/DS dims starting at chunk c0 (QK, 32-dim chunks) / block d0
// (PV, 16-dim blocks).  With DS > 1 the partial scores of the DS waves that
// share the query rows are summed through LDS (fixed order, so the DS waves
// hold bit-identical scores and take identical softmax decisions).
//   kPassMain:  m_ref is set at the row's first valid tile; later tiles only
//               flag scores above m_ref + kRefSlackLog2.
//   kPassMax:   scores only; m_ref becomes the exact running max.
//   kPassFixed: m_ref is already the exact max.
// The O accumulator is only ever touched by MFMAs here, never rescaled.
template <int RB, int DS, int PASS, bool P_HILO>
__device__ __forceinline__ void compute_tile(const uint8_t SMD_LDS *tile, float SMD_LDS *sx,
                                             const bf16x8 (&qreg)[16 / DS], const int (&qk_base)[4],
                                             const int (&pv_base)[8], uint32_t vbits, int wave,
                                             int lane, int grp, int ds, float scale_log2,
                                             WaveState<32 / DS> &w) {
  constexpr int NC = 16 / DS, ND = 32 / DS;
  const int c0 = ds * NC, d0 = ds * ND;
  // ---- QK: S^T tiles for kv rows 0..15 (s0) and 16..31 (s1) over this wave's dims
  constexpr int kPre = NC < 4 ? NC : 4;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 k0[kPre], k1[kPre];
  auto qk_load = [&](int c) {
    const int cg = c0 + c;
    const uint8_t SMD_LDS *p = tile + qk_base[cg & 3] + 256 * (cg >> 2);
    k0[c % kPre] = *(const bf16x8 SMD_LDS *)(p);
    k1[c % kPre] = *(const bf16x8 SMD_LDS *)(p + 16 * kLdsRow);
  };
#pragma unroll
  for (int c = 0; c < kPre; ++c) qk_load(c);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const bf16x8 a0 = k0[c % kPre], a1 = k1[c % kPre];
    if (c + kPre < NC) qk_load(c + kPre);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[c], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[c], s1, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads kPre steps ahead
  }
  if constexpr (DS > 1) {
    f32x4 SMD_LDS *mine = (f32x4 SMD_LDS *)(sx + (wave * 64 + lane) * 8);
    mine[0] = s0;
    mine[1] = s1;
    __syncthreads();
    const int rb = wave % RB;
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const f32x4 SMD_LDS *o = (const f32x4 SMD_LDS *)(sx + ((rb + e * RB) * 64 + lane) * 8);
      s0 += o[0];
      s1 += o[1];
    }
  }

  // ---- scores; this lane holds kv rows 4grp+i (s0) and 16+4grp+i (s1)
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = ((vbits >> (4 * grp + i)) & 1) ? s0[i] * scale_log2 : -INFINITY;
    x[4 + i] = ((vbits >> (16 + 4 * grp + i)) & 1) ? s1[i] * scale_log2 : -INFINITY;
  }
  float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  tmax = group_max(tmax);
  if constexpr (PASS == kPassMax) {
    w.m_ref = fmaxf(w.m_ref, tmax);
    return;
  }
  if constexpr (PASS == kPassMain) {
    if (w.m_ref == -INFINITY) w.m_ref = tmax;  // nothing accumulated yet for this row
    w.overflow |= tmax > w.m_ref + kRefSlackLog2;
  }
  const float m_use = (w.m_ref == -INFINITY) ? 0.f : w.m_ref;
  float psum = 0.f;
  bf16x8 pb, pl;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = exp2_fast(x[i] - m_use);
    psum += p;
    pb[i] = (__bf16)p;
    // P_HILO: p = hi + lo with both parts bf16, so the PV product carries
    // about 16 significant bits of p instead of 8 (needed for FP32 partials).
    if constexpr (P_HILO) pl[i] = (__bf16)(p - (float)pb[i]);
  }
  w.l_run += psum;

  // ---- PV: O^T[16d.., m] += V^T . P^T for this wave's dims, V^T read transposed
  constexpr int kPv = ND < 4 ? ND : 4;
  bf16x4 vlo[kPv], vhi[kPv];
  auto pv_load = [&](int d) {
    const int dg = d0 + d;
    const uint8_t SMD_LDS *p = tile + pv_base[dg & 7] + 256 * (dg >> 3);
    vlo[d % kPv] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(p));
    vhi[d % kPv] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(p + 16 * kLdsRow));
  };
#pragma unroll
  for (int d = 0; d < kPv; ++d) pv_load(d);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const bf16x8 av = __builtin_shufflevector(vlo[d % kPv], vhi[d % kPv], 0, 1, 2, 3, 4, 5, 6, 7);
    if (d + kPv < ND) pv_load(d + kPv);
    w.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, w.acc[d], 0, 0, 0);
    if constexpr (P_HILO) w.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl, w.acc[d], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Walk the split's tiles once.  While tile t is computed from LDS, the rows
// of tiles t+1 and t+2 are in flight into registers; the rows of t+1 are
// stored to the other LDS buffer after the math, and one barrier per tile
// publishes them.  Indices come from the LDS index blocks; the block after
// the current one is re-read every step (cache hits after the first) and
// stored three tiles before it is first needed.  Every step issues the same
// loads (rows past the end read the zero row), so the compiler's vmcnt waits
// let two tiles stay in flight.
template <int RB, int DS, bool FP8, bool PACKED, bool P_HILO, int PASS>
__device__ __forceinline__ void run_split(const DecodeArgs &a, Smem<DS> &sm, const int32_t *row_idx, int p0,
                                          int p1, int wave, int lane, int grp, int ds,
                                          const bf16x8 (&qreg)[16 / DS], const int (&qk_base)[4],
                                          const int (&pv_base)[8], WaveState<32 / DS> &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  uint8_t SMD_LDS *tile0 = (uint8_t SMD_LDS *)&sm.tile[0][0];
  float SMD_LDS *sx = (float SMD_LDS *)&sm.sx[0];
  int32_t SMD_LDS *ib0 = (int32_t SMD_LDS *)&sm.ibuf[0][0];
  // LDS address of the 32 indices of tile k
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  Staged<FP8> sa, sb;
  const uint8_t *zrow = g_zero_row;
  const GatherLanes gl = make_gather_lanes(wave, lane);
  const int blk0 = load_idx_block(row_idx, p0, p1, 0);
  __syncthreads();  // the buffers may still be read by a previous pass
  ib0[threadIdx.x] = blk0;
  __syncthreads();
  load_rows<FP8, PACKED>(a, zrow, gl, tidx(0), p0, p1, wave, lane, sa);
  load_rows<FP8, PACKED>(a, zrow, gl, tidx(1), p0 + kBK, p1, wave, lane, sb);
  store_rows<FP8>(tile0, wave, lane, sa);
  __syncthreads();
  uint32_t v_cur = tile_valid_bits(tidx(0), p0, p1, lane, a.num_rows32);
  // step t: tile t in buffer t&1; `nx` holds (in flight) the rows of t+1; the
  // other staging set is refilled with the rows of t+2.  The loop runs two
  // steps per iteration so each staging set has fixed registers; a padding
  // step (t == ntiles) computes an all-masked tile of zero rows, which leaves
  // every state unchanged, so the math is unconditional (a branch around it
  // would make the allocator copy the accumulators).
  auto step = [&](int t, Staged<FP8> &nx, Staged<FP8> &fill) {
    const int nb = t / kTilesPerIdxBlock + 1;  // the next index block
    const int blk = load_idx_block(row_idx, p0, p1, nb);
    load_rows<FP8, PACKED>(a, zrow, gl, tidx(t + 2), p0 + (t + 2) * kBK, p1, wave, lane, fill);
    compute_tile<RB, DS, PASS, P_HILO>(tile0 + (t & 1) * kTileBytes, sx, qreg, qk_base, pv_base, v_cur, wave,
                                       lane, grp, ds, a.scale_log2, w);
    store_rows<FP8>(tile0 + ((t + 1) & 1) * kTileBytes, wave, lane, nx);
    if (t % kTilesPerIdxBlock == kTilesPerIdxBlock - 3) ib0[(nb & 1) * kIdxBlock + threadIdx.x] = blk;
    __syncthreads();
    v_cur = tile_valid_bits(tidx(t + 1), p0 + (t + 1) * kBK, p1, lane, a.num_rows32);
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sb, sa);
    step(t + 1, sa, sb);
  }
}


// ----------------------------------------------------------------------------
// per-workgroup building blocks used by both kernels
// ----------------------------------------------------------------------------

// Q^T as the B operand of the QK MFMAs: chunk c of this wave's dim slice holds
// dims 32*cg + 8*grp .. +7 (cg = ds*NC + c) of query row qrow.
template <int DS>
__device__ __forceinline__ void load_q(const DecodeArgs &a, int64_t qrow, int ds, int grp,
                                       bf16x8 (&qreg)[16 / DS]) {
  constexpr int NC = 16 / DS;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int cg = ds * NC + c;
    const uint16_t *src = (cg < 14) ? a.q_nope + qrow * kNope + 32 * cg + 8 * grp
                                    : a.q_rope + qrow * kRope + 32 * (cg - 14) + 8 * grp;
    qreg[c] = *(const bf16x8 *)src;
  }
}

// Per-lane LDS offsets.  QK: row j, logical chunk 4c+grp -> physical
// (4c+grp) ^ swz(j); the xor only touches the low 4 chunk bits, so c>>2 is an
// immediate 256-byte step.  PV: lanes 4t+q of a group supply row 4grp+t at
// dims 16d+4q, logical chunk 2d+(q>>1), byte 8(q&1) within it.
__device__ __forceinline__ void lds_bases(int j, int grp, int (&qk_base)[4], int (&pv_base)[8]) {
  const int fj = swz(j);
#pragma unroll
  for (int c = 0; c < 4; ++c) qk_base[c] = j * kLdsRow + (((4 * c + grp) ^ fj) << 4);
  const int tq = j >> 2, qq = j & 3;
  const int tr_row = 4 * grp + tq;
  const int ftr = swz(tr_row);
#pragma unroll
  for (int d = 0; d < 8; ++d) pv_base[d] = tr_row * kLdsRow + (((2 * d + (qq >> 1)) ^ ftr) << 4) + ((qq & 1) << 3);
}

// Attend the workgroup's query rows over index positions [p0, p1) of row_idx:
// the main pass, and the exact-max two-pass redo when some score overflowed
// the reference max.  Leaves the unnormalised O^T, the reference max (log2
// domain) and this lane's share of the weight sum in w.
template <int RB, bool FP8, bool PACKED, bool P_HILO>
__device__ __forceinline__ void attend_range(const DecodeArgs &a, Smem<4 / RB> &sm, const int32_t *row_idx, int p0,
                                             int p1, int wave, int lane, int grp, int ds,
                                             const bf16x8 (&qreg)[4 * RB], const int (&qk_base)[4],
                                             const int (&pv_base)[8], WaveState<8 * RB> &w) {
  constexpr int DS = 4 / RB, ND = 32 / DS;
#pragma unroll
  for (int d = 0; d < ND; ++d) w.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  w.m_ref = -INFINITY;
  w.l_run = 0.f;
  w.overflow = false;
  run_split<RB, DS, FP8, PACKED, P_HILO, kPassMain>(a, sm, row_idx, p0, p1, wave, lane, grp, ds, qreg, qk_base,
                                                    pv_base, w);
  if (__syncthreads_or(w.overflow)) {
    // Rare: a score ran far above its row's first-tile max.  Redo the range
    // with the exact max (found by a scores-only sweep) as the reference.
#pragma unroll
    for (int d = 0; d < ND; ++d) w.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    w.m_ref = -INFINITY;
    w.l_run = 0.f;
    run_split<RB, DS, FP8, PACKED, P_HILO, kPassMax>(a, sm, row_idx, p0, p1, wave, lane, grp, ds, qreg, qk_base,
                                                     pv_base, w);
    run_split<RB, DS, FP8, PACKED, P_HILO, kPassFixed>(a, sm, row_idx, p0, p1, wave, lane, grp, ds, qreg,
                                                       qk_base, pv_base, w);
  }
}

// Total weight sum of this lane's query row (the same in all four 16-lane groups).
__device__ __forceinline__ float row_total(float l_run) {
  float l = l_run;
  l = group_sum(l);
  return l;
}

// Final bf16 output of one query row with the sink folded in (direct_scale).
// dst points at dim 16*dbase + 4*grp of the row; the lse is written when
// lse_dst is non-null.
template <int ND>
__device__ __forceinline__ void write_direct(const WaveState<ND> &w, float l_tot, float sink_ln, uint16_t *dst,
                                             float *lse_dst) {
  const OutScale sc = direct_scale(w.m_ref, l_tot, sink_ln);
#pragma unroll
  for (int d = 0; d < ND; ++d) *(u32x2 *)(dst + 16 * d) = pack_bf16x4(w.acc[d], sc.inv);
  if (lse_dst != nullptr) *lse_dst = sc.lse;
}

// Partial of one query row (no sink, partial_scale): o in bf16, the lse in
// fp32.  dst as in write_direct.
template <int ND>
__device__ __forceinline__ void write_partial_bf16(const WaveState<ND> &w, float l_tot, uint16_t *dst,
                                                   float *lse_dst) {
  const OutScale sc = partial_scale(w.m_ref, l_tot);
#pragma unroll
  for (int d = 0; d < ND; ++d) *(u32x2 *)(dst + 16 * d) = pack_bf16x4(w.acc[d], sc.inv);
  if (lse_dst != nullptr) *lse_dst = sc.lse;
}

}  // namespace smd
