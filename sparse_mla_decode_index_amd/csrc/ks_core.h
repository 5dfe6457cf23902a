// Building blocks of the wave-independent sparse MLA decode for gfx950
// (MI355X): row gather (bf16 and fp8 pools), softmax step, output epilogues.  The
// kernel's work decomposition and pipeline are in ks8_core.h.
//
// What is computed (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
// decode on gfx950", Design): per query row, a 512-wide dot product (448 NoPE
// + 64 RoPE dims) with every selected latent row, an online softmax that also
// counts a per-head sink logit, and a PV product over the same 512-wide rows.
//
// Gather: one load instruction per selected row, 16 bytes per lane, so a row
// is one contiguous 1 KiB read (the row base comes from a per-lane address
// vector by readlane).  Loading straight into MFMA operand order would put 16
// different rows on consecutive lanes, which costs the L1 one tag lookup per
// lane.  Invalid indices and positions past the range address a zero row, so
// every half-tile issues the same loads and the compiler's wait counts stay
// exact.
//
// Orientation: S^T[16 kv x 16 q] = K . Q^T with v_mfma_f32_16x16x32_bf16, so
// lane (j, g) holds the scores of query row j for kv rows 4g..4g+3 and the
// softmax statistics are per-lane values.  The softmax keeps a reference max
// per query row, fixed at its first valid half-tile (exp2 domain, scale
// pre-multiplied by log2(e)); a score more than 2^32 above it sends the wave
// through an exact-max second pass, so the accumulators are never rescaled.
#pragma once

#include "common.h"

namespace smd {
namespace ks {

using smd::bf16x4;
using smd::bf16x8;
using smd::exp2_fast;
using smd::f32_to_bf16_rne;
using smd::f32x4;
using smd::g_zero_row;
using smd::group_max;
using smd::group_sum;
using smd::kLn2;
using smd::kLog2e;
using smd::kPassFixed;
using smd::kPassMain;
using smd::kPassMax;
using smd::kRefSlackLog2;
using smd::Pass;
using smd::swz;
using smd::u32x2;
using smd::u32x4;
using smd::ue8m0_scale;

constexpr int kHalf = 16;                        // index positions per half-tile
constexpr int kRowBytes = 1024;                  // one bf16 row in LDS
constexpr int kHalfBytes = kHalf * kRowBytes;    // 16 KiB

// Gathered data of one half-tile in this lane's registers: v[i] = bytes
// 16*lane .. +16 of row i of the half-tile (i 0..15).
struct Half {
  u32x4 v[16];
};

// Per-lane constants.
struct Lane {
  int lane, r, q, j, g;  // r = kv row / j = query row (lane % 16); q = g = lane / 16
  int wb[4];             // QK A-operand read offsets (chunk group 0..3 of a 256-byte column)
  int pv[8];             // transposed-read offsets for dim block d & 7
};

__device__ __forceinline__ Lane make_lane(int lane) {
  Lane L;
  L.lane = lane;
  L.r = L.j = lane & 15;
  L.q = L.g = lane >> 4;
  const int sw = swz(L.r);
  // A operand of step ks: chunk 4ks + q of row r = 16*(ks >> 2) + (4*(ks & 3) + q);
  // the XOR stays inside the low 4 bits.
#pragma unroll
  for (int i = 0; i < 4; ++i) L.wb[i] = L.r * kRowBytes + (((4 * i + L.q) ^ sw) << 4);
  // PV: lanes 4t+u of group g read row 4g+t, dims 16d+4u..+4 = logical chunk
  // 2d + (u >> 1), byte 8(u & 1); chunk 2d = 16*(d >> 3) + 2(d & 7).
  const int t = L.j >> 2, u = L.j & 3;
  const int tr = 4 * L.g + t;
  const int ftr = swz(tr);
#pragma unroll
  for (int d = 0; d < 8; ++d) L.pv[d] = tr * kRowBytes + (((2 * d + (u >> 1)) ^ ftr) << 4) + ((u & 1) << 3);
  return L;
}

// The index list of one index row.  With two sources, positions [0, km) are
// entries of the first list (rows of the first pool) and positions [km, K)
// entries of the second list (rows of the second pool), in that order; with
// one source every position is in the first.
template <bool TWO>
struct Src {
  const int32_t *first;
  const int32_t *second;
  int km;
  __device__ __forceinline__ bool in_second(int p) const { return TWO && p >= km; }
  __device__ __forceinline__ int32_t at(int p) const {
    if constexpr (TWO)
      return *(p < km ? first + p : second + (p - km));
    else
      return first[p];
  }
  // index idx at position p names a row of its pool
  __device__ __forceinline__ bool row_ok(const DecodeArgs &a, int p, int32_t idx) const {
    return (uint32_t)idx < (in_second(p) ? a.num_rows2_32 : a.num_rows32);
  }
};

// Base of the NoPE / RoPE / code arrays of the pool a row comes from.
__device__ __forceinline__ const uint8_t *nope_base(const DecodeArgs &a, bool second) {
  return second ? a.kv2_nope : a.kv_nope;
}
__device__ __forceinline__ const uint8_t *rope_base(const DecodeArgs &a, bool second) {
  return second ? a.kv2_rope : a.kv_rope;
}
__device__ __forceinline__ const uint8_t *scale_base(const DecodeArgs &a, bool second) {
  return second ? a.kv2_scale : a.kv_scale;
}

// Address of row l % 16 of a half-tile in lane l: the selected NoPE row, or
// the zero row when the position is past the range or the index is invalid.
template <bool PACKED>
__device__ __forceinline__ uint64_t row_address(const DecodeArgs &a, uint32_t idx, bool valid, bool second) {
  const uint64_t stride = PACKED ? (uint64_t)a.row_stride32 : (uint64_t)a.nope_stride_b;
  return valid ? (uint64_t)(uintptr_t)(nope_base(a, second) + (uint64_t)idx * stride)
               : (uint64_t)(uintptr_t)g_zero_row;
}

// One contiguous 1 KiB load per row; row i's base is read from lane i of the
// address vector.  Split layouts (RoPE in its own array) take lanes 56..63
// from the RoPE row.
template <bool PACKED>
__device__ __forceinline__ void issue_half(const DecodeArgs &a, uint32_t idx, bool valid, bool second, const Lane &L,
                                           Half &h) {
  const uint64_t naddr = row_address<PACKED>(a, idx, valid, second);
  uint64_t raddr = 0;
  if constexpr (!PACKED)
    raddr = valid ? (uint64_t)(uintptr_t)(rope_base(a, second) + (uint64_t)idx * (uint64_t)a.rope_stride_b)
                  : (uint64_t)(uintptr_t)g_zero_row + 2 * kNope;
  // The rebuilt row pointers are global-address-space pointers, so the loads
  // are global loads with the row base in SGPRs: a generic (flat) load would
  // also count against the LDS wait counter and stall every LDS wait on it.
  typedef const uint8_t SMD_GLOBAL *gptr;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint64_t nb = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(naddr >> 32), i) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((uint32_t)naddr, i);
    if constexpr (PACKED) {
      h.v[i] = *(const u32x4 SMD_GLOBAL *)((gptr)(uintptr_t)nb + 16 * L.lane);
    } else {
      const uint64_t rb = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(raddr >> 32), i) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((uint32_t)raddr, i);
      const gptr p = L.lane < kNope / 8 ? (gptr)(uintptr_t)nb + 16 * L.lane
                                        : (gptr)(uintptr_t)rb + 16 * (L.lane - kNope / 8);
      h.v[i] = *(const u32x4 SMD_GLOBAL *)p;
    }
  }
}

// Gathered data of one fp8 half-tile.  A row is 448 e4m3 NoPE bytes with one
// UE8M0 code per 64-byte block, plus 64 bf16 RoPE dims (128 bytes).  Lane l
// serves row l / 4 and the quarter s = l % 4 of every 64-byte piece of it:
// n[t] = NoPE bytes 64t + 16s .. +16 (code block t), r[u] = RoPE bytes
// 64u + 16s .. +16, code = the row's 8 code bytes (7 codes + pad).  Four
// consecutive lanes read 64 contiguous bytes of one row.
struct Half8 {
  u32x4 n[7];
  u32x4 r[2];
  uint32_t code[2];
};

// Loads of one fp8 half-tile; idx / valid are those of row lane / 4.  Masked
// rows read the zero row (e4m3 zeros, code 0).
__device__ __forceinline__ void issue_half_fp8(const DecodeArgs &a, uint32_t idx, bool valid, bool second,
                                               const Lane &L, Half8 &h) {
  typedef const uint8_t SMD_GLOBAL *gptr;
  const uint8_t *z = g_zero_row;
  const gptr pn = (gptr)(uintptr_t)(valid ? nope_base(a, second) + (uint64_t)idx * (uint64_t)a.nope_stride_b : z);
  const gptr pr = (gptr)(uintptr_t)(valid ? rope_base(a, second) + (uint64_t)idx * (uint64_t)a.rope_stride_b : z);
  const gptr pc = (gptr)(uintptr_t)(valid ? scale_base(a, second) + (uint64_t)idx * (uint64_t)a.scale_stride_b : z);
  const int off = 16 * (L.lane & 3);
#pragma unroll
  for (int t = 0; t < 7; ++t) h.n[t] = *(const u32x4 SMD_GLOBAL *)(pn + off + 64 * t);
#pragma unroll
  for (int u = 0; u < 2; ++u) h.r[u] = *(const u32x4 SMD_GLOBAL *)(pr + off + 64 * u);
  h.code[0] = *(const uint32_t SMD_GLOBAL *)pc;
  h.code[1] = *(const uint32_t SMD_GLOBAL *)(pc + 4);
}

// Per-wave softmax state and O^T accumulator: acc[d][i] = sum over rows of
// 2^(x - m_ref) V[row][16d + 4g + i] for query row j of this lane.
struct State {
  f32x4 acc[32];
  float m_ref;    // reference max (log2 domain), the same in the four groups
  float l_run;    // this lane's share of sum 2^(x - m_ref)
  bool overflow;  // a score exceeded m_ref + kRefSlackLog2 (this lane)
};

// Softmax weights of one half-tile for this lane's 4 kv rows (4g..4g+3) of
// one query row, given that row's running state (reference max, this lane's
// share of the sum, overflow flag); vbits bit r = row r of the half-tile is
// valid.  Returns P as bf16 (and the low part of the two-part P with P_HILO).
template <int PASS, bool P_HILO>
__device__ __forceinline__ void softmax_step(f32x4 s, uint32_t vbits, float scale_log2, const Lane &L, float &m_ref,
                                             float &l_run, bool &overflow, bf16x4 &pb, bf16x4 &pl) {
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = ((vbits >> (4 * L.g + i)) & 1) ? s[i] * scale_log2 : -INFINITY;
  float tmax = group_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  if constexpr (PASS == kPassMax) {
    m_ref = fmaxf(m_ref, tmax);
    return;
  }
  if constexpr (PASS == kPassMain) {
    if (m_ref == -INFINITY) m_ref = tmax;  // nothing accumulated yet for this row
    overflow |= tmax > m_ref + kRefSlackLog2;
  }
  const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = exp2_fast(x[i] - m_use);
    psum += p;
    pb[i] = (__bf16)p;
    // P_HILO: p = hi + lo with both parts bf16, so the PV product carries
    // about 16 significant bits of p instead of 8 (FP32-partial precision).
    if constexpr (P_HILO) pl[i] = (__bf16)(p - (float)pb[i]);
  }
  l_run += psum;
}

template <int PASS, bool P_HILO>
__device__ __forceinline__ void softmax_half(f32x4 s, uint32_t vbits, float scale_log2, const Lane &L, State &st,
                                             bf16x4 &pb, bf16x4 &pl) {
  softmax_step<PASS, P_HILO>(s, vbits, scale_log2, L, st.m_ref, st.l_run, st.overflow, pb, pl);
}

// Final bf16 output of one query row with the sink folded in (direct_scale);
// dst points at dim 128*w + 4g of the row for the w-th quarter of the dims;
// the lse is written when lse_dst is non-null.
__device__ __forceinline__ void write_direct(const f32x4 (&o)[8], float m, float l, float sink_ln, uint16_t *dst,
                                             float *lse_dst) {
  const OutScale sc = direct_scale(m, l, sink_ln);
#pragma unroll
  for (int d = 0; d < 8; ++d) *(u32x2 *)(dst + 16 * d) = pack_bf16x4(o[d], sc.inv);
  if (lse_dst != nullptr) *lse_dst = sc.lse;
}

// FP32 partial of one query row (no sink, partial_scale).  dst as in write_direct.
__device__ __forceinline__ void write_partial(const f32x4 (&o)[8], float m, float l, float *dst, float *lse_dst) {
  const OutScale sc = partial_scale(m, l);
#pragma unroll
  for (int d = 0; d < 8; ++d) *(f32x4 *)(dst + 16 * d) = o[d] * sc.inv;
  if (lse_dst != nullptr) *lse_dst = sc.lse;
}

// The same partial with o rounded to bf16 (lse stays FP32): the form of
// partials that only feed the merge.  dst indexes bf16 elements.
__device__ __forceinline__ void write_partial_bf16(const f32x4 (&o)[8], float m, float l, uint16_t *dst,
                                                   float *lse_dst) {
  const OutScale sc = partial_scale(m, l);
#pragma unroll
  for (int d = 0; d < 8; ++d) *(u32x2 *)(dst + 16 * d) = pack_bf16x4(o[d], sc.inv);
  if (lse_dst != nullptr) *lse_dst = sc.lse;
}

// A partial as the call needs it: FP32 when the caller reads the partials
// (hilo), bf16 in the same buffer when they only feed the merge.  off is the
// element offset of the row's first dim.
__device__ __forceinline__ void write_partial_any(bool f32, const f32x4 (&o)[8], float m, float l, float *part_o,
                                                  int64_t off, float *lse_dst) {
  if (f32)
    write_partial(o, m, l, part_o + off, lse_dst);
  else
    write_partial_bf16(o, m, l, (uint16_t *)part_o + off, lse_dst);
}

}  // namespace ks
}  // namespace smd
