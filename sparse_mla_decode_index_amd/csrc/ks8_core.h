// Device core of the wave-independent sparse MLA decode.
//
// A workgroup of 8 waves owns one block of 16 query rows (heads x MTP
// positions sharing one index list) and a range of index positions, cut into
// half-tiles of 16 positions; wave w takes half-tiles w, w+8, w+16, ... and
// computes all 512 dims of the 16 query rows, so the main loop needs no
// barrier: the waves only meet at the end, where their (O, m, l) states are
// merged through LDS.  It is laid out for two waves per SIMD, so that one
// wave's memory and LDS waits overlap the other's issue:
//   - Q^T sits once in LDS (16 KiB, shared by the 8 waves) instead of in
//     every wave's VGPRs; QK reads its B operand from there;
//   - one gathered register set per wave: the rows of half-tile k+1 are in
//     flight while half-tile k is computed;
//   - one 16 KiB LDS buffer per wave; PV runs per half-tile with
//     v_mfma_f32_16x16x16_bf16 (k = 16 rows), V^T by ds_read_b64_tr_b16.
// fp8 pools are gathered as e4m3 bytes + UE8M0 codes + bf16 RoPE and
// dequantised in registers on the way into LDS (e4m3 x 2^(code-127) is exact
// in bf16), so the buffer layout and everything after it are the bf16 ones.
// LDS: 16 KiB + 8 x 16 KiB = 144 KiB per workgroup.
#pragma once

#include "ks_core.h"

namespace smd {
namespace ks8 {

using ks::bf16x4;
using ks::bf16x8;
using ks::f32x4;
using ks::Half;
using ks::Lane;
using ks::State;
using ks::u32x2;
using ks::u32x4;

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kHalf = ks::kHalf;
constexpr int kHalfBytes = ks::kHalfBytes;

struct Smem {
  uint8_t q[16 * 64 * 16];         // Q^T: 16 B per (k-step, lane)
  uint8_t buf[kWaves][kHalfBytes];  // one half-tile buffer per wave
  float stat_m[4][16];
  float stat_l[4][16];
};

// Q^T of the block into LDS: B operand of k-step ks for lane l = dims
// 32ks + 8(l/16) .. +8 of query row l % 16.  Each wave stores two k-steps.
__device__ __forceinline__ void stage_q(const DecodeArgs &a, int64_t qrow, int wave, const Lane &L, Smem &sm) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ks = 2 * wave + h;
    const uint16_t *src = ks < 14 ? a.q_nope + qrow * kNope + 32 * ks + 8 * L.q
                                  : a.q_rope + qrow * kRope + 32 * (ks - 14) + 8 * L.q;
    *(u32x4 SMD_LDS *)((uint8_t SMD_LDS *)sm.q + (ks * 64 + L.lane) * 16) = *(const u32x4 *)src;
  }
}

// Row formats of the pool: bf16 with RoPE right after NoPE in one row, bf16
// with RoPE in its own array, fp8 e4m3 NoPE + UE8M0 codes + bf16 RoPE.
enum Fmt { kBf16Packed = 0, kBf16Split = 1, kFp8 = 2 };

template <int FMT>
struct Gathered {
  typedef Half type;
};
template <>
struct Gathered<kFp8> {
  typedef ks::Half8 type;
};

// Gathered bf16 rows of a half-tile into the wave's buffer: row i, chunk
// `lane` -> physical chunk lane ^ swz(i) (one row of 64 distinct chunks per
// store).
__device__ __forceinline__ void store_half(const Half &h, uint8_t SMD_LDS *buf, const Lane &L) {
#pragma unroll
  for (int i = 0; i < 16; ++i) *(u32x4 SMD_LDS *)(buf + i * ks::kRowBytes + ((L.lane ^ ks::swz(i)) << 4)) = h.v[i];
}

// Gathered fp8 rows, dequantised, into the same layout: the 16 e4m3 bytes of
// block t, quarter s become bf16 chunks 8t + 2s and 8t + 2s + 1; RoPE piece u
// is chunk 56 + 4u + s.  Odd rows store their odd chunk first, so each
// 8-lane group of a store covers 8 distinct 16-byte bank groups.
__device__ __forceinline__ void store_half(const ks::Half8 &h, uint8_t SMD_LDS *buf, const Lane &L) {
  const int r = L.lane >> 2, s = L.lane & 3;
  const int sw = ks::swz(r);
  const int e = r & 1;
  uint8_t SMD_LDS *row = buf + r * ks::kRowBytes;
#pragma unroll
  for (int t = 0; t < 7; ++t) {
    const float sc = ks::ue8m0_scale((h.code[t >> 2] >> (8 * (t & 3))) & 0xffu);
    u32x4 c[2];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      c[w >> 1][2 * (w & 1)] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)h.n[t][w], sc, false));
      c[w >> 1][2 * (w & 1) + 1] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)h.n[t][w], sc, true));
    }
    const int c0 = 8 * t + 2 * s;
    *(u32x4 SMD_LDS *)(row + (((c0 + e) ^ sw) << 4)) = e ? c[1] : c[0];
    *(u32x4 SMD_LDS *)(row + (((c0 + 1 - e) ^ sw) << 4)) = e ? c[0] : c[1];
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) *(u32x4 SMD_LDS *)(row + (((56 + 4 * u + s) ^ sw) << 4)) = h.r[u];
}

// QK over the half-tile in `buf`: A operands from the buffer, B operands from
// the shared Q^T.
__device__ __forceinline__ f32x4 qk_lds(const uint8_t SMD_LDS *qs, const uint8_t SMD_LDS *buf, const Lane &L) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  constexpr int kPre = 2;
  bf16x8 ka[kPre], kb[kPre];
  auto load = [&](int ks) {
    ka[ks % kPre] = *(const bf16x8 SMD_LDS *)(buf + L.wb[ks & 3] + 256 * (ks >> 2));
    kb[ks % kPre] = *(const bf16x8 SMD_LDS *)(qs + (ks * 64 + L.lane) * 16);
  };
#pragma unroll
  for (int ks = 0; ks < kPre; ++ks) load(ks);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const bf16x8 k = ka[ks % kPre], q = kb[ks % kPre];
    if (ks + kPre < 16) load(ks + kPre);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, q, s, 0, 0, 0);
  }
  return s;
}

// PV over one half-tile (after the half-tile's softmax): O^T[512 x 16] += V^T[512 x 16] . P^T[16 x 16]; lane
// (j, g) supplies P of kv rows 4g..4g+3 for query row j, the transposed read
// gives dim 16d + (lane % 16) of rows 4g..4g+3.
template <bool P_HILO>
__device__ __forceinline__ void pv_half(const uint8_t SMD_LDS *buf, bf16x4 p, bf16x4 pl, const Lane &L, State &st) {
  const s16x4 pb = __builtin_bit_cast(s16x4, p);
  s16x4 plb;
  if constexpr (P_HILO) plb = __builtin_bit_cast(s16x4, pl);
  constexpr int kPre = 4;
  bf16x4 v[kPre];
  auto load = [&](int d) {
    v[d % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(buf + L.pv[d & 7] + 256 * (d >> 3)));
  };
#pragma unroll
  for (int d = 0; d < kPre; ++d) load(d);
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const s16x4 va = __builtin_bit_cast(s16x4, v[d % kPre]);
    if (d + kPre < 32) load(d + kPre);
    st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.acc[d], 0, 0, 0);
    if constexpr (P_HILO) st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plb, st.acc[d], 0, 0, 0);
  }
}

// The gather pipeline of one wave: the register set with the rows of the
// next half-tile to compute, the indices of the half-tile after it, and the
// valid-row bits of the rows in the register set.
template <int FMT>
struct Pipe {
  typename Gathered<FMT>::type h;
  int32_t i_next;  // index of row row_of<FMT>(L) of the next-but-one half-tile
  uint32_t vb;
  int nk;  // half-tiles of this wave
};

// The half-tile row whose index this lane holds (and, for fp8, gathers).
template <int FMT>
__device__ __forceinline__ int row_of(const Lane &L) {
  return FMT == kFp8 ? (L.lane >> 2) : L.r;
}

// Half-tile k of this wave covers positions p0 + 16*(wave + 8k) + 0..15.
template <int FMT>
__device__ __forceinline__ int pos_of(int p0, int wave, int k, const Lane &L) {
  return p0 + kHalf * (wave + kWaves * k) + row_of<FMT>(L);
}

// Valid-row bits of a half-tile (bit r = row r) from each lane's validity of
// row row_of<FMT>(lane); fp8 lanes 4r..4r+3 share row r.
template <int FMT>
__device__ __forceinline__ uint32_t row_bits(bool v) {
  uint64_t b = __ballot(v);
  if constexpr (FMT == kFp8) {
    b &= 0x1111111111111111ull;
    b = (b | (b >> 3)) & 0x0303030303030303ull;
    b = (b | (b >> 6)) & 0x000F000F000F000Full;
    b = (b | (b >> 12)) & 0x000000FF000000FFull;
    b = b | (b >> 24);
  }
  return (uint32_t)b & 0xffffu;
}

template <int FMT>
__device__ __forceinline__ void issue(const DecodeArgs &a, uint32_t idx, bool valid, bool second, const Lane &L,
                                      typename Gathered<FMT>::type &h) {
  if constexpr (FMT == kFp8)
    ks::issue_half_fp8(a, idx, valid, second, L, h);
  else
    ks::issue_half<FMT == kBf16Packed>(a, idx, valid, second, L, h);
}

// Start the pipeline: indices of half-tiles 0 and 1, rows of half-tile 0.
template <int FMT, class SRC>
__device__ __forceinline__ void prime(const DecodeArgs &a, const SRC &src, int p0, int p1, int wave, const Lane &L,
                                      Pipe<FMT> &pp) {
  const int nh = (p1 - p0 + kHalf - 1) / kHalf;
  pp.nk = nh > wave ? (nh - wave + kWaves - 1) / kWaves : 0;
  if (pp.nk == 0) return;
  const int q0 = min(pos_of<FMT>(p0, wave, 0, L), p1 - 1);
  const int32_t i0 = src.at(q0);
  pp.i_next = src.at(min(pos_of<FMT>(p0, wave, 1, L), p1 - 1));
  const bool v0 = pos_of<FMT>(p0, wave, 0, L) < p1 && src.row_ok(a, q0, i0);
  issue<FMT>(a, (uint32_t)i0, v0, src.in_second(q0), L, pp.h);
  pp.vb = row_bits<FMT>(v0);
}

// One wave's sweep over its half-tiles of [p0, p1), from a primed pipeline.
// Per half-tile k: store the gathered rows of k, refill the register set with
// the rows of k+1 (their indices were loaded one step earlier), load the
// indices of k+2, then QK, softmax and PV of k from LDS while k+1 is in
// flight.  Every step issues the same loads (positions past p1 read the zero
// row), so the compiler's wait counts stay exact.
template <int FMT, bool P_HILO, int PASS, class SRC>
__device__ __forceinline__ void sweep(const DecodeArgs &a, const SRC &src, int p0, int p1, int wave, const Lane &L,
                                      const uint8_t SMD_LDS *qs, uint8_t SMD_LDS *buf, State &st, Pipe<FMT> &pp) {
  for (int k = 0; k < pp.nk; ++k) {
    store_half(pp.h, buf, L);
    const int qn = min(pos_of<FMT>(p0, wave, k + 1, L), p1 - 1);
    const bool vn = pos_of<FMT>(p0, wave, k + 1, L) < p1 && src.row_ok(a, qn, pp.i_next);
    issue<FMT>(a, (uint32_t)pp.i_next, vn, src.in_second(qn), L, pp.h);
    pp.i_next = src.at(min(pos_of<FMT>(p0, wave, k + 2, L), p1 - 1));
    const uint32_t vb = pp.vb;
    pp.vb = row_bits<FMT>(vn);
    const f32x4 s = qk_lds(qs, buf, L);
    bf16x4 p, pl;
    ks::softmax_half<PASS, P_HILO>(s, vb, a.scale_log2, L, st, p, pl);
    if constexpr (PASS != ks::kPassMax) pv_half<P_HILO>(buf, p, pl, L, st);
  }
}

// The wave's attention over its share of [p0, p1) from a primed pipeline: the
// main sweep, and the exact-max redo when a score overflowed the reference.
template <int FMT, bool P_HILO, class SRC>
__device__ __forceinline__ void attend(const DecodeArgs &a, const SRC &src, int p0, int p1, int wave, const Lane &L,
                                       const uint8_t SMD_LDS *qs, uint8_t SMD_LDS *buf, State &st, Pipe<FMT> &pp) {
#pragma unroll
  for (int d = 0; d < 32; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_ref = -INFINITY;
  st.l_run = 0.f;
  st.overflow = false;
  sweep<FMT, P_HILO, ks::kPassMain>(a, src, p0, p1, wave, L, qs, buf, st, pp);
  if (__ballot(st.overflow)) {  // wave-uniform
    // Rare: a score ran far above its row's first-half-tile max.  Redo this
    // wave's share with the exact max (a scores-only sweep) as the reference.
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.l_run = 0.f;
    prime<FMT>(a, src, p0, p1, wave, L, pp);
    sweep<FMT, P_HILO, ks::kPassMax>(a, src, p0, p1, wave, L, qs, buf, st, pp);
    prime<FMT>(a, src, p0, p1, wave, L, pp);
    sweep<FMT, P_HILO, ks::kPassFixed>(a, src, p0, p1, wave, L, qs, buf, st, pp);
  }
}

// Merge of the eight waves' states.  Waves 4..7 hand their states to waves
// 0..3 through LDS; then each of waves 0..3 dumps its state and reduces a
// quarter of the dims over the four: each ends
// with dims 16d + 4g + i, d = 8w .. 8w+7, of this lane's query row j in o,
// the merged reference max m and weight sum l.  Returns false on waves 4..7.
__device__ __forceinline__ bool merge_waves(Smem &sm, int wave, const Lane &L, State &st, f32x4 (&o)[8], float &m,
                                            float &l) {
  __syncthreads();  // every wave is done with Q^T and its buffer
  uint8_t SMD_LDS *base = (uint8_t SMD_LDS *)&sm.buf[0][0];  // 128 KiB: 4 states of 32 KiB
  f32x4 SMD_LDS *dump = (f32x4 SMD_LDS *)(base + (wave & 3) * 32768);
  float SMD_LDS *side = (float SMD_LDS *)&sm.q[0] + (wave & 3) * 128;  // m_ref, l_run per lane
  if (wave >= 4) {
#pragma unroll
    for (int d = 0; d < 32; ++d) dump[d * 64 + L.lane] = st.acc[d];
    side[L.lane] = st.m_ref;
    side[64 + L.lane] = st.l_run;
  }
  __syncthreads();
  if (wave < 4) {
    const float mb = side[L.lane], lb = side[64 + L.lane];
    const float mm = fmaxf(st.m_ref, mb);
    const float sa = st.m_ref == -INFINITY ? 0.f : ks::exp2_fast(st.m_ref - mm);
    const float sb = mb == -INFINITY ? 0.f : ks::exp2_fast(mb - mm);
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[d] = st.acc[d] * sa + dump[d * 64 + L.lane] * sb;
    st.m_ref = mm;
    st.l_run = st.l_run * sa + lb * sb;
  }
  __syncthreads();
  // four-wave merge over the same 128 KiB (each of waves 0..3 dumps its state
  // into its own 32 KiB)
  if (wave < 4) {
#pragma unroll
    for (int d = 0; d < 32; ++d) dump[d * 64 + L.lane] = st.acc[d];
    const float l_row = ks::group_sum(st.l_run);
    if (L.g == 0) {
      sm.stat_m[wave][L.j] = st.m_ref;
      sm.stat_l[wave][L.j] = l_row;
    }
  }
  __syncthreads();
  if (wave >= 4) return false;
  float mw[4], lw[4];
  m = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = sm.stat_m[w][L.j];
    lw[w] = sm.stat_l[w][L.j];
    m = fmaxf(m, mw[w]);
  }
  l = 0.f;
  float sc[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sc[w] = mw[w] == -INFINITY ? 0.f : ks::exp2_fast(mw[w] - m);
    l += sc[w] * lw[w];
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 SMD_LDS *src = (const f32x4 SMD_LDS *)(base + w * 32768);
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] += sc[w] * src[(8 * wave + d) * 64 + L.lane];
  }
  return true;
}

}  // namespace ks8
}  // namespace smd
