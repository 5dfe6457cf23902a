// Device core of sparse MLA decode for gfx950 (MI355X): wave-independent
// attention of one 16-query-row block over a range of index positions.
//
// What is computed (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
// decode on gfx950", Design): per query row, a 512-wide dot product (448 NoPE
// + 64 RoPE dims) with every selected latent row, an online softmax that also
// counts a per-head sink logit, and a PV product over the same 512-wide rows.
//
// Work decomposition.  A workgroup of 4 waves owns one block of 16 query rows
// (heads x MTP positions sharing one index list) and a range [p0, p1) of index
// positions.  The range is cut into half-tiles of 16 positions; wave w takes
// half-tiles w, w+4, w+8, ...  Each wave owns all 512 dims of the 16 query
// rows, so the main loop needs no barrier: the waves only meet at the end,
// where their (O, m, l) states are merged through LDS.
//
// Per half-tile, per wave:
//   gather   bf16 pools (fp8 pools use the row-block kernel): one load
//            instruction per selected row, 16 bytes per lane, so a row is one
//            contiguous 1 KiB read (the row base comes from a per-lane address
//            vector by readlane).  Each wave stores its rows to its own LDS
//            buffer (16 KiB, 16-byte chunks XOR-swizzled), from which QK reads
//            its A operands and PV its transposed V^T.  (Loading straight into
//            MFMA operand order would put 16 different rows on consecutive
//            lanes, which costs the L1 one tag lookup per lane.)  Invalid
//            indices and positions past p1 address a zero row, so every
//            half-tile issues the same loads and the compiler's wait counts
//            stay exact.
//   QK       S^T[16 kv x 16 q] = K . Q^T with v_mfma_f32_16x16x32_bf16; Q^T
//            stays resident (64 VGPRs).  In this orientation lane (j, g) holds
//            the scores of query row j for kv rows 4g..4g+3, so the softmax
//            statistics are per-lane values.
//   softmax  a reference max per query row, fixed at its first valid
//            half-tile (exp2 domain, scale pre-multiplied by log2(e)); a score
//            more than 2^32 above it sends the wave through an exact-max
//            second pass, so the accumulators are never rescaled.
//   PV       every second half-tile,
//            O^T[512 x 16] += V^T[512 x 32] . P^T[32 x 16] with V^T read by
//            ds_read_b64_tr_b16 from the two buffers and P^T taken from the
//            softmax registers.
#pragma once

#include "smd_internal.h"

#include <math.h>

namespace smd {
namespace ks {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SMD_LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;                        // waves per workgroup
constexpr int kHalf = 16;                        // index positions per half-tile
constexpr int kRowBytes = 1024;                  // one bf16 row in LDS
constexpr int kHalfBytes = kHalf * kRowBytes;    // 16 KiB
constexpr int kWaveLds = 2 * kHalfBytes;         // two half-tile buffers per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A row's reference max is fixed at its first valid half-tile; a later score
// more than this far above it (log2 domain) triggers the exact-max second pass.
constexpr float kRefSlackLog2 = 32.f;

// Zero bytes read in place of every masked row.
static __device__ __attribute__((aligned(256))) uint8_t g_zero_row[1024];

// Shared memory of a workgroup: the waves' half-tile buffers, reused at the end
// for the cross-wave merge (each wave then dumps its accumulators into its
// own 32 KiB), plus the per-row statistics of the merge.
struct Smem {
  uint8_t buf[kWaves][kWaveLds];
  float stat_m[kWaves][16];
  float stat_l[kWaves][16];
};

// XOR permutation of the 16-byte chunks of row r in a half-tile buffer.  It
// only touches the low 4 chunk bits and makes conflict-free both the 16-byte
// stores of the gathered pieces (16 rows x 4 chunks per instruction) and the
// 8-byte transposed reads (16 rows x 2 chunks per instruction).
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four 16-lane groups (lanes j, j+16, j+32, j+48) with the
// gfx950 permlane swaps (VALU, no LDS round trip).
__device__ __forceinline__ float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

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

// Q^T as the B operand of the QK MFMAs: step ks = dims 32ks + 8q .. +8
// (ks < 14 from q_nope, 14 and 15 from q_rope).
__device__ __forceinline__ void load_q(const DecodeArgs &a, int64_t qrow, int q, bf16x8 (&qreg)[16]) {
  const uint16_t *qn = a.q_nope + qrow * kNope;
  const uint16_t *qr = a.q_rope + qrow * kRope;
#pragma unroll
  for (int s = 0; s < 14; ++s) qreg[s] = *(const bf16x8 *)(qn + 32 * s + 8 * q);
#pragma unroll
  for (int s = 0; s < 2; ++s) qreg[14 + s] = *(const bf16x8 *)(qr + 32 * s + 8 * q);
}

// Address of row l % 16 of a half-tile in lane l: the selected NoPE row, or
// the zero row when the position is past the range or the index is invalid.
template <bool PACKED>
__device__ __forceinline__ uint64_t row_address(const DecodeArgs &a, uint32_t idx, bool valid) {
  const uint64_t stride = PACKED ? (uint64_t)a.row_stride32 : (uint64_t)a.nope_stride_b;
  return valid ? (uint64_t)(uintptr_t)(a.kv_nope + (uint64_t)idx * stride) : (uint64_t)(uintptr_t)g_zero_row;
}

// One contiguous 1 KiB load per row; row i's base is read from lane i of the
// address vector.  Split layouts (RoPE in its own array) take lanes 56..63
// from the RoPE row.
template <bool PACKED>
__device__ __forceinline__ void issue_half(const DecodeArgs &a, uint32_t idx, bool valid, const Lane &L, Half &h) {
  const uint64_t naddr = row_address<PACKED>(a, idx, valid);
  uint64_t raddr = 0;
  if constexpr (!PACKED)
    raddr = valid ? (uint64_t)(uintptr_t)(a.kv_rope + (uint64_t)idx * (uint64_t)a.rope_stride_b)
                  : (uint64_t)(uintptr_t)g_zero_row + 2 * kNope;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint64_t nb = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(naddr >> 32), i) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((uint32_t)naddr, i);
    if constexpr (PACKED) {
      h.v[i] = *(const u32x4 *)((const uint8_t *)(uintptr_t)nb + 16 * L.lane);
    } else {
      const uint64_t rb = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(raddr >> 32), i) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((uint32_t)raddr, i);
      const uint8_t *p = L.lane < kNope / 8 ? (const uint8_t *)(uintptr_t)nb + 16 * L.lane
                                            : (const uint8_t *)(uintptr_t)rb + 16 * (L.lane - kNope / 8);
      h.v[i] = *(const u32x4 *)p;
    }
  }
}

// QK over one half-tile: the gathered rows are stored to the LDS buffer `buf`
// (row i, chunk `lane` -> physical chunk lane ^ swz(i): one row of 64 distinct
// chunks per instruction, conflict-free) and the A operands read back (step
// ks: 16 rows x chunks 4ks + q, also conflict-free).
__device__ __forceinline__ f32x4 qk_half(const Half &h, const bf16x8 (&qreg)[16], uint8_t SMD_LDS *buf,
                                         const Lane &L) {
#pragma unroll
  for (int i = 0; i < 16; ++i) *(u32x4 SMD_LDS *)(buf + i * kRowBytes + ((L.lane ^ swz(i)) << 4)) = h.v[i];
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  constexpr int kPre = 4;  // LDS reads issued ahead of the QK MFMAs
  bf16x8 ka[kPre];
#pragma unroll
  for (int ks = 0; ks < kPre; ++ks) ka[ks] = *(const bf16x8 SMD_LDS *)(buf + L.wb[ks & 3] + 256 * (ks >> 2));
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const bf16x8 k = ka[ks % kPre];
    if (ks + kPre < 16)
      ka[ks % kPre] = *(const bf16x8 SMD_LDS *)(buf + L.wb[(ks + kPre) & 3] + 256 * ((ks + kPre) >> 2));
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qreg[ks], s, 0, 0, 0);
  }
  return s;
}

// Per-wave softmax state and O^T accumulator: acc[d][i] = sum over rows of
// 2^(x - m_ref) V[row][16d + 4g + i] for query row j of this lane.
struct State {
  f32x4 acc[32];
  float m_ref;    // reference max (log2 domain), the same in the four groups
  float l_run;    // this lane's share of sum 2^(x - m_ref)
  bool overflow;  // a score exceeded m_ref + kRefSlackLog2 (this lane)
};

enum Pass { kPassMain = 0, kPassMax = 1, kPassFixed = 2 };

// Softmax weights of one half-tile for this lane's 4 kv rows (4g..4g+3);
// vbits bit r = row r of the half-tile is valid.  Returns P as bf16 (and the
// low part of the two-part P with P_HILO).
template <int PASS, bool P_HILO>
__device__ __forceinline__ void softmax_half(f32x4 s, uint32_t vbits, float scale_log2, const Lane &L, State &st,
                                             bf16x4 &pb, bf16x4 &pl) {
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = ((vbits >> (4 * L.g + i)) & 1) ? s[i] * scale_log2 : -INFINITY;
  float tmax = group_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  if constexpr (PASS == kPassMax) {
    st.m_ref = fmaxf(st.m_ref, tmax);
    return;
  }
  if constexpr (PASS == kPassMain) {
    if (st.m_ref == -INFINITY) st.m_ref = tmax;  // nothing accumulated yet for this row
    st.overflow |= tmax > st.m_ref + kRefSlackLog2;
  }
  const float m_use = st.m_ref == -INFINITY ? 0.f : st.m_ref;
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
  st.l_run += psum;
}

// PV over a pair of half-tiles held in LDS buffers ba (positions of the first
// half) and bb (second half): k slot 8g + u is row 4g + u of the first half
// for u < 4 and row 4g + u - 4 of the second half otherwise, in both operands.
template <bool P_HILO>
__device__ __forceinline__ void pv_pair(const uint8_t SMD_LDS *ba, const uint8_t SMD_LDS *bb, bf16x4 pa, bf16x4 pb,
                                        bf16x4 la, bf16x4 lb, const Lane &L, State &st) {
  const bf16x8 p = __builtin_shufflevector(pa, pb, 0, 1, 2, 3, 4, 5, 6, 7);
  bf16x8 pl;
  if constexpr (P_HILO) pl = __builtin_shufflevector(la, lb, 0, 1, 2, 3, 4, 5, 6, 7);
  constexpr int kPre = 4;  // transposed-read pairs issued ahead of the PV MFMAs
  bf16x4 va[kPre], vb[kPre];
  auto load = [&](int d) {
    const int off = L.pv[d & 7] + 256 * (d >> 3);
    va[d % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(ba + off));
    vb[d % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(bb + off));
  };
#pragma unroll
  for (int d = 0; d < kPre; ++d) load(d);
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const bf16x8 v = __builtin_shufflevector(va[d % kPre], vb[d % kPre], 0, 1, 2, 3, 4, 5, 6, 7);
    if (d + kPre < 32) load(d + kPre);
    st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, p, st.acc[d], 0, 0, 0);
    if constexpr (P_HILO) st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pl, st.acc[d], 0, 0, 0);
  }
}

// One wave's sweep over its half-tiles of [p0, p1) (half-tile k of this wave
// covers positions p0 + 16*(wave + 4k) + 0..15).  Pipeline per half-tile k:
// load the indices of k+3, consume the gathered registers of k (QK, LDS
// store), refill them with the rows of k+2, softmax, and every second
// half-tile PV over the pair.  Two register sets alternate, so the rows of
// one half-tile are always in flight while another is computed; every step
// issues the same loads (positions past p1 read the zero row), which keeps the
// compiler's wait counts exact.  Odd counts are padded with an all-masked
// half-tile, which leaves the state unchanged.
template <bool PACKED, bool P_HILO, int PASS>
__device__ __forceinline__ void sweep(const DecodeArgs &a, const int32_t *row_idx, int p0, int p1, int wave,
                                      const Lane &L, const bf16x8 (&qreg)[16], uint8_t SMD_LDS *wbuf, State &st) {
  const int nh = (p1 - p0 + kHalf - 1) / kHalf;              // half-tiles of the range
  const int nk = nh > wave ? (nh - wave + kWaves - 1) / kWaves : 0;  // ... of this wave
  if (nk == 0) return;
  const int nk2 = (nk + 1) & ~1;
  auto pos_of = [&](int k) { return p0 + kHalf * (wave + kWaves * k) + L.r; };
  auto load_idx = [&](int k) { return row_idx[min(pos_of(k), p1 - 1)]; };
  auto valid_of = [&](int k, int32_t idx) { return pos_of(k) < p1 && (uint32_t)idx < a.num_rows32; };

  Half hx, hy;
  int32_t i0 = load_idx(0), i1 = load_idx(1);
  int32_t i2 = load_idx(2);
  bool v0 = valid_of(0, i0), v1 = valid_of(1, i1);
  issue_half<PACKED>(a, (uint32_t)i0, v0, L, hx);
  issue_half<PACKED>(a, (uint32_t)i1, v1, L, hy);
  uint32_t vb_x = (uint32_t)__ballot(v0) & 0xffffu, vb_y = (uint32_t)__ballot(v1) & 0xffffu;
  int32_t i_even = i2, i_odd = 0;  // indices of half-tiles k+2 for the next even / odd step
  bf16x4 pa, la, pb, lb;

  for (int k = 0; k < nk2; k += 2) {
    // ---- even step: half-tile k in hx (buffer 0)
    i_odd = load_idx(k + 3);
    {
      const f32x4 s = qk_half(hx, qreg, wbuf, L);
      const uint32_t vb = vb_x;
      const bool vn = valid_of(k + 2, i_even);
      issue_half<PACKED>(a, (uint32_t)i_even, vn, L, hx);
      vb_x = (uint32_t)__ballot(vn) & 0xffffu;
      softmax_half<PASS, P_HILO>(s, vb, a.scale_log2, L, st, pa, la);
    }
    // ---- odd step: half-tile k+1 in hy (buffer 1), then PV over the pair
    i_even = load_idx(k + 4);
    {
      const f32x4 s = qk_half(hy, qreg, wbuf + kHalfBytes, L);
      const uint32_t vb = vb_y;
      const bool vn = valid_of(k + 3, i_odd);
      issue_half<PACKED>(a, (uint32_t)i_odd, vn, L, hy);
      vb_y = (uint32_t)__ballot(vn) & 0xffffu;
      softmax_half<PASS, P_HILO>(s, vb, a.scale_log2, L, st, pb, lb);
    }
    if constexpr (PASS != kPassMax) pv_pair<P_HILO>(wbuf, wbuf + kHalfBytes, pa, pb, la, lb, L, st);
  }
}

// The wave's attention over its share of [p0, p1): the main sweep, and the
// exact-max redo when a score overflowed the reference max.
template <bool PACKED, bool P_HILO>
__device__ __forceinline__ void attend(const DecodeArgs &a, const int32_t *row_idx, int p0, int p1, int wave,
                                       const Lane &L, const bf16x8 (&qreg)[16], uint8_t SMD_LDS *wbuf, State &st) {
#pragma unroll
  for (int d = 0; d < 32; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_ref = -INFINITY;
  st.l_run = 0.f;
  st.overflow = false;
  sweep<PACKED, P_HILO, kPassMain>(a, row_idx, p0, p1, wave, L, qreg, wbuf, st);
  if (__ballot(st.overflow)) {  // wave-uniform
    // Rare: a score ran far above its row's first-half-tile max.  Redo this
    // wave's share with the exact max (a scores-only sweep) as the reference.
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.l_run = 0.f;
    sweep<PACKED, P_HILO, kPassMax>(a, row_idx, p0, p1, wave, L, qreg, wbuf, st);
    sweep<PACKED, P_HILO, kPassFixed>(a, row_idx, p0, p1, wave, L, qreg, wbuf, st);
  }
}

// Merge of the four waves' states through LDS.  Afterwards wave v holds, for
// this lane's query row j, the merged sum over dims 16d + 4g + i with
// d = 8v .. 8v+7 in o[d - 8v], the merged reference max m (log2 domain, -inf
// when no valid entry) and the merged weight sum l.
__device__ __forceinline__ void merge_waves(Smem &sm, int wave, const Lane &L, const State &st, f32x4 (&o)[8],
                                            float &m, float &l) {
  // each wave dumps its accumulators into its own buffers (its reads of them
  // are complete: LDS operations of one wave execute in order)
  f32x4 SMD_LDS *dump = (f32x4 SMD_LDS *)&sm.buf[wave][0];
#pragma unroll
  for (int d = 0; d < 32; ++d) dump[d * 64 + L.lane] = st.acc[d];
  const float l_row = group_sum(st.l_run);
  if (L.g == 0) {
    sm.stat_m[wave][L.j] = st.m_ref;
    sm.stat_l[wave][L.j] = l_row;
  }
  __syncthreads();
  float mw[kWaves], lw[kWaves];
  m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = sm.stat_m[w][L.j];
    lw[w] = sm.stat_l[w][L.j];
    m = fmaxf(m, mw[w]);
  }
  l = 0.f;
  float sc[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    sc[w] = mw[w] == -INFINITY ? 0.f : exp2_fast(mw[w] - m);
    l += sc[w] * lw[w];
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const f32x4 SMD_LDS *src = (const f32x4 SMD_LDS *)&sm.buf[w][0];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] += sc[w] * src[(8 * wave + d) * 64 + L.lane];
  }
}

// Final bf16 output of one query row with the sink folded in:
// out = O / (l + e^(sink - m)), lse = m + ln(l + e^(sink - m)) (natural log).
// dst points at dim 128*wave + 4g of the row; the lse is written when lse_dst
// is non-null.
__device__ __forceinline__ void write_direct(const f32x4 (&o)[8], float m, float l, float sink_ln, uint16_t *dst,
                                             float *lse_dst) {
  const float sink2 = sink_ln * kLog2e;
  const float mf = fmaxf(m, sink2);
  float inv = 0.f, lse_v = -INFINITY;
  if (mf != -INFINITY) {
    const float e = exp2_fast(m - mf);
    const float z = l * e + exp2_fast(sink2 - mf);
    inv = e / z;
    lse_v = (mf + __log2f(z)) * kLn2;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    u32x2 v;
    v[0] = (uint32_t)f32_to_bf16_rne(o[d][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[d][1] * inv) << 16);
    v[1] = (uint32_t)f32_to_bf16_rne(o[d][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[d][3] * inv) << 16);
    *(u32x2 *)(dst + 16 * d) = v;
  }
  if (lse_dst != nullptr) *lse_dst = lse_v;
}

// FP32 partial of one query row (no sink): o = O / l, lse = m + ln l; an empty
// range gives o = 0, lse = -inf.  dst as in write_direct.
__device__ __forceinline__ void write_partial(const f32x4 (&o)[8], float m, float l, float *dst, float *lse_dst) {
  float inv = 0.f, lse_v = -INFINITY;
  if (l > 0.f) {
    inv = 1.f / l;
    lse_v = (m + __log2f(l)) * kLn2;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) *(f32x4 *)(dst + 16 * d) = o[d] * inv;
  if (lse_dst != nullptr) *lse_dst = lse_v;
}

}  // namespace ks
}  // namespace smd
