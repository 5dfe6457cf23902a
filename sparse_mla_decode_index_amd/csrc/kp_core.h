// Device core of the dim-split sparse MLA decode (gfx950), for workloads that
// fill the GPU with blocks of 32 query rows.
//
// What is computed is the same as in ks8_core.h (vLLM page "[ROCm][DSV4][Perf]
// Optimize Triton sparse-MLA decode on gfx950", Design): per query row a
// 512-wide QK dot with every selected latent row, an online softmax with a
// per-head sink, and a PV product over the same 512-wide rows.
//
// A workgroup of 8 waves owns 32 query rows (two blocks of 16) and a range of
// index positions.  Waves 2k and 2k+1 form pair k, which takes half-tiles k,
// k+4, ... of 16 positions (the two waves of a pair run on different SIMDs,
// and the two waves of a SIMD belong to different pairs).  Wave h = w & 1 of
// a pair owns the 256 dims [256h, 256h+256) of every row: it gathers only those dims (512 bytes of a
// bf16 row; 256 e4m3 bytes + 4 codes, or 192 e4m3 bytes + 3 codes + the 64
// RoPE dims of an fp8 row), stores them to its own 8 KiB LDS buffer, computes
// the partial scores of both query blocks over its dims (one K operand read
// feeds two MFMAs), and accumulates O for its dims.  The two halves of a pair
// add their partial scores through LDS once per half-tile, ordered by a step
// flag per wave rather than a workgroup barrier, so pairs drift apart and one
// wave's LDS phase overlaps its SIMD neighbour's MFMA phase (a + b is the same
// float in both waves, so both run the same softmax).  Per unit of work this moves about a third less through LDS
// than the 16-row layout of ks8_core.h, where LDS bandwidth binds.
//
// LDS: Q^T 32 KiB + 8 x 8 KiB buffers + 32 KiB of score exchange = 128 KiB,
// reused at the end for the merge of the four pairs' states.
#pragma once

#include "ks_core.h"

namespace smd {
namespace kp {

using ks::bf16x4;
using ks::bf16x8;
using ks::f32x4;
using ks::Lane;
using ks::u32x4;

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kPairs = 4;         // KV lanes of a workgroup
constexpr int kRows = 32;         // query rows of a workgroup
constexpr int kHalfRow = 512;     // one row's 256 dims in LDS (bf16)
constexpr int kBufBytes = 16 * kHalfRow;

// Row formats (the same as ks8_core.h).
enum Fmt { kBf16Packed = 0, kBf16Split = 1, kFp8 = 2 };

struct Smem {
  union {
    struct {
      uint8_t q[2 * 2 * 8 * 64 * 16];  // Q^T: [half][block][k-step][lane] x 16 B
      uint8_t buf[8][kBufBytes];       // one half-row buffer per wave
      f32x4 xs[2][8][2][64];           // partial scores [step parity][wave][block][lane]
    } m;
    f32x4 dump[4][32][64];  // merge: four wave states of 32 KiB
  } u;
  float stat[4][4][64];  // merge: [slot][m0, m1, l0, l1][lane]
  int flag[8];           // per wave: score-exchange steps published
};

// Per-lane constants of the half-row layout.  Row r of a buffer holds the
// 32 chunks (16 B, 8 dims) of the wave's half; chunk c sits at c ^ swz(r).
struct PLane {
  int wb[4];  // QK A-operand offsets (chunk group 0..3 of a 128-byte column)
  int pv[8];  // transposed-read offsets for dim block d & 7
};

__device__ __forceinline__ PLane make_plane(const Lane &L) {
  PLane P;
  const int sw = ks::swz(L.r);
  // A operand of k-step ks (dims 32ks + 8q of the half): chunk 4ks + q =
  // 16*(ks >> 2) + (4*(ks & 3) + q); the XOR stays in the low 4 bits.
#pragma unroll
  for (int i = 0; i < 4; ++i) P.wb[i] = L.r * kHalfRow + (((4 * i + L.q) ^ sw) << 4);
  // PV: lanes 4t+u of group g read row 4g+t, dims 16d + 4u..+4 of the half =
  // chunk 2d + (u >> 1), byte 8(u & 1); chunk 2d = 16*(d >> 3) + 2(d & 7).
  const int t = L.j >> 2, u = L.j & 3;
  const int tr = 4 * L.g + t;
  const int ftr = ks::swz(tr);
#pragma unroll
  for (int d = 0; d < 8; ++d) P.pv[d] = tr * kHalfRow + (((2 * d + (u >> 1)) ^ ftr) << 4) + ((u & 1) << 3);
  return P;
}

// Gathered data of one half-tile, bf16: v[i] = chunk (lane & 31) of the
// wave's half of row 2i + (lane >> 5).
struct HalfB {
  u32x4 v[8];
};
// fp8, half 0: n[t] = e4m3 bytes 64t + 16s of row lane / 4 (s = lane % 4,
// code block t = 0..3), code = codes 0..3.  Half 1: n[t] = bytes 256 + 64t +
// 16s (blocks 4..6, n[3] unused), r[u] = RoPE bytes 64u + 16s, code = codes
// 4..7.
struct HalfF {
  u32x4 n[4];
  u32x4 r[2];
  uint32_t code;
};

template <int FMT>
struct Gathered {
  typedef HalfB type;
};
template <>
struct Gathered<kFp8> {
  typedef HalfF type;
};

// The half-tile row whose index this lane holds (and, for fp8, gathers).
template <int FMT>
__device__ __forceinline__ int row_of(const Lane &L) {
  return FMT == kFp8 ? (L.lane >> 2) : L.r;
}

// Loads of one half-tile for dims half h; idx / valid are those of row
// row_of<FMT>(lane).  Masked rows read the zero row.
template <int FMT>
__device__ __forceinline__ void issue(const DecodeArgs &a, uint32_t idx, bool valid, bool second, int h,
                                      const Lane &L, typename Gathered<FMT>::type &g) {
  typedef const uint8_t SMD_GLOBAL *gptr;
  if constexpr (FMT == kFp8) {
    const uint8_t *z = ks::g_zero_row;
    const gptr pn =
        (gptr)(uintptr_t)(valid ? ks::nope_base(a, second) + (uint64_t)idx * (uint64_t)a.nope_stride_b : z);
    const gptr pc =
        (gptr)(uintptr_t)(valid ? ks::scale_base(a, second) + (uint64_t)idx * (uint64_t)a.scale_stride_b : z);
    const int off = 16 * (L.lane & 3);
    if (h == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) g.n[t] = *(const u32x4 SMD_GLOBAL *)(pn + off + 64 * t);
      g.code = *(const uint32_t SMD_GLOBAL *)pc;
    } else {
      const gptr pr =
          (gptr)(uintptr_t)(valid ? ks::rope_base(a, second) + (uint64_t)idx * (uint64_t)a.rope_stride_b : z);
#pragma unroll
      for (int t = 0; t < 3; ++t) g.n[t] = *(const u32x4 SMD_GLOBAL *)(pn + 256 + off + 64 * t);
#pragma unroll
      for (int u = 0; u < 2; ++u) g.r[u] = *(const u32x4 SMD_GLOBAL *)(pr + off + 64 * u);
      g.code = *(const uint32_t SMD_GLOBAL *)(pc + 4);
    }
  } else {
    constexpr bool PACKED = FMT == kBf16Packed;
    const uint64_t naddr = ks::row_address<PACKED>(a, idx, valid, second);
    uint64_t raddr = 0;
    if constexpr (!PACKED)
      raddr = valid ? (uint64_t)(uintptr_t)(ks::rope_base(a, second) + (uint64_t)idx * (uint64_t)a.rope_stride_b)
                    : (uint64_t)(uintptr_t)ks::g_zero_row + 2 * kNope;
    const int c = L.lane & 31;
    const bool hi = L.lane >= 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // rows 2i (lanes 0..31) and 2i+1 (lanes 32..63): their bases from lanes 2i, 2i+1
      const uint64_t b0 = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(naddr >> 32), 2 * i) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((uint32_t)naddr, 2 * i);
      const uint64_t b1 = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(naddr >> 32), 2 * i + 1) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((uint32_t)naddr, 2 * i + 1);
      const uint64_t nb = hi ? b1 : b0;
      if constexpr (PACKED) {
        g.v[i] = *(const u32x4 SMD_GLOBAL *)((gptr)(uintptr_t)nb + kHalfRow * h + 16 * c);
      } else {
        const uint64_t r0 = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(raddr >> 32), 2 * i) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((uint32_t)raddr, 2 * i);
        const uint64_t r1 = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(raddr >> 32), 2 * i + 1) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((uint32_t)raddr, 2 * i + 1);
        const uint64_t rb = hi ? r1 : r0;
        // half 1, chunks 24..31 are the RoPE dims 448..511
        const gptr p = (h == 1 && c >= 24) ? (gptr)(uintptr_t)rb + 16 * (c - 24)
                                           : (gptr)(uintptr_t)nb + kHalfRow * h + 16 * c;
        g.v[i] = *(const u32x4 SMD_GLOBAL *)p;
      }
    }
  }
}

// Gathered rows into the wave's buffer (fp8 dequantised on the way: e4m3 x
// 2^(code-127) is exact in bf16).
__device__ __forceinline__ void store(const HalfB &g, int h, uint8_t SMD_LDS *buf, const Lane &L) {
  const int c = L.lane & 31;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 2 * i + (L.lane >> 5);
    *(u32x4 SMD_LDS *)(buf + r * kHalfRow + ((c ^ ks::swz(r)) << 4)) = g.v[i];
  }
}

__device__ __forceinline__ void store(const HalfF &g, int h, uint8_t SMD_LDS *buf, const Lane &L) {
  const int r = L.lane >> 2, s = L.lane & 3;
  const int sw = ks::swz(r);
  const int e = r & 1;  // odd rows store their odd chunk first (fewer bank conflicts)
  uint8_t SMD_LDS *row = buf + r * kHalfRow;
  const int nt = h == 0 ? 4 : 3;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t >= nt) break;
    const float sc = ks::ue8m0_scale((g.code >> (8 * t)) & 0xffu);
    u32x4 c[2];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      c[w >> 1][2 * (w & 1)] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)g.n[t][w], sc, false));
      c[w >> 1][2 * (w & 1) + 1] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)g.n[t][w], sc, true));
    }
    const int c0 = 8 * t + 2 * s;
    *(u32x4 SMD_LDS *)(row + (((c0 + e) ^ sw) << 4)) = e ? c[1] : c[0];
    *(u32x4 SMD_LDS *)(row + (((c0 + 1 - e) ^ sw) << 4)) = e ? c[0] : c[1];
  }
  if (h == 1) {
#pragma unroll
    for (int u = 0; u < 2; ++u) *(u32x4 SMD_LDS *)(row + (((24 + 4 * u + s) ^ sw) << 4)) = g.r[u];
  }
}

// Q^T of the 32 rows into LDS: B operand of (half h, block qb, k-step ks) for
// lane l = dims 256h + 32ks + 8(l/16) .. +8 of query row 16qb + l % 16.  Wave w
// stores the four (h, qb, ks) of index 4w .. 4w+3.
__device__ __forceinline__ void stage_q(const DecodeArgs &a, const int64_t (&qrow)[2], int wave, const Lane &L,
                                        Smem &sm) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = 4 * wave + i;  // = (h * 2 + qb) * 8 + ks
    const int ks = x & 7, qb = (x >> 3) & 1, h = x >> 4;
    const int dim = 256 * h + 32 * ks + 8 * L.q;
    const uint16_t *src = dim < kNope ? a.q_nope + qrow[qb] * kNope + dim : a.q_rope + qrow[qb] * kRope + (dim - kNope);
    *(u32x4 SMD_LDS *)((uint8_t SMD_LDS *)sm.u.m.q + (x * 64 + L.lane) * 16) = *(const u32x4 *)src;
  }
}

// Per-wave state: O^T of the wave's 256 dims for both query blocks,
// acc[2d + qb][i] = sum over rows of 2^(x - m_ref[qb]) V[row][256h + 16d + 4g + i]
// for query row j of block qb.
struct State {
  f32x4 acc[32];
  float m_ref[2];
  float l_run[2];
  bool overflow;
  int step;  // score exchanges done (across passes; the same in both waves of a pair)
};

// Partial scores of both blocks over the wave's dims, from the wave's buffer
// (A = K) and the shared Q^T (B).
__device__ __forceinline__ void qk(const uint8_t SMD_LDS *qh, const uint8_t SMD_LDS *buf, const PLane &P,
                                   const Lane &L, f32x4 &s0, f32x4 &s1) {
  s0 = f32x4{0.f, 0.f, 0.f, 0.f};
  s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 k = *(const bf16x8 SMD_LDS *)(buf + P.wb[ks & 3] + 256 * (ks >> 2));
    const bf16x8 q0 = *(const bf16x8 SMD_LDS *)(qh + (ks * 64 + L.lane) * 16);
    const bf16x8 q1 = *(const bf16x8 SMD_LDS *)(qh + ((8 + ks) * 64 + L.lane) * 16);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, q0, s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, q1, s1, 0, 0, 0);
  }
}

// PV of one half-tile over the wave's dims for both blocks.
template <bool P_HILO>
__device__ __forceinline__ void pv(const uint8_t SMD_LDS *buf, const bf16x4 (&p)[2], const bf16x4 (&pl)[2],
                                   const PLane &P, State &st) {
  const s16x4 p0 = __builtin_bit_cast(s16x4, p[0]), p1 = __builtin_bit_cast(s16x4, p[1]);
  s16x4 l0, l1;
  if constexpr (P_HILO) {
    l0 = __builtin_bit_cast(s16x4, pl[0]);
    l1 = __builtin_bit_cast(s16x4, pl[1]);
  }
  constexpr int kPre = 4;
  bf16x4 v[kPre];
  auto load = [&](int d) {
    v[d % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(buf + P.pv[d & 7] + 256 * (d >> 3)));
  };
#pragma unroll
  for (int d = 0; d < kPre; ++d) load(d);
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    const s16x4 va = __builtin_bit_cast(s16x4, v[d % kPre]);
    if (d + kPre < 16) load(d + kPre);
    st.acc[2 * d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, p0, st.acc[2 * d], 0, 0, 0);
    st.acc[2 * d + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, p1, st.acc[2 * d + 1], 0, 0, 0);
    if constexpr (P_HILO) {
      st.acc[2 * d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, l0, st.acc[2 * d], 0, 0, 0);
      st.acc[2 * d + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, l1, st.acc[2 * d + 1], 0, 0, 0);
    }
  }
}

// The gather pipeline of one wave (as in ks8_core.h).
template <int FMT>
struct Pipe {
  typename Gathered<FMT>::type g;
  int32_t i_next;  // index of row row_of<FMT>(L) of the next-but-one half-tile
  uint32_t vb;
};

// Half-tile i of pair k covers positions p0 + 16*(k + 4i) + 0..15.
template <int FMT>
__device__ __forceinline__ int pos_of(int p0, int k, int i, const Lane &L) {
  return p0 + 16 * (k + kPairs * i) + row_of<FMT>(L);
}

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

// Start the pipeline: indices of half-tiles 0 and 1, rows of half-tile 0.
template <int FMT, class SRC>
__device__ __forceinline__ void prime(const DecodeArgs &a, const SRC &src, int p0, int p1, int k, int h,
                                      const Lane &L, Pipe<FMT> &pp) {
  const int q0 = min(pos_of<FMT>(p0, k, 0, L), p1 - 1);
  const int32_t i0 = src.at(q0);
  pp.i_next = src.at(min(pos_of<FMT>(p0, k, 1, L), p1 - 1));
  const bool v0 = pos_of<FMT>(p0, k, 0, L) < p1 && src.row_ok(a, q0, i0);
  issue<FMT>(a, (uint32_t)i0, v0, src.in_second(q0), h, L, pp.g);
  pp.vb = row_bits<FMT>(v0);
}

// Publish this wave's step count (after its score partials) and wait for the
// partner's.  Both waves of a pair run the same number of exchanges, so the
// wait always ends; the bound only turns a broken invariant into wrong numbers
// instead of a hung GPU.
__device__ __forceinline__ void exchange_sync(Smem &sm, int wave, int step, const Lane &L) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the partials are in LDS
  if (L.lane == 0) *(volatile int SMD_LDS *)&sm.flag[wave] = step;
  const volatile int SMD_LDS *f = (const volatile int SMD_LDS *)&sm.flag[wave ^ 1];
  for (int it = 0; it < (1 << 20); ++it) {
    if (*f >= step) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");  // the partner's partials are read after the flag
}

// The workgroup's sweep: every wave runs nk steps (the most any pair has), a
// pair past its last half-tile reads masked rows.  Exchange slots alternate
// with the step count; a wave rewrites a slot two exchanges later, by which
// time its partner, having published the exchange in between, has read it.
template <int FMT, bool P_HILO, int PASS, class SRC>
__device__ __forceinline__ void sweep(const DecodeArgs &a, const SRC &src, int p0, int p1, int nk, int wave,
                                      const Lane &L, const PLane &P, Smem &sm, State &st, Pipe<FMT> &pp) {
  const int k = wave >> 1, h = wave & 1;
  const uint8_t SMD_LDS *qh = (const uint8_t SMD_LDS *)sm.u.m.q + h * (16 * 64 * 16);
  uint8_t SMD_LDS *buf = (uint8_t SMD_LDS *)sm.u.m.buf[wave];
  for (int i = 0; i < nk; ++i) {
    store(pp.g, h, buf, L);
    const int qn = min(pos_of<FMT>(p0, k, i + 1, L), p1 - 1);
    const bool vn = pos_of<FMT>(p0, k, i + 1, L) < p1 && src.row_ok(a, qn, pp.i_next);
    issue<FMT>(a, (uint32_t)pp.i_next, vn, src.in_second(qn), h, L, pp.g);
    pp.i_next = src.at(min(pos_of<FMT>(p0, k, i + 2, L), p1 - 1));
    const uint32_t vb = pp.vb;
    pp.vb = row_bits<FMT>(vn);
    f32x4 s0, s1;
    qk(qh, buf, P, L, s0, s1);
    const int par = st.step & 1;
    f32x4 SMD_LDS *xw = (f32x4 SMD_LDS *)&sm.u.m.xs[par][wave][0][0];
    const f32x4 SMD_LDS *xr = (const f32x4 SMD_LDS *)&sm.u.m.xs[par][wave ^ 1][0][0];
    xw[L.lane] = s0;
    xw[64 + L.lane] = s1;
    st.step += 1;
    exchange_sync(sm, wave, st.step, L);
    s0 += xr[L.lane];
    s1 += xr[64 + L.lane];
    bf16x4 p[2], pl[2];
    ks::softmax_step<PASS, P_HILO>(s0, vb, a.scale_log2, L, st.m_ref[0], st.l_run[0], st.overflow, p[0], pl[0]);
    ks::softmax_step<PASS, P_HILO>(s1, vb, a.scale_log2, L, st.m_ref[1], st.l_run[1], st.overflow, p[1], pl[1]);
    if constexpr (PASS != ks::kPassMax) pv<P_HILO>(buf, p, pl, P, st);
  }
}

__device__ __forceinline__ void reset(State &st) {
#pragma unroll
  for (int d = 0; d < 32; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_ref[0] = st.m_ref[1] = -INFINITY;
  st.l_run[0] = st.l_run[1] = 0.f;
}

// The workgroup's attention over [p0, p1): the main sweep, and the exact-max
// redo of every wave when any score overflowed its reference (the decision is
// workgroup-wide, so every wave runs the same barriers).
template <int FMT, bool P_HILO, class SRC>
__device__ __forceinline__ void attend(const DecodeArgs &a, const SRC &src, int p0, int p1, int wave,
                                       const Lane &L, const PLane &P, Smem &sm, State &st, Pipe<FMT> &pp) {
  const int nh = (p1 - p0 + 15) / 16;
  const int nk = (nh + kPairs - 1) / kPairs;
  const int k = wave >> 1, h = wave & 1;
  reset(st);
  st.overflow = false;
  st.step = 0;
  sweep<FMT, P_HILO, ks::kPassMain>(a, src, p0, p1, nk, wave, L, P, sm, st, pp);
  if (__syncthreads_or(st.overflow)) {
    // Rare: a score ran far above its row's first-half-tile max.  Redo with
    // the exact max (a scores-only sweep) as the reference.
    reset(st);
    prime<FMT>(a, src, p0, p1, k, h, L, pp);
    sweep<FMT, P_HILO, ks::kPassMax>(a, src, p0, p1, nk, wave, L, P, sm, st, pp);
    prime<FMT>(a, src, p0, p1, k, h, L, pp);
    sweep<FMT, P_HILO, ks::kPassFixed>(a, src, p0, p1, nk, wave, L, P, sm, st, pp);
  }
}

// Merge of the four pairs' states, per dims half: pairs 2, 3 hand over to
// pairs 0, 1, then pair 1 to pair 0.  Waves 0 and 1 end with the merged state
// of dims half 0 and 1 (O in acc, reference max m[qb], this lane's share of
// the sum in l_run[qb]); returns false on the other waves.
__device__ __forceinline__ bool merge_pairs(Smem &sm, int wave, const Lane &L, State &st) {
  const int k = wave >> 1, h = wave & 1;
  __syncthreads();  // every wave is done with the buffers and the exchange
  auto give = [&](int slot) {
#pragma unroll
    for (int d = 0; d < 32; ++d) sm.u.dump[slot][d][L.lane] = st.acc[d];
    sm.stat[slot][0][L.lane] = st.m_ref[0];
    sm.stat[slot][1][L.lane] = st.m_ref[1];
    sm.stat[slot][2][L.lane] = st.l_run[0];
    sm.stat[slot][3][L.lane] = st.l_run[1];
  };
  auto take = [&](int slot) {
    float sa[2], sb[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mb = sm.stat[slot][qb][L.lane], lb = sm.stat[slot][2 + qb][L.lane];
      const float mm = fmaxf(st.m_ref[qb], mb);
      sa[qb] = st.m_ref[qb] == -INFINITY ? 0.f : ks::exp2_fast(st.m_ref[qb] - mm);
      sb[qb] = mb == -INFINITY ? 0.f : ks::exp2_fast(mb - mm);
      st.m_ref[qb] = mm;
      st.l_run[qb] = st.l_run[qb] * sa[qb] + lb * sb[qb];
    }
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[d] = st.acc[d] * sa[d & 1] + sm.u.dump[slot][d][L.lane] * sb[d & 1];
  };
  if (k >= 2) give(2 * (k - 2) + h);
  __syncthreads();
  if (k < 2) take(2 * k + h);
  __syncthreads();
  if (k == 1) give(h);
  __syncthreads();
  if (k != 0) return false;
  take(h);
  return true;
}

}  // namespace kp
}  // namespace smd
