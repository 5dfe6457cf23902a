// Wide waves of the sparse MLA decode (gfx950): each of a workgroup's 4 waves
// owns 32 query rows and all 512 dims, so one gathered 32-row KV tile serves
// 128 query rows.  Both contractions run on v_mfma_f32_32x32x16_bf16, the
// bf16 shape that issues at the highest rate on gfx950 with one wave per SIMD
// (about 2.4x the rate of 16x16x32 in a back-to-back measurement).
//
// Per 32-row tile and wave:
//   QK       S^T[32 kv x 32 q] = K[32 x 512] . Q^T[512 x 32]: 32 k-steps of 16
//            dims.  Lane l holds
//            query row q = l mod 32 and the 16 kv rows 8b + 4u + i (b, i in
//            0..3, u = l / 32); its partner lane l ^ 32 holds the other 16.
//   softmax  a reference max per query row fixed at its first valid tile
//            (exp2 domain); a score more than 2^32 above it sends the
//            workgroup through an exact-max second pass (common.h), so the
//            accumulators are never rescaled.  Row max and sum need one
//            permlane32 swap.
//   PV       O^T[512 x 32 q] += V^T[512 x 32 kv] . P^T[32 kv x 32 q]: for each
//            block of 32 dims, two MFMAs over kv rows 0..15 and 16..31.  The
//            score registers are the B operand as they come out of QK (bf16),
//            with the contraction index k = 8u + e of MFMA h standing for kv
//            row 16h + 8(e / 4) + 4u + e mod 4; the V^T operand is read from
//            LDS in the same order by two ds_read_b64_tr_b16 of 4 rows each.
// The 16 O^T blocks of 32 x 32 fp32 fill all 256 AGPRs.  Q^T k-steps below KQ
// sit in VGPRs, the rest in the wave's own LDS region.
//
// The tile is row-major, 1 KiB per row, with the 16-byte chunks of row r
// permuted by an XOR of swz32(r): the QK reads (one chunk column of rows
// 0..15 per 16 lanes) and the transposed reads (rows 4k..4k+3 x 64 bytes per
// 32 lanes) touch distinct banks.
//
// Two walks over a range's tiles:
//   - bf16 pools: rows staged through one VGPR set, software-pipelined: the
//     rows of tile t+1 are stored to the second bf16 tile between the QK
//     MFMAs of tile t and the loads of tile t+2 go out right after them;
//   - fp8 pools: direct-to-LDS loads (global_load_lds) fill a ring of three
//     raw tiles with no VGPRs held, so tiles t+1..t+3 are in flight while t is
//     computed; each wave dequantises its own rows of the next raw tile into
//     the shared bf16 tile (e4m3 x 2^(code-127), exact in bf16).  The index
//     blocks arrive the same way, so no vector load's wait drains the ring.
#pragma once

#include "decode_core.h"
#include "quant.h"

#include <type_traits>

namespace smd {

// The lane id from an opaque asm: offsets derived from it are recomputed
// where they are used instead of being hoisted out of the sequence loop (and
// spilled, each use then waiting for a scratch reload).
__device__ __forceinline__ int opaque_lane() {
  int lane;
  asm volatile(
      "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
      "v_mbcnt_hi_u32_b32 %0, -1, %0"
      : "=v"(lane));
  return lane;
}

constexpr int kWideRows = 128;     // query rows per workgroup (4 waves x 32)
constexpr int kQRegStaged = 12;    // Q^T k-steps (16 dims) in VGPRs next to a staged row set
constexpr int kQRegDma = 18;       // ... when the gather holds no VGPRs
constexpr int kQkPre = 3;          // QK: LDS reads in flight ahead of their MFMA
constexpr int kPvPre = 4;          // PV: V^T operands in flight ahead of their MFMA

// Raw fp8 rows of one tile as the direct-to-LDS loads leave them, per wave
// (rows 8w..8w+7 of the tile, local row r = 0..7): NoPE [8][32][16 B] at 0
// (logical chunks 28..31 of a row are padding), RoPE [8][8][16 B] at 4096,
// UE8M0 codes [8][8 B] at 5120, then padding, so that the slots also hold the
// four 16 KiB staging slices.  Two variants:
//   - plain (SWZ = false): chunks in order, regions 5504 bytes apart;
//     only the owning wave reads a region (its dequantisation);
//   - swizzled (SWZ = true, the fp8 QK): the 16-byte chunks of a row are
//     permuted (raw_swz_nope / raw_swz_rope) and the regions are 64 mod 256
//     bytes (16 banks) apart, so that the fp8 QK's operand reads -- one
//     chunk column of 16 rows of two neighbouring regions per 16 lanes --
//     touch all 64 banks once.  (Measured on the plain walk, which does not
//     need it, the swizzle cost 2%.)
constexpr int kRawNope = 0, kRawRope = 4096, kRawCode = 5120;
template <bool SWZ>
constexpr int raw_wave() {
  return SWZ ? 5696 : 5120 + 384;
}
template <bool SWZ>
constexpr int raw_slot() {
  return 4 * raw_wave<SWZ>();
}
static_assert(raw_wave<true>() % 256 == 64 && raw_wave<true>() >= kRawCode + 64, "raw region spacing");

// Position of logical chunk c of local row r in the swizzled layout:
// c ^ raw_swz_nope(r) (NoPE), c ^ raw_swz_rope(r) (RoPE).  NoPE rows are 512
// bytes apart (the same banks): the XOR spreads the 8 rows of a region over
// chunk columns {x, x^1, x^2, x^3, x^8 .. x^11} mod 16, and the next region,
// 4 columns further, takes the other 8.  RoPE rows are 128 bytes apart (odd
// rows 8 columns further); the XOR spreads each parity over 4 columns and
// the next region again takes the rest.
template <bool SWZ>
__device__ __forceinline__ int raw_swz_nope(int r) {
  return SWZ ? ((r & 3) | ((r >> 2) << 3)) : 0;
}
template <bool SWZ>
__device__ __forceinline__ int raw_swz_rope(int r) {
  return SWZ ? ((r >> 1) & 3) : 0;
}

// Slots of the raw ring: the plain walk reads tile t out of its slot before
// the loads of t+3 reuse it; the fp8 QK reads tile t's slot during its
// compute, so it keeps a fourth.
template <bool QF8>
constexpr int raw_slots() {
  return QF8 ? 4 : 3;
}
constexpr int kRawAhead = 3;  // tiles whose loads are in flight ahead of the one computed

template <bool FP8>
struct SmemWide;

template <>
struct SmemWide<false> {
  uint8_t tile[2][kTileBytes];                  // double-buffered bf16 tiles
  int32_t ibuf[2][kIdxBlock];                   // index blocks
  uint8_t qs[4][32 - kQRegStaged][64 * 16];     // [wave][k-step - KQ][lane]
};

// The direct-to-LDS targets (the raw ring and the index blocks) are separate
// __shared__ objects (WideDma): the compiler orders any read of a possible
// target after every load in flight (a full vmcnt wait), so those two are
// read only through inline asm with the waits issued by hand, and everything
// the MFMA path reads lives in this other object.
template <>
struct SmemWide<true> {
  uint8_t tile[1][kTileBytes];                  // the bf16 tile being computed
  uint8_t qs[4][32 - kQRegDma][64 * 16];
};

struct WideDma {
  uint8_t SMD_LDS *raw;   // [raw_slots][raw_slot]: ring of raw fp8 tiles
  int32_t SMD_LDS *ibuf;  // [2][kIdxBlock]: index blocks
};

// fp8 pools walk on the direct-to-LDS ring, bf16 pools on the staged walk.
// (The staged walk also takes fp8 rows; on the ragged MTP4 fp8 workload it ran
// 6% slower than the ring: 381 against 359 us.)
template <bool FP8>
constexpr bool wide_ring() {
  return FP8;
}

template <bool RING>
constexpr int wide_qreg() {
  return RING ? kQRegDma : kQRegStaged;
}

// Softmax state and O^T of a wide wave's 32 query rows.
struct WideState {
  f32x16 acc[16];  // acc[D][e] = sum_j 2^(x_j - m_ref) V[j][32D + 8(e/4) + 4u + e%4], query row q
  float m_ref;     // reference max (log2 domain), the same in lanes l and l ^ 32
  float l_run;     // this lane's share of sum_j 2^(x_j - m_ref)
  bool overflow;   // some score exceeded m_ref + kRefSlackLog2 (this lane)
};

// Per-lane LDS byte offsets of the 32x32 operands in a tile:
//   qk[m]: QK A operand of k-steps ks with ks mod 8 = m: row l mod 32, logical
//          chunk 2m + l / 32 (k-step ks adds 256 * (ks / 8));
//   pv[4a + dd]: transposed read of 4 rows for dim blocks D with D mod 4 = dd:
//          lane 4t + q of 16-lane group G supplies row 8a + 4(G / 2) + t and
//          dims 32D + 16(G mod 2) + 4q, so lane j of group G receives dim
//          32D + 16(G mod 2) + j of those 4 rows (block D adds 256 * (D / 4),
//          kv half h adds 16 rows).
struct WideLanes {
  int qk[8];
  int pv[8];
};

__device__ __forceinline__ WideLanes wide_lanes(int lane) {
  WideLanes L;
  const int r = lane & 31, u = lane >> 5;
#pragma unroll
  for (int m = 0; m < 8; ++m) L.qk[m] = r * kLdsRow + (((2 * m + u) ^ swz32(r)) << 4);
  const int G = lane >> 4, t = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      const int row = 8 * a + 4 * (G >> 1) + t;  // swz32 of row + 16h equals swz32(row)
      const int c = 4 * dd + 2 * (G & 1) + (q >> 1);
      L.pv[4 * a + dd] = row * kLdsRow + ((c ^ swz32(row)) << 4) + 8 * (q & 1);
    }
  }
  return L;
}

// QK, softmax weights and PV of one 32-row tile for a wide wave.  PASS as in
// decode_core.h: kPassMain fixes the reference max at the row's first valid
// tile and flags overflows, kPassMax only finds the exact max, kPassFixed
// accumulates against it.
struct NoWork {
  __device__ __forceinline__ void operator()(int) const {}
};

// mid(i), i = 0 .. kMidSlots-1, runs between the QK MFMAs (after k-step
// 4i + 1) and post(0) right after the last of them: work of the next tile
// (its LDS stores, the loads of the one after) issued while the matrix core
// is busy.  It must not touch `tile`.
constexpr int kMidSlots = 8;

// Softmax weights of a tile's scores for a wide wave: score e of this lane is
// kv row 8(e/4) + 4u + e%4.  Returns false in the max-only pass (nothing to
// accumulate).  pb (and pl with P_HILO) become PV's B operands.
template <int PASS, bool P_HILO>
__device__ __forceinline__ bool softmax_wide(f32x16 &s, uint32_t vbits, int lane, float scale_log2, WideState &w,
                                             bf16x8 (&pb)[2], bf16x8 (&pl)[2]) {
  // A tile whose 32 rows are all valid (wave-uniform) skips the masking; the
  // max then comes from the raw scores (scale_log2 > 0 keeps the order).
  float tmax;
  const bool all_valid = vbits == 0xffffffffu && scale_log2 > 0.f;
  if (all_valid) {
    tmax = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, s[e]);
    tmax *= scale_log2;
  } else {
    const uint32_t vb = vbits >> (4 * (lane >> 5));
#pragma unroll
    for (int e = 0; e < 16; ++e)
      s[e] = ((vb >> (8 * (e >> 2) + (e & 3))) & 1) ? s[e] * scale_log2 : -INFINITY;
    tmax = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, s[e]);
  }
  tmax = half_max(tmax);
  if constexpr (PASS == kPassMax) {
    w.m_ref = fmaxf(w.m_ref, tmax);
    return false;
  }
  if constexpr (PASS == kPassMain) {
    if (w.m_ref == -INFINITY) w.m_ref = tmax;  // nothing accumulated yet for this row
    w.overflow |= tmax > w.m_ref + kRefSlackLog2;
  }
  const float m_use = (w.m_ref == -INFINITY) ? 0.f : w.m_ref;
  // p = 2^(x - m_use) with x = s * scale_log2 (unmasked) or s (masked, already scaled)
  const float mul = all_valid ? scale_log2 : 1.f;
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float p = exp2_fast(__builtin_fmaf(s[e], mul, -m_use));
    psum += p;
    pb[e >> 3][e & 7] = (__bf16)p;
    // P_HILO: p = hi + lo with both parts bf16, so the PV product carries
    // about 16 significant bits of p instead of 8 (FP32-partial precision).
    if constexpr (P_HILO) pl[e >> 3][e & 7] = (__bf16)(p - (float)pb[e >> 3][e & 7]);
  }
  w.l_run += psum;
  return true;
}

// PV of a tile for a wide wave: MFMA i = 16h + D covers dims 32D.. and kv
// rows 16h..16h+15, the V^T operand read from the bf16 tile.
template <bool P_HILO>
__device__ __forceinline__ void pv_wide(const uint8_t SMD_LDS *tile, const WideLanes &L, const bf16x8 (&pb)[2],
                                        const bf16x8 (&pl)[2], WideState &w) {
  bf16x8 va[kPvPre];
  auto pv_load = [&](int i) {
    const int h = i >> 4, D = i & 15;
    const uint8_t SMD_LDS *base = tile + 16 * kLdsRow * h + 256 * (D >> 2);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(base + L.pv[D & 3]));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(base + L.pv[4 + (D & 3)]));
    va[i % kPvPre] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
#pragma unroll
  for (int i = 0; i < kPvPre; ++i) pv_load(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const bf16x8 av = va[i % kPvPre];
    if (i + kPvPre < 32) pv_load(i + kPvPre);
    const int h = i >> 4, D = i & 15;
    w.acc[D] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[h], w.acc[D], 0, 0, 0);
    if constexpr (P_HILO) w.acc[D] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pl[h], w.acc[D], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KQ, int PASS, bool P_HILO, class Mid = NoWork, class Post = NoWork>
__device__ __forceinline__ void compute_tile_wide(const uint8_t SMD_LDS *tile, const bf16x8 (&qreg)[KQ],
                                                  const uint8_t SMD_LDS *qs, const WideLanes &L, uint32_t vbits,
                                                  int lane, float scale_log2, WideState &w, Mid mid = Mid(),
                                                  Post post = Post()) {
  // ---- QK (one accumulator chain: a second would push O out of the AGPRs)
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
  bf16x8 ka[kQkPre], ql[kQkPre];
  auto qk_load = [&](int ks) {
    ka[ks % kQkPre] = *(const bf16x8 SMD_LDS *)(tile + L.qk[ks & 7] + 256 * (ks >> 3));
    if (ks >= KQ) ql[ks % kQkPre] = *(const bf16x8 SMD_LDS *)(qs + ((ks - KQ) * 64 + lane) * 16);
  };
#pragma unroll
  for (int ks = 0; ks < kQkPre; ++ks) qk_load(ks);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) {
    const bf16x8 av = ka[ks % kQkPre];
    const bf16x8 bv = ks < KQ ? qreg[ks < KQ ? ks : 0] : ql[ks % kQkPre];
    if (ks + kQkPre < 32) qk_load(ks + kQkPre);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, s, 0, 0, 0);
    if (ks % 4 == 1) mid(ks / 4);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads kQkPre steps ahead of their MFMAs
  }
  post(0);

  bf16x8 pb[2], pl[2];
  if (softmax_wide<PASS, P_HILO>(s, vbits, lane, scale_log2, w, pb, pl)) pv_wide<P_HILO>(tile, L, pb, pl, w);
}

// Walk the range's tiles once with one staged register set (bf16 and fp8
// pools), software-pipelined by one tile.  Step t computes tile t from its
// LDS buffer; between its QK MFMAs the rows of tile t+1 (staged in registers
// since step t-1) are stored -- fp8 rows dequantised on the way -- to the
// other buffer, and right after the QK MFMAs the loads of tile t+2 are issued
// into the freed registers, so the gather, the dequantisation and the stores
// run while the matrix core is busy.  One barrier per step.  Indices come
// from the LDS index blocks as in run_split.
template <bool FP8, bool PACKED, bool P_HILO, int PASS>
__device__ __forceinline__ void run_split_wide(const DecodeArgs &a, SmemWide<false> &sm, const int32_t *row_idx,
                                               int p0, int p1, int wave, int lane,
                                               const bf16x8 (&qreg)[kQRegStaged], const WideLanes &L,
                                               WideState &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  uint8_t SMD_LDS *tile0 = (uint8_t SMD_LDS *)&sm.tile[0][0];
  int32_t SMD_LDS *ib0 = (int32_t SMD_LDS *)&sm.ibuf[0][0];
  const uint8_t SMD_LDS *qs = (const uint8_t SMD_LDS *)&sm.qs[wave][0][0];
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  Staged<FP8> sa;
  const uint8_t *zrow = g_zero_row;
  const GatherLanes gl = make_gather_lanes<kLay32>(wave, lane);
  const int blk0 = load_idx_block(row_idx, p0, p1, 0);
  __syncthreads();  // the buffers may still be read by a previous pass
  ib0[threadIdx.x] = blk0;
  __syncthreads();
  load_rows<FP8, PACKED>(a, zrow, gl, tidx(0), p0, p1, wave, lane, sa);
  store_rows<FP8, kLay32>(tile0, wave, lane, sa);
  load_rows<FP8, PACKED>(a, zrow, gl, tidx(1), p0 + kBK, p1, wave, lane, sa);
  __syncthreads();
  uint32_t v_cur = tile_valid_bits(tidx(0), p0, p1, lane, a.num_rows32);
  for (int t = 0; t < ntiles; ++t) {
    const int nb = t / kTilesPerIdxBlock + 1;  // the next index block
    const int blk = load_idx_block(row_idx, p0, p1, nb);
    uint8_t SMD_LDS *next = tile0 + ((t + 1) & 1) * kTileBytes;
    auto mid = [&](int i) {
      if (i < kStorePieces<FP8>) store_row_piece<FP8, kLay32>(next, wave, opaque_lane(), sa, i);
    };
    auto post = [&](int) { load_rows<FP8, PACKED>(a, zrow, gl, tidx(t + 2), p0 + (t + 2) * kBK, p1, wave, lane, sa); };
    compute_tile_wide<kQRegStaged, PASS, P_HILO>(tile0 + (t & 1) * kTileBytes, qreg, qs, L, v_cur, lane,
                                                 a.scale_log2, w, mid, post);
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

// Direct-to-LDS loads of this wave's 8 rows of a tile (indices at tidx) into
// its raw region `dst` (layout above): loads 0..3 bring the NoPE of rows
// 2k + (lane >> 5), load 4 the RoPE of row lane >> 3, load 5 the codes, 4
// bytes per lane (lanes 0..15: row lane / 2, half lane % 2).  Invalid rows
// and positions past p1 read the zero row, as in load_rows.
// dma_rows_fp8_part issues part `part` of them: 0 and 1 the NoPE of rows
// 0..3 and 4..7 (two loads each), 2 the RoPE and the codes; widx holds the
// wave's 8 indices.
template <bool SWZ>
__device__ __forceinline__ void dma_rows_fp8_part(const DecodeArgs &a, const uint32_t (&widx)[8], int first_pos,
                                                  int p1, int wave, int lane, uint8_t SMD_LDS *dst, int part) {
  const int rows_left = p1 - first_pos - wave * (kBK / 4);
  const uint8_t *z = g_zero_row;
  // Padding positions re-read a chunk of their own row (chunk 27; code lanes
  // 16..63 repeat lanes 0..15): the zero row is one cache line that every
  // wave would hit at once.
  if (part < 2) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int k = 2 * part + kk;
      const int r = 2 * k + (lane >> 5);
      const int c = min((lane & 31) ^ raw_swz_nope<SWZ>(r), 27);  // the logical chunk landing at position lane & 31
      // widx[2k + (lane >> 5)] with a mask, not a select: a select between two
      // elements of widx may be folded into an indexed load, which goes through
      // scratch memory
      const uint32_t idx = widx[2 * k] ^ ((widx[2 * k] ^ widx[2 * k + 1]) & (0u - (uint32_t)(lane >> 5)));
      const bool v = r < rows_left && idx < a.num_rows32;
      const uint8_t *src = v ? a.kv_nope + (uint64_t)idx * (uint64_t)a.nope_stride_b + 16 * c : z + 16 * c;
      lds_dma<16>(src, dst + kRawNope + 1024 * k);
    }
    return;
  }
  {
    const int r = lane >> 3;
    const int c = (lane & 7) ^ raw_swz_rope<SWZ>(r);
    const uint32_t idx = pick8(widx, r);
    const bool v = r < rows_left && idx < a.num_rows32;
    const uint8_t *src = (v ? a.kv_rope + (uint64_t)idx * (uint64_t)a.rope_stride_b : z) + 16 * c;
    lds_dma<16>(src, dst + kRawRope);
  }
  const int r = (lane >> 1) & 7;
  const uint32_t idx = pick8(widx, r);
  const bool v = r < rows_left && idx < a.num_rows32;
  const uint8_t *src = (v ? a.kv_scale + (uint64_t)idx * (uint64_t)a.scale_stride_b : z) + 4 * (lane & 1);
  lds_dma<4>(src, dst + kRawCode);
}

template <bool SWZ>
__device__ __forceinline__ void dma_rows_fp8(const DecodeArgs &a, const int32_t SMD_LDS *tidx, int first_pos, int p1,
                                             int wave, int lane, uint8_t SMD_LDS *dst) {
  uint32_t widx[8];
  lds_read_idx8(tidx + wave * (kBK / 4), widx);
#pragma unroll
  for (int part = 0; part < 3; ++part) dma_rows_fp8_part<SWZ>(a, widx, first_pos, p1, wave, lane, dst, part);
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
template <bool SWZ>
__device__ __forceinline__ void raw_to_staged(const uint8_t SMD_LDS *src, Staged<true> &st) {
  // The lane id comes from an opaque asm so that the lane offsets below are
  // recomputed in the loop rather than hoisted: hoisted, they get spilled,
  // and the wait for their reload would land in the loop and drain the ring.
  const int lane = opaque_lane();
  const int h = lane >> 5;
  const int c = min(lane & 31, 27);
  // logical chunk c of row 2j + h sits at position c ^ raw_swz_nope(2j + h)
  const uint32_t a0 = (uint32_t)(uintptr_t)(src + kRawNope + 512 * h);
  uint32_t an[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) an[j] = a0 + 1024 * j + 16 * (c ^ raw_swz_nope<SWZ>(2 * j + h));
  const uint32_t a2 = (uint32_t)(uintptr_t)(src + kRawCode + h * 8 + (c >> 2));
  const int rr = lane >> 3;  // RoPE: logical chunk lane & 7 of row lane >> 3
  const uint32_t a3 = (uint32_t)(uintptr_t)(src + kRawRope + 128 * rr + 16 * ((lane & 7) ^ raw_swz_rope<SWZ>(rr)));
  // the code of row 2j + h at a2 + 16 j
  static_assert(kRawCode <= 65535 - 48, "ds offsets");
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %10\n\t"
      "ds_read_b128 %2, %11\n\t"
      "ds_read_b128 %3, %12\n\t"
      "ds_read_u8 %4, %13\n\t"
      "ds_read_u8 %5, %13 offset:16\n\t"
      "ds_read_u8 %6, %13 offset:32\n\t"
      "ds_read_u8 %7, %13 offset:48\n\t"
      "ds_read_b128 %8, %14\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(st.v[0]), "=&v"(st.v[1]), "=&v"(st.v[2]), "=&v"(st.v[3]), "=&v"(st.code[0]), "=&v"(st.code[1]),
        "=&v"(st.code[2]), "=&v"(st.code[3]), "=&v"(st.rope)
      : "v"(an[0]), "v"(an[1]), "v"(an[2]), "v"(an[3]), "v"(a2), "v"(a3)
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

// LDS staging slice of one wave (32 rows x 512 bytes) for the coalesced Q^T
// loads and output stores: byte c*16 .. c*16+15 of row q sits at chunk
// (c ^ q) mod 32 of the row, so the row-wise 16-byte accesses (one or two
// rows per instruction) and the fragment-wise ones (32 rows, one chunk
// column) both touch distinct banks.
constexpr int kStageRow = 512;
constexpr int kStageWave = 32 * kStageRow;  // 16 KiB
__device__ __forceinline__ int stage_off(int q, int c) { return q * kStageRow + (((c ^ q) & 31) << 4); }

// The staging slice of wave `wave`: a quarter of the double-buffered bf16
// tiles (bf16 pools) or of the raw ring (fp8 pools), both idle between a
// range's walk and the next one.
template <bool RING>
__device__ __forceinline__ uint8_t SMD_LDS *wide_stage(SmemWide<RING> &sm, const WideDma &dm, int wave) {
  if constexpr (RING) {
    static_assert(raw_slots<false>() * raw_slot<false>() >= 4 * kStageWave, "staging slices fit the raw ring");
    return dm.raw + wave * kStageWave;
  } else {
    static_assert(sizeof(sm.tile) >= 4 * kStageWave, "staging slices fit the tiles");
    return (uint8_t SMD_LDS *)&sm.tile[0][0] + wave * kStageWave;
  }
}

// Q^T of the wave's 32 query rows as QK B operands (k-step ks of lane l holds
// dims 16ks + 8(l / 32) .. +8 of row qbase + l mod 32); k-steps below KQ go to
// VGPRs, the rest to the wave's qs region.  The wave's rows are consecutive
// rows qbase .. qbase + 31 of q_nope / q_rope, so they are read row-wise (two
// rows of 512 bytes per load instruction) into the staging slice in two
// halves of 256 dims, then picked up fragment-wise.  The caller has made the
// slice free (a barrier after the last use of the tiles or the ring).
template <int KQ>
__device__ __forceinline__ void load_q_wide(const DecodeArgs &a, int64_t qbase, int, uint8_t SMD_LDS *stage,
                                            uint8_t SMD_LDS *qs, bf16x8 (&qreg)[KQ]) {
  const int lane = opaque_lane();
  const int c = lane & 31, hr = lane >> 5;
  // both halves' loads go out before the first LDS store: one round trip
  u32x4 v[2][16];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {  // rows 2k + hr, 16-byte chunk c of this half
      const int64_t row = qbase + 2 * k + hr;
      const uint16_t *src;
      if (half == 0)
        src = a.q_nope + row * kNope + 8 * c;
      else
        src = c < 24 ? a.q_nope + row * kNope + 256 + 8 * c : a.q_rope + row * kRope + 8 * (c - 24);
      v[half][k] = *(const u32x4 *)src;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int k = 0; k < 16; ++k) *(u32x4 SMD_LDS *)(stage + stage_off(2 * k + hr, c)) = v[half][k];
    // fragments: k-step ks = 16 half + j reads chunk 2j + hr of row c
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ks = 16 * half + j;
      const bf16x8 f = *(const bf16x8 SMD_LDS *)(stage + stage_off(c, 2 * j + hr));
      if (ks < KQ)
        qreg[ks < KQ ? ks : 0] = f;
      else
        *(bf16x8 SMD_LDS *)(qs + ((ks - KQ) * 64 + lane) * 16) = f;
    }
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
template <bool P_HILO, int PASS>
__device__ __forceinline__ void run_split_wide_dma(const DecodeArgs &a, SmemWide<true> &sm, const WideDma &dm,
                                                   const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                   const bf16x8 (&qreg)[kQRegDma], const WideLanes &L,
                                                   WideState &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  uint8_t SMD_LDS *tile = (uint8_t SMD_LDS *)&sm.tile[0][0];
  uint8_t SMD_LDS *raw = dm.raw;
  int32_t SMD_LDS *ib0 = dm.ibuf;
  const uint8_t SMD_LDS *qs = (const uint8_t SMD_LDS *)&sm.qs[wave][0][0];
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  constexpr int kSlots = raw_slots<false>();
  auto slot = [&](int k) { return raw + (k % kSlots) * raw_slot<false>() + wave * raw_wave<false>(); };
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
  for (int k = 0; k < kRawAhead; ++k) dma_rows_fp8<false>(a, tidx(k), p0 + k * kBK, p1, wave, lane, slot(k));
  for (int t = 0; t < ntiles; ++t) {
    wait_vm<6 * (kRawAhead - 1)>();
    Staged<true> st;
    raw_to_staged<false>(slot(t), st);
    const uint32_t v_cur = tile_valid_bits_dma(tidx(t), p0 + t * kBK, p1, lane, a.num_rows32);
    barrier_lds();  // A (this wave's raw reads of slot t % 3 are done too)
    dma_rows_fp8<false>(a, tidx(t + kRawAhead), p0 + (t + kRawAhead) * kBK, p1, wave, lane, slot(t + kRawAhead));
    if (t % kTilesPerIdxBlock == 0) {
      const int nb = t / kTilesPerIdxBlock + 1;
      dma_idx_block(row_idx, p0, p1, nb, wave, lane, ib0 + (nb & 1) * kIdxBlock);
    }
    store_rows<true, kLay32>(tile, wave, opaque_lane(), st);  // row offsets recomputed, not kept
    barrier_lds();  // B
    compute_tile_wide<kQRegDma, PASS, P_HILO>(tile, qreg, qs, L, v_cur, lane, a.scale_log2, w);
  }
  wait_vm<0>();  // no load may land in LDS after the walk
}

// bf16 pools on a direct-to-LDS ring (the split-KV wide kernel): the slots
// are bf16 tiles in the compute layout -- lane x of a row's load fetches
// logical chunk x ^ swz32(r) and lands at chunk x -- so a tile is computed
// straight from its slot, with no staging registers and no LDS stores.
// Three slots: the tile computed and the two whose loads are in flight.
constexpr bool kWideBf16Ring = true;  // (the register-staged walk measured 4-5% slower here)
constexpr int kRingBSlots = 3;
struct SmemWideB {
  uint8_t qs[4][32 - kQRegDma][64 * 16];  // Q^T k-steps kQRegDma .. 31 per wave
};

// Direct-to-LDS loads of this wave's 8 rows of a bf16 tile (rows 8w .. 8w+7,
// indices at tidx), one 1 KiB row per load.  Invalid rows and positions past
// p1 read the zero row.
template <bool PACKED>
__device__ __forceinline__ void dma_rows_bf16(const DecodeArgs &a, const int32_t SMD_LDS *tidx, int first_pos, int p1,
                                              int wave, int lane, uint8_t SMD_LDS *tile) {
  uint32_t widx[8];
  lds_read_idx8(tidx + wave * (kBK / 4), widx);
  const int rows_left = p1 - first_pos - wave * (kBK / 4);
  const uint8_t *z = g_zero_row;
#pragma unroll
  for (int i = 0; i < kBK / 4; ++i) {
    const int r = wave * (kBK / 4) + i;
    const int c = lane ^ swz32(r);
    const uint32_t idx = widx[i];
    const bool v = i < rows_left && idx < a.num_rows32;
    const uint8_t *src;
    if constexpr (PACKED)
      src = v ? a.kv_nope + (uint64_t)idx * a.row_stride32 + 16 * c : z + 16 * c;
    else if (!v)
      src = z + 16 * c;
    else
      src = c < kNope / 8 ? a.kv_nope + (uint64_t)idx * (uint64_t)a.nope_stride_b + 16 * c
                          : a.kv_rope + (uint64_t)idx * (uint64_t)a.rope_stride_b + 16 * (c - kNope / 8);
    lds_dma<16>(src, tile + r * kLdsRow);
  }
}

// Walk the range's tiles once (bf16 pools) on the bf16 ring.  Step t: wait
// for this wave's loads of tile t (the 8 of tile t+1 may still fly), read its
// valid bits, barrier (everyone's rows of t have landed and tile t-1 is done:
// its slot is free), issue tile t+2 into that slot (and, at t % 8 == 0,
// index block t/8 + 1), compute t from its slot.  Index block k is read from
// step 8k - 2 on; issued at step 8(k-1), it has landed by the wait of step
// 8k - 3 and that step's barrier publishes it.  The block it replaces was
// last read at step 8k - 9.
template <bool PACKED, bool P_HILO, int PASS>
__device__ __forceinline__ void run_split_wide_ringb(const DecodeArgs &a, SmemWideB &sm, const WideDma &dm,
                                                     const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                     const bf16x8 (&qreg)[kQRegDma], const WideLanes &L,
                                                     WideState &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  uint8_t SMD_LDS *raw = dm.raw;
  int32_t SMD_LDS *ib0 = dm.ibuf;
  const uint8_t SMD_LDS *qs = (const uint8_t SMD_LDS *)&sm.qs[wave][0][0];
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  auto slot = [&](int k) { return raw + (k % kRingBSlots) * kTileBytes; };
  constexpr int kAhead = kRingBSlots - 1;
  // A real vmcnt(0), as in run_split_wide_dma.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if constexpr (PASS != kPassMain) {  // the main pass's caller has done this, with the Q^T load
    __syncthreads();  // the ring may still be read by a previous pass
    dma_idx_block(row_idx, p0, p1, 0, wave, lane, ib0);
    wait_vm<0>();
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kAhead; ++k) dma_rows_bf16<PACKED>(a, tidx(k), p0 + k * kBK, p1, wave, lane, slot(k));
  for (int t = 0; t < ntiles; ++t) {
    wait_vm<(kBK / 4) * (kAhead - 1)>();
    const uint32_t v_cur = tile_valid_bits_dma(tidx(t), p0 + t * kBK, p1, lane, a.num_rows32);
    barrier_lds();
    dma_rows_bf16<PACKED>(a, tidx(t + kAhead), p0 + (t + kAhead) * kBK, p1, wave, lane, slot(t + kAhead));
    if (t % kTilesPerIdxBlock == 0) {
      const int nb = t / kTilesPerIdxBlock + 1;
      dma_idx_block(row_idx, p0, p1, nb, wave, lane, ib0 + (nb & 1) * kIdxBlock);
    }
    compute_tile_wide<kQRegDma, PASS, P_HILO>(slot(t), qreg, qs, L, v_cur, lane, a.scale_log2, w);
  }
  wait_vm<0>();  // no load may land in LDS after the walk
}

// ---------------------------------------------------------------------------
// fp8 QK ("a8w8", the persistent decode object of the aiter page "[ASM][HIP]
// [MLA v4 nm] Split plan helper and persistent decode kernel", Summary part
// 2): q_nope is quantised the way the cache writer quantises a latent row's
// NoPE (UE8M0 code per 64-dim block, E4M3FN bytes; quant.h), and the NoPE
// half of QK runs on v_mfma_scale_f32_32x32x64_f8f6f4 straight from the
// pool's bytes, the pool's UE8M0 codes and q's codes as the E8M0 block scales
// of the two operands.  RoPE (bf16 in the pool) stays on the bf16 MFMA, and P
// and PV stay bf16: V's scales vary along PV's contraction (one code per kv
// row and 64 dims), which the block scales of the MFMA cannot express.
//
// Operand layout of the scaled MFMA (checked on gfx950 with an in-bounds
// probe): lane l feeds row (A) / column (B) l mod 32 with 32 bytes, the
// first 16 in k-block 0 and the next 16 in k-block 1 of the 64 k, paired
// byte for byte between A and B; the scale of k-block kb of row / column r
// comes from lane r + 32 kb (byte opsel of its scale register).  Here both
// k-blocks of a lane carry one 64-dim block's values, so lane (r, u = l / 32)
// holds dims 64b + 32u .. +32 in order on both sides and the two lanes of a
// row carry the same code.

// q of a wide wave's 32 query rows (lane l: row l mod 32, u = l / 32).
// NQF of the 7 blocks sit in registers, the others in the wave's LDS region.
template <int NQF>
struct QF8Regs {
  i32x8 f[NQF];      // e4m3 bytes of NoPE dims 64b + 32u .. +32 (block b < NQF)
  uint32_t code[2];  // UE8M0 code of block b in byte b mod 4 of code[b / 4]
};

// q's operands in LDS, per wave: the RoPE part (bf16 B operands of 4
// k-steps; k-step j of lane l at (64 j + l) * 16, dims 448 + 16j + 8u .. +8),
// then NoPE blocks b >= NQF (block b of lane l at kQRopeWave + ((b - NQF) * 64
// + l) * 32).
constexpr int kQRopeWave = 4 * 64 * 16;
template <int NQF>
constexpr int qf8_lds_wave() {
  return kQRopeWave + (7 - NQF) * 64 * 32;
}

// Load and quantise q for the fp8 QK: the rows go row-wise through the
// wave's staging slice as in load_q_wide; lane (r, u) then picks up the 32
// values of its half of each block, the pair (r, u = 0 / 1) agrees on the
// block's code with one permlane32 swap, and each value is stored as the
// E4M3FN byte nearest to x * 2^(127 - code) (the hardware conversion rounds
// to nearest even; the scaling by a power of two is exact).
template <int NQF>
__device__ __forceinline__ void load_q_wide_fp8(const DecodeArgs &a, int64_t qbase, uint8_t SMD_LDS *stage,
                                                uint8_t SMD_LDS *qrope, QF8Regs<NQF> &q) {
  const int lane = opaque_lane();
  const int c = lane & 31, hr = lane >> 5;
  u32x4 v[2][16];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {  // rows 2k + hr, 16-byte chunk c of this half
      const int64_t row = qbase + 2 * k + hr;
      const uint16_t *src;
      if (half == 0)
        src = a.q_nope + row * kNope + 8 * c;
      else
        src = c < 24 ? a.q_nope + row * kNope + 256 + 8 * c : a.q_rope + row * kRope + 8 * (c - 24);
      v[half][k] = *(const u32x4 *)src;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  q.code[0] = q.code[1] = 0u;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int k = 0; k < 16; ++k) *(u32x4 SMD_LDS *)(stage + stage_off(2 * k + hr, c)) = v[half][k];
    // block b of this half: chunks 8(b mod 4) + 4 hr + i of row c (dims 64b + 32 hr + 8i ..)
#pragma unroll
    for (int bb = 0; bb < (half == 0 ? 4 : 3); ++bb) {
      const int b = 4 * half + bb;
      float x[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 w4 = *(const u32x4 SMD_LDS *)(stage + stage_off(c, 8 * bb + 4 * hr + i));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * i + 2 * e] = __uint_as_float(w4[e] << 16);
          x[8 * i + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      }
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));  // fmaxf ignores NaN
      const uint32_t code = ue8m0_code(half_max(m));
      const int e = 127 - (int)code;
      i32x8 f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * k], e), ldexpf(x[4 * k + 1], e), 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * k + 2], e), ldexpf(x[4 * k + 3], e), wd, true);
        f[k] = wd;
      }
      if (b < NQF)
        q.f[b < NQF ? b : 0] = f;
      else
        *(i32x8 SMD_LDS *)(qrope + kQRopeWave + ((b - NQF) * 64 + lane) * 32) = f;
      q.code[b >> 2] |= code << (8 * (b & 3));
    }
    if (half == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(bf16x8 SMD_LDS *)(qrope + (64 * j + lane) * 16) = *(const bf16x8 SMD_LDS *)(stage + stage_off(c, 24 + 2 * j + hr));
    }
  }
}

// Per-lane byte offsets, from a slot's first region, of the fp8 QK's A
// operands in the swizzled ring (lane l: kv row R = l mod 32 of the tile,
// which is local row r = R mod 8 of region R / 8; u = l / 32).  NoPE block b,
// half e: logical chunk 4b + 2u + e sits at position 4 (b ^ 2 hi) + ((2u + e)
// ^ (r mod 4)) with hi = r / 4, i.e. at nope[e][(b / 2) mod 2] + 64 b.  RoPE
// k-step j: chunk 2j + u at position 2 (j ^ (s / 2)) + (u ^ (s mod 2)) with
// s = raw_swz_rope(r), i.e. at rope[j mod 2] + 32 j.  code: the row's 8 code
// bytes.
struct RawLanes {
  uint32_t nope[2][2];
  uint32_t rope[2];
  uint32_t code;
};

__device__ __forceinline__ RawLanes raw_lanes(int lane) {
  constexpr int W = raw_wave<true>();
  const int R = lane & 31, u = lane >> 5, reg = R >> 3, r = R & 7, hi = r >> 2;
  const int rowbase = reg * W + kRawNope + (r >> 1) * 1024 + (r & 1) * 512;
  RawLanes K;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int lo = (2 * u + e) ^ (r & 3);
    K.nope[e][0] = (uint32_t)(rowbase + 16 * lo + 128 * hi);
    K.nope[e][1] = (uint32_t)(rowbase + 16 * lo - 128 * hi);
  }
  const int sr = raw_swz_rope<true>(r);
  const int rb = reg * W + kRawRope + 128 * r + 16 * (u ^ (sr & 1));
  K.rope[0] = (uint32_t)(rb + 32 * (sr >> 1));
  K.rope[1] = (uint32_t)(rb - 32 * (sr >> 1));
  K.code = (uint32_t)(reg * W + kRawCode + 8 * r);
  return K;
}

// One scaled fp8 MFMA (e4m3 A and B) whose block scales are byte `sel` of the
// scale registers (the byte select is an immediate; sel folds to a constant
// once the caller's loop is unrolled).
__device__ __forceinline__ f32x16 mfma_fp8_block(int sel, const i32x8 &a, const i32x8 &b, const f32x16 &c, int sa,
                                                 int sb) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 1, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 2, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 3, sa, 3, sb);
  }
}

// S^T[32 kv x 32 q] of one tile from its raw slot: 7 scaled fp8 MFMAs (k = 64
// dims each) and 4 bf16 MFMAs (RoPE).  The slot is read with plain LDS loads:
// its loads have landed and been published by a barrier before this runs.
template <int NQF>
__device__ __forceinline__ f32x16 qk_wide_fp8(const uint8_t SMD_LDS *slot, const QF8Regs<NQF> &q,
                                              const uint8_t SMD_LDS *qrope, int lane, const RawLanes &K) {
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
  const u32x2 kc = *(const u32x2 SMD_LDS *)(slot + K.code);
  u32x4 ka[2][2];
  i32x8 qa[2];  // q blocks >= NQF, read with their K operands
  auto ld = [&](int b) {
    const int sel = (b >> 1) & 1;
    ka[b & 1][0] = *(const u32x4 SMD_LDS *)(slot + K.nope[0][sel] + 64 * b);
    ka[b & 1][1] = *(const u32x4 SMD_LDS *)(slot + K.nope[1][sel] + 64 * b);
    if (b >= NQF) qa[b & 1] = *(const i32x8 SMD_LDS *)(qrope + kQRopeWave + ((b - NQF) * 64 + lane) * 32);
  };
  bf16x8 kr[2], qr[2];
  auto ldr = [&](int j) {
    kr[j & 1] = *(const bf16x8 SMD_LDS *)(slot + K.rope[j & 1] + 32 * j);
    qr[j & 1] = *(const bf16x8 SMD_LDS *)(qrope + (64 * j + lane) * 16);
  };
  ld(0);
  ld(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const u32x4 lo = ka[b & 1][0], hi = ka[b & 1][1];
    const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    if (b + 2 < 7) ld(b + 2);
    if (b >= 5) ldr(b - 5);  // the RoPE operands take the freed NoPE buffers' turn
    const i32x8 bv = b < NQF ? q.f[b < NQF ? b : 0] : qa[b & 1];
    s = mfma_fp8_block(b & 3, av, bv, s, (int)kc[b >> 2], (int)q.code[b >> 2]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8 av = kr[j & 1], bv = qr[j & 1];
    if (j + 2 < 4) ldr(j + 2);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, s, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// Walk the range's tiles once with the fp8 QK: a ring of four swizzled raw
// slots, tile k's loads going to slot k % 4 at step k - 3.  Step t:
//   wait for this wave's loads of tile t (12 younger loads allowed: tiles
//   t+1 and t+2);
//   barrier A (every wave's rows of tile t have landed; everyone is done with
//   the PV of t-1, so the bf16 tile is free, and with the QK of t-1, so slot
//   (t+3) % 4 is free);
//   issue the loads of tile t+3 (and, at t % 8 == 0, index block t/8 + 1);
//   dequantise this wave's rows of tile t (read out of the slot before
//   barrier A) into the bf16 tile for PV; QK of tile t from its raw slot;
//   softmax weights;
//   barrier B (the bf16 tile is complete), PV.
// (Issuing the loads and the stores between the QK MFMAs instead ran 9%
// slower on the ragged MTP4 fp8 workload.)
// The index blocks follow run_split_wide_dma's schedule.
template <bool P_HILO, int PASS, bool RESIDENT, int NQF>
__device__ __forceinline__ void run_split_wide_qf8(const DecodeArgs &a, uint8_t SMD_LDS *tile,
                                                   const uint8_t SMD_LDS *qrope, const WideDma &dm,
                                                   const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                   const QF8Regs<NQF> &q, const WideLanes &L, WideState &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  constexpr int kSlots = raw_slots<true>();
  uint8_t SMD_LDS *raw = dm.raw;
  int32_t SMD_LDS *ib0 = dm.ibuf;
  auto tidx = [&](int k) {
    return ib0 + ((k / kTilesPerIdxBlock) & 1) * kIdxBlock + (k % kTilesPerIdxBlock) * kBK;
  };
  auto slot = [&](int k) { return raw + (k % kSlots) * raw_slot<true>(); };
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), as in run_split_wide_dma
  if constexpr (PASS != kPassMain) {
    __syncthreads();
    dma_idx_block(row_idx, p0, p1, 0, wave, lane, ib0);
    wait_vm<0>();
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kRawAhead; ++k)
    dma_rows_fp8<true>(a, tidx(k), p0 + k * kBK, p1, wave, lane, slot(k) + wave * raw_wave<true>());
  // Lane offsets inside the loop come from opaque_lane(): recomputed (a few
  // VALU) rather than hoisted and spilled, since every spill reload would
  // wait for the whole ring of loads in flight.
  const RawLanes K0 = raw_lanes(lane);
  const WideLanes L0 = wide_lanes(lane);
  for (int t = 0; t < ntiles; ++t) {
    // RESIDENT keeps the lane offsets in registers; otherwise they come from
    // opaque_lane() and are recomputed (a few VALU) rather than hoisted and
    // spilled, since every spill reload would wait for the whole ring of
    // loads in flight
    const int ln = RESIDENT ? lane : opaque_lane();
    wait_vm<6 * (kRawAhead - 1)>();
    Staged<true> st;
    if constexpr (PASS != kPassMax) raw_to_staged<true>(slot(t) + wave * raw_wave<true>(), st);
    const uint32_t v_cur = tile_valid_bits_dma(tidx(t), p0 + t * kBK, p1, ln, a.num_rows32);
    barrier_lds();  // A
    dma_rows_fp8<true>(a, tidx(t + kRawAhead), p0 + (t + kRawAhead) * kBK, p1, wave,
                       RESIDENT ? lane : opaque_lane(), slot(t + kRawAhead) + wave * raw_wave<true>());
    if (t % kTilesPerIdxBlock == 0) {
      const int nb = t / kTilesPerIdxBlock + 1;
      dma_idx_block(row_idx, p0, p1, nb, wave, lane, ib0 + (nb & 1) * kIdxBlock);
    }
    if constexpr (PASS != kPassMax) store_rows<true, kLay32>(tile, wave, RESIDENT ? lane : opaque_lane(), st);
    f32x16 s = qk_wide_fp8(slot(t), q, qrope, ln, RESIDENT ? K0 : raw_lanes(opaque_lane()));
    bf16x8 pb[2], pl[2];
    const bool acc = softmax_wide<PASS, P_HILO>(s, v_cur, ln, a.scale_log2, w, pb, pl);
    barrier_lds();  // B
    if (acc) pv_wide<P_HILO>(tile, RESIDENT ? L0 : wide_lanes(opaque_lane()), pb, pl, w);
  }
  wait_vm<0>();  // no load may land in LDS after the walk
}

// The bf16 tile of the fp8-QK walk and q's RoPE operands (its raw ring and
// index blocks are the WideDma objects).
template <int NQF>
struct SmemWideQ {
  uint8_t tile[1][kTileBytes];
  uint8_t qrope[4][qf8_lds_wave<NQF>()];  // q's operands in LDS, per wave
};

// attend_range_wide for the fp8 QK (fp8 pools): the main pass, and the
// exact-max two-pass redo when some score overflowed its reference max.
// Ends with a barrier; the tile and the ring are then free.  RESIDENT: the
// walk keeps its lane offsets in registers (a caller with registers to
// spare), else it recomputes them each tile.  NQF of q's 7 fp8 blocks stay
// in registers, the rest in LDS.
template <bool P_HILO, bool RESIDENT, int NQF>
__device__ __forceinline__ void attend_range_wide_qf8(const DecodeArgs &a, SmemWideQ<NQF> &sm, const WideDma &dm,
                                                      const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                      int64_t qbase, QF8Regs<NQF> &q, const WideLanes &L,
                                                      WideState &w) {
  auto reset = [&]() {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) w.acc[d][e] = 0.f;
    }
    w.m_ref = -INFINITY;
    w.l_run = 0.f;
  };
  uint8_t SMD_LDS *tile = (uint8_t SMD_LDS *)&sm.tile[0][0];
  uint8_t SMD_LDS *qrope = (uint8_t SMD_LDS *)&sm.qrope[wave][0];
  __syncthreads();  // the tile, the ring and the index blocks may still be in use by a previous range
  if (p1 > p0) dma_idx_block(row_idx, p0, p1, 0, wave, lane, dm.ibuf);
  load_q_wide_fp8(a, qbase, dm.raw + wave * kStageWave, qrope, q);
  reset();
  w.overflow = false;
  run_split_wide_qf8<P_HILO, kPassMain, RESIDENT, NQF>(a, tile, qrope, dm, row_idx, p0, p1, wave, lane, q, L, w);
  if (__syncthreads_or(w.overflow)) {
    reset();
    run_split_wide_qf8<P_HILO, kPassMax, RESIDENT, NQF>(a, tile, qrope, dm, row_idx, p0, p1, wave, lane, q, L, w);
    run_split_wide_qf8<P_HILO, kPassFixed, RESIDENT, NQF>(a, tile, qrope, dm, row_idx, p0, p1, wave, lane, q, L, w);
  }
  __syncthreads();  // as in attend_range_wide
}

// Attend the wide wave's 32 query rows (rows qbase .. qbase + 31 of the
// queries; this lane's row is qbase + lane % 32) over positions [p0, p1) of
// row_idx: the main pass, and the exact-max two-pass redo when some score
// overflowed its reference max anywhere in the workgroup.  Ends with a
// barrier, so the tiles and the ring are free for the epilogue's staging.
template <bool FP8, bool PACKED, bool P_HILO, bool RING = wide_ring<FP8>()>
__device__ __forceinline__ void attend_range_wide(const DecodeArgs &a, SmemWide<RING> &sm, const WideDma &dm,
                                                  const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                  int64_t qbase, bf16x8 (&qreg)[wide_qreg<RING>()],
                                                  const WideLanes &L, WideState &w) {
  auto reset = [&]() {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) w.acc[d][e] = 0.f;
    }
    w.m_ref = -INFINITY;
    w.l_run = 0.f;
  };
  auto walk = [&](auto pass) {
    constexpr int PASS = decltype(pass)::value;
    if constexpr (RING)
      run_split_wide_dma<P_HILO, PASS>(a, sm, dm, row_idx, p0, p1, wave, lane, qreg, L, w);
    else
      run_split_wide<FP8, PACKED, P_HILO, PASS>(a, sm, row_idx, p0, p1, wave, lane, qreg, L, w);
  };
  __syncthreads();  // the tiles, the ring and the index blocks may still be in use by a previous range
  if constexpr (RING) {
    // The first index block of the main pass goes out ahead of the Q^T
    // loads: the two round trips overlap instead of following each other.
    if (p1 > p0) dma_idx_block(row_idx, p0, p1, 0, wave, lane, dm.ibuf);
  }
  load_q_wide<wide_qreg<RING>()>(a, qbase, lane, wide_stage<RING>(sm, dm, wave),
                                 (uint8_t SMD_LDS *)&sm.qs[wave][0][0], qreg);
  reset();
  w.overflow = false;
  walk(std::integral_constant<int, kPassMain>{});
  if (__syncthreads_or(w.overflow)) {
    reset();
    walk(std::integral_constant<int, kPassMax>{});
    walk(std::integral_constant<int, kPassFixed>{});
  }
  // every wave's loads have landed (each waited for its own) and its tile
  // reads are done before the epilogue stages through the ring or the tiles
  __syncthreads();
}

// attend_range_wide for bf16 pools on the bf16 ring (run_split_wide_ringb).
template <bool PACKED, bool P_HILO>
__device__ __forceinline__ void attend_range_wide_b(const DecodeArgs &a, SmemWideB &sm, const WideDma &dm,
                                                    const int32_t *row_idx, int p0, int p1, int wave, int lane,
                                                    int64_t qbase, bf16x8 (&qreg)[kQRegDma], const WideLanes &L,
                                                    WideState &w) {
  auto reset = [&]() {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) w.acc[d][e] = 0.f;
    }
    w.m_ref = -INFINITY;
    w.l_run = 0.f;
  };
  __syncthreads();  // the ring and the index blocks may still be in use by a previous range
  if (p1 > p0) dma_idx_block(row_idx, p0, p1, 0, wave, lane, dm.ibuf);
  static_assert(kRingBSlots * kTileBytes >= 4 * kStageWave, "staging slices fit the ring");
  load_q_wide<kQRegDma>(a, qbase, lane, dm.raw + wave * kStageWave, (uint8_t SMD_LDS *)&sm.qs[wave][0][0], qreg);
  reset();
  w.overflow = false;
  run_split_wide_ringb<PACKED, P_HILO, kPassMain>(a, sm, dm, row_idx, p0, p1, wave, lane, qreg, L, w);
  if (__syncthreads_or(w.overflow)) {
    reset();
    run_split_wide_ringb<PACKED, P_HILO, kPassMax>(a, sm, dm, row_idx, p0, p1, wave, lane, qreg, L, w);
    run_split_wide_ringb<PACKED, P_HILO, kPassFixed>(a, sm, dm, row_idx, p0, p1, wave, lane, qreg, L, w);
  }
  __syncthreads();  // as in attend_range_wide
}

// Outputs of a wide wave's 32 query rows, stored row-wise through the wave's
// staging slice (the accumulators hold dims 32D + 8b + 4u .. +4 of row
// lane % 32 in acc[D][4b .. 4b+3], u = lane / 32).
__device__ __forceinline__ f32x4 wide_quad(const f32x16 &v, int b) {
  return f32x4{v[4 * b], v[4 * b + 1], v[4 * b + 2], v[4 * b + 3]};
}


// The other pieces of a split row group, for the merge below (at most
// kRegMergeMax of them).
constexpr int kRegMergeMax = 8;
struct PiecePtrs {
  const uint16_t *o;  // bf16 rows, kDim apart
  const float *lse;
};
struct NoPieces {
  __device__ PiecePtrs operator()(int) const { return PiecePtrs{nullptr, nullptr}; }
};

// What a wide wave writes for its 32 rows, row-wise through its staging
// slice:
//   !MERGE: bf16 out = scale * O, or (f32) FP32 rows = scale * O (a split
//           partial); scale belongs to this lane's row (lane % 32);
//    MERGE: bf16 out = the merge of this piece and the n >= 1 other pieces
//           part(0..n-1) of a split row group (merge_weights_wide gives the
//           weights): this piece's partial is scale * O (scale = 1 / l_tot,
//           the value its partial would hold) at position own_k of the span;
//           for row r the other pieces' weights sit at tbl[32 k + r], this
//           piece's at tbl[32 kRegMergeMax + r] and 1 / Z at
//           tbl[32 (kRegMergeMax + 1) + r].  Per element, in span order from
//           zero with one fused multiply-add per piece, then times 1 / Z: the
//           operations of merge_pieces_narrow, so a row group merged here and
//           one merged from the workspace hold the same bits (this piece's
//           partial is rounded to bf16 first, as its slot would hold it).
// dst points at dim 0 of the wave's first row, rows row_stride elements
// apart (uint16_t for bf16, float for FP32); part(k).o points at dim 0 of the
// wave's first row in the k-th other piece's bf16 partial (rows kDim
// elements apart).  Four passes of 128 dims: the wave's part goes to the stage in fp32
// in the accumulator layout (lane (q, u) holds row q); a merge then works
// row-wise (lane (q, u): rows 2k + u, dims 4q..4q+3 of the pass), loading the
// other pieces' rows in that layout, and writes its sums back to the stage;
// the rows leave in 16-byte stores: FP32 lane (q, u) takes rows 2k + u, dims
// 4q..4q+3; bf16 lane l takes rows 4k + l / 16, dims 8 (l mod 16) .. +7.  The
// first other piece's rows of the next pass are loaded before this pass's
// stores go out (a load waits for every store issued before it), once this
// pass's sums no longer need the registers.  Every LDS read of a phase is
// issued before its first use, and global addresses are a wave-uniform row
// base plus a 32-bit lane offset recomputed in each pass from a fresh lane
// id: 64-bit per-lane offsets kept across passes get spilled, and every
// reload waits for all the stores in flight.  (The passes are unrolled: acc
// may only be indexed by constants.)
template <bool MERGE, class Part = NoPieces>
__device__ __forceinline__ void store_rows_wide(const WideState &w, float scale, bool f32, void *dst,
                                                int64_t row_stride, uint8_t SMD_LDS *stage, Part part = Part(),
                                                int n = 0, int own_k = 0, const float SMD_LDS *tbl = nullptr) {
  auto piece_loads = [&](int pass, int j, u32x2 (&v)[16]) {
    const int lane = opaque_lane();
    const uint32_t poff = (uint32_t)((lane >> 5) * kDim + 128 * pass + 4 * (lane & 31)) * 2;
    const char *src = (const char *)part(j).o;
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = *(const u32x2 *)(src + (size_t)(2 * k * kDim * 2) + poff);
  };
  u32x2 pre[16];  // MERGE: the first other piece's rows of the next pass
  if constexpr (MERGE) piece_loads(0, 0, pre);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int lane = opaque_lane();
    const int q = lane & 31, u = lane >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i)  // i = 4dd + b: dims 32dd + 8b + 4u of the pass, chunk 8dd + 2b + u
      *(f32x4 SMD_LDS *)(stage + stage_off(q, 8 * (i >> 2) + 2 * (i & 3) + u)) =
          wide_quad(w.acc[4 * pass + (i >> 2)], i & 3) * scale;
    if constexpr (MERGE) {
      f32x4 o[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto add = [&](const u32x2 (&v)[16], const float SMD_LDS *wt) {  // o += wt[row] * v, row 2k + u
        float c[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) c[k] = wt[2 * k + u];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          o[k][0] = __builtin_fmaf(c[k], bf16_lo(v[k][0]), o[k][0]);
          o[k][1] = __builtin_fmaf(c[k], bf16_hi(v[k][0]), o[k][1]);
          o[k][2] = __builtin_fmaf(c[k], bf16_lo(v[k][1]), o[k][2]);
          o[k][3] = __builtin_fmaf(c[k], bf16_hi(v[k][1]), o[k][3]);
        }
      };
      auto add_own = [&]() {  // this piece's partial, rounded to bf16 as its slot would hold it
        u32x2 t[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const f32x4 x = *(const f32x4 SMD_LDS *)(stage + stage_off(2 * k + u, q));
          t[k] = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        }
        add(t, tbl + kRegMergeMax * 32);
      };
      if (own_k == 0) add_own();
      add(pre, tbl);  // the first other piece (the registers of pre are free after this)
#pragma unroll 1
      for (int j = 1; j < n; ++j) {
        if (j == own_k) add_own();
        u32x2 v[16];
        piece_loads(pass, j, v);
        add(v, tbl + j * 32);
      }
      if (own_k == n) add_own();
      if (pass < 3) piece_loads(pass + 1, 0, pre);
      float fin[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) fin[k] = tbl[(kRegMergeMax + 1) * 32 + 2 * k + u];
#pragma unroll
      for (int k = 0; k < 16; ++k) *(f32x4 SMD_LDS *)(stage + stage_off(2 * k + u, q)) = o[k] * fin[k];
    }
    char *drow = (char *)dst;
    if (!MERGE && f32) {
      const uint32_t voff = (uint32_t)(u * row_stride + 128 * pass + 4 * q) * 4;
      f32x4 o[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) o[k] = *(const f32x4 SMD_LDS *)(stage + stage_off(2 * k + u, q));
#pragma unroll
      for (int k = 0; k < 16; ++k) *(f32x4 *)(drow + (size_t)(2 * k * row_stride * 4) + voff) = o[k];
    } else {
      const int j = lane & 15, rr = lane >> 4;
      const uint32_t voff = (uint32_t)(rr * row_stride + 128 * pass + 8 * j) * 2;
      f32x4 o[8][2];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + rr;
        o[k][0] = *(const f32x4 SMD_LDS *)(stage + stage_off(r, 2 * j));
        o[k][1] = *(const f32x4 SMD_LDS *)(stage + stage_off(r, 2 * j + 1));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        u32x4 v;
        v[0] = pack_bf16x2(o[k][0][0], o[k][0][1]);
        v[1] = pack_bf16x2(o[k][0][2], o[k][0][3]);
        v[2] = pack_bf16x2(o[k][1][0], o[k][1][1]);
        v[3] = pack_bf16x2(o[k][1][2], o[k][1][3]);
        *(u32x4 *)(drow + (size_t)(4 * k * row_stride * 2) + voff) = v;
      }
    }
  }
}

// Weights for the piece of a split row group that finds every other piece
// already arrived: it merges straight from its registers and never writes or
// rereads a partial of its own.  The arithmetic is that of
// merge_pieces_narrow, with this piece's partial (o = O / l_tot, lse = m_ref
// ln 2 + ln l_tot, as partial_scale gives them) taken from registers:
//   mx  = max(sink, lse of every piece),  w_i = 2^((lse_i - mx) log2 e),
//   Z   = 2^((sink - mx) log2 e) + w_i summed in span order,
//   out = (sum_i w_i o_i, in span order) / Z,  lse = mx + ln Z
// (aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
// kernel", Summary part 1: pieces combine by their log-sum-exp, the sink
// once).  The n <= kRegMergeMax other pieces are part(0..n-1) in span order
// and this one sits at position own_k.  Leaves, for row r, the other pieces'
// weights in tbl[32 k + r], this piece's in tbl[32 kRegMergeMax + r] and 1 / Z
// in tbl[32 (kRegMergeMax + 1) + r] (tbl holds (kRegMergeMax + 2) * 32
// floats), and for this lane's row its partial scale in inv_l and the lse in
// lse_out.  An empty merge (no piece holds a row and no sink) gives zero
// weights and 1 / Z = 0 (zero output) and lse = -inf.
template <class Part>
__device__ __forceinline__ void merge_weights_wide(const WideState &w, float l_tot, float sink_ln, Part part, int n,
                                                   int own_k, float SMD_LDS *tbl, float &inv_l, float &lse_out) {
  const int lane = opaque_lane();
  const int q = lane & 31, u = lane >> 5;
  const OutScale ps = partial_scale(w.m_ref, l_tot);
  inv_l = ps.inv;
  float lo[kRegMergeMax];
#pragma unroll
  for (int k = 0; k < kRegMergeMax; ++k) lo[k] = k < n ? part(k).lse[q] : -INFINITY;
  float mx = fmaxf(sink_ln, ps.lse);
#pragma unroll
  for (int k = 0; k < kRegMergeMax; ++k) mx = fmaxf(mx, lo[k]);
  float c[kRegMergeMax], fin = 0.f, w_own = 0.f;
  lse_out = -INFINITY;
#pragma unroll
  for (int k = 0; k < kRegMergeMax; ++k) c[k] = 0.f;
  if (mx != -INFINITY) {
    float z = exp2_fast((sink_ln - mx) * kLog2e);
    w_own = exp2_fast((ps.lse - mx) * kLog2e);
#pragma unroll
    for (int k = 0; k <= kRegMergeMax; ++k) {
      if (k == own_k) z += w_own;
      if (k < kRegMergeMax && k < n) {
        c[k] = exp2_fast((lo[k] - mx) * kLog2e);
        z += c[k];
      }
    }
    fin = 1.f / z;
    lse_out = mx + logf(z);
  }
  if (u == 0) {
#pragma unroll
    for (int k = 0; k < kRegMergeMax; ++k) tbl[k * 32 + q] = c[k];
    tbl[kRegMergeMax * 32 + q] = w_own;
    tbl[(kRegMergeMax + 1) * 32 + q] = fin;
  }
}

}  // namespace smd
