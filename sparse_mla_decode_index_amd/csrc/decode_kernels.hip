// Split-KV sparse MLA decode and stage-2 merge kernels for gfx950 (MI355X).
//
// What is computed (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
// decode on gfx950", Design): per query row, a 512-wide dot product (448 NoPE
// + 64 RoPE dims) with every selected latent row, an online softmax that also
// counts a per-head sink logit, and a PV product over the same 512-wide rows.
// Split partials and their merge follow the aiter page "[ASM][HIP][MLA v4 nm]
// Split plan helper and persistent decode kernel", Summary part 1.
//
// Work decomposition.  A workgroup owns one index row b, one group of
// 16*WAVES query rows (heads x MTP positions sharing that row) and one split
// r of the row's index positions.  Each wave owns 16 query rows.
//
// Per 32-row KV tile:
//   gather   every valid selected row is copied HBM -> LDS with one
//            16-byte-per-lane direct-to-LDS load per row (bf16), or loaded
//            into registers, dequantised (e4m3 x 2^(code-127) -> bf16) and
//            stored (fp8).  Invalid or out-of-split rows are copied from a
//            zero row, so stale LDS contents (even NaN) never reach the MFMAs.
//   QK       S^T[32 kv x 16 q] = K[32 x 512] . Q^T[512 x 16] with
//            v_mfma_f32_16x16x32_bf16; K is read from LDS, Q stays in VGPRs.
//            In this orientation each lane holds scores of one query row, so
//            the softmax statistics are per-lane values.
//   softmax  running max m and sum l per query row, reduced across the four
//            16-lane groups with two cross-lane exchanges; exp2 with the
//            scale pre-multiplied by log2(e).
//   PV       O^T[512 x 16] += V^T[512 x 32] . P^T[32 x 16]; P^T is the score
//            tile itself converted to bf16 in registers (no LDS round trip),
//            V^T comes from LDS with ds_read_b64_tr_b16 transposed reads.
// The LDS tile is row-major, 1 KiB per row, with the 16-byte chunks of row r
// permuted by an XOR of swz(r) so that both the 16-byte QK reads (16 rows, one
// column) and the 8-byte transposed reads (8 rows, 32 bytes each) touch
// distinct banks.
#include "smd_internal.h"

#include <math.h>

namespace smd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SMD_LDS __attribute__((address_space(3)))
#define SMD_GLOBAL __attribute__((address_space(1)))

constexpr int kBK = 32;                      // KV rows per tile
constexpr int kLdsRow = 1024;                // bytes per bf16 row in LDS
constexpr int kTileBytes = kBK * kLdsRow;    // 32 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// A zero row used as the source of every masked row (1 KiB of zero bytes:
// bf16 zeros, e4m3 zeros and UE8M0 code 0).
__device__ __attribute__((aligned(256))) uint8_t g_zero_row[1024];

// XOR permutation of 16-byte chunks for row r of a tile.  Rows r and r+16 share
// it.  swz is a bijection on 0..15 (QK reads of 16 consecutive rows hit 16
// distinct chunk slots) and maps rows 0..7 / 8..15 to even / odd values (the
// transposed reads of 8 rows x 32 bytes cover 256 distinct bytes).
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// HBM -> LDS copy of 16 bytes per active lane: lane l writes LDS bytes
// [lds + 16l, lds + 16l + 16).  Written as inline assembly so that the
// compiler does not order later LDS reads of the *other* tile buffer behind
// it; every caller waits for completion explicitly (s_waitcnt vmcnt(0))
// before the copied tile is read.
// M0 is reserved by the compiler, so the assembly saves and restores it.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}
// The same with 4 bytes per lane (lane l writes [lds + 4l, lds + 4l + 4)).
__device__ __forceinline__ void dma4(const void *src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void SMD_LDS *p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ float wave_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// UE8M0 code -> fp32 scale 2^(code-127).  Code 0 is the subnormal 2^-127.
__device__ __forceinline__ float ue8m0_scale(uint32_t code) {
  return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
}

// fp8 rows are first copied raw into LDS (448 e4m3 bytes, 128 RoPE bytes, 8
// code bytes per row), then expanded to the bf16 tile layout in one pass.
constexpr int kRawRow = 592;                 // 576 data bytes + 8 code bytes + pad
constexpr int kRawBytes = kBK * kRawRow;     // 18944
// A row's reference max is fixed at its first tile with a valid entry; a later
// score more than this far above it (log2 domain) sends the workgroup through
// an exact-max second pass, so every p = 2^(x - m_ref) stays <= 2^32.
constexpr float kRefSlackLog2 = 32.f;

template <int WAVES, bool FP8>
struct Smem {
  uint8_t tile[2][kTileBytes];
  uint8_t raw[FP8 ? kRawBytes : 16];
};

// Issue the HBM -> LDS copies of the tile rows this wave owns.  `idx_v` holds,
// in lane rr < 32, the pool row of tile row rr; bit rr of `valid` says whether
// that row is gathered (else the zero row is copied).
template <int WAVES, bool FP8>
__device__ __forceinline__ void issue_tile(const DecodeArgs &a, uint8_t SMD_LDS *tile,
                                           uint8_t SMD_LDS *raw, int wave, int lane, int idx_v,
                                           uint64_t valid) {
  constexpr int kRowsPerWave = kBK / WAVES;
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int rr = wave + k * WAVES;
    const int idx = __builtin_amdgcn_readlane(idx_v, rr);
    const bool v = (valid >> rr) & 1;
    if constexpr (!FP8) {
      // lane copies logical 16-byte chunk c of the row into physical slot `lane`
      const int c = lane ^ swz(rr);
      const uint8_t *nb = v ? a.kv_nope + (int64_t)idx * a.nope_stride_b : g_zero_row;
      const uint8_t *rb = v ? a.kv_rope + (int64_t)idx * a.rope_stride_b - kNope * 2 : g_zero_row;
      const uint8_t *src = (c < kNope / 8 ? nb : rb) + c * 16;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(tile + rr * kLdsRow)));
    } else {
      const uint8_t *nb = v ? a.kv_nope + (int64_t)idx * a.nope_stride_b : g_zero_row;
      const uint8_t *rb = v ? a.kv_rope + (int64_t)idx * a.rope_stride_b - kNope : g_zero_row;
      const uint8_t *sb = v ? a.kv_scale + (int64_t)idx * a.scale_stride_b : g_zero_row;
      if (lane < 36) {
        const uint8_t *src = (lane < 28 ? nb : rb) + lane * 16;
        dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(raw + rr * kRawRow)));
      }
      if (lane < 2) {
        dma4(sb + lane * 4, __builtin_amdgcn_readfirstlane(lds_addr(raw + rr * kRawRow + 576)));
      }
    }
  }
}

// fp8 raw rows -> bf16 tile rows: e4m3 x 2^(code-127) (exact in bf16), RoPE copied.
template <int WAVES>
__device__ __forceinline__ void dequant_tile(uint8_t SMD_LDS *tile, const uint8_t SMD_LDS *raw) {
  constexpr int kJobs = kBK * 36;
  constexpr int kThreads = WAVES * 64;
#pragma unroll
  for (int j0 = 0; j0 < kJobs; j0 += kThreads) {
    const int job = j0 + (int)threadIdx.x;
    if (kJobs % kThreads == 0 || job < kJobs) {
      const int rr = job / 36, ch = job - rr * 36;
      const uint8_t SMD_LDS *src = raw + rr * kRawRow;
      uint8_t SMD_LDS *dst = tile + rr * kLdsRow;
      const int f = swz(rr);
      const u32x4 w = *(const u32x4 SMD_LDS *)(src + ch * 16);
      if (ch < 28) {
        const float sc = ue8m0_scale(src[576 + (ch >> 2)]);
        u32x4 lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], sc, false));
          const uint32_t u1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], sc, true));
          if (q < 2) { lo[2 * q] = u0; lo[2 * q + 1] = u1; }
          else { hi[2 * q - 4] = u0; hi[2 * q - 3] = u1; }
        }
        *(u32x4 SMD_LDS *)(dst + (((2 * ch) ^ f) << 4)) = lo;
        *(u32x4 SMD_LDS *)(dst + (((2 * ch + 1) ^ f) << 4)) = hi;
      } else {
        *(u32x4 SMD_LDS *)(dst + (((kNope / 8 + ch - 28) ^ f) << 4)) = w;
      }
    }
  }
}

// Indices of tile `t` of positions [p0, p1): lane rr < 32 holds the pool row of
// tile row rr, or -1 beyond p1.
__device__ __forceinline__ int load_tile_indices(const int32_t *row_idx, int p0, int p1, int t, int lane) {
  const int pos = p0 + t * kBK + lane;
  return (lane < kBK && pos < p1) ? row_idx[pos] : -1;
}

__device__ __forceinline__ uint64_t tile_valid_mask(int idx_v, int64_t num_rows) {
  return __ballot(idx_v >= 0 && (int64_t)idx_v < num_rows) & 0xffffffffull;
}

// Per-wave state of the softmax and the O^T accumulator.
struct WaveState {
  f32x4 acc[32];  // acc[d][i] = sum_j 2^(x_j - m_ref) V[j][16d + 4grp + i]
  float m_ref;    // reference max (log2 domain), same in the four 16-lane groups
  float l_run;    // this lane's share of sum_j 2^(x_j - m_ref)
  bool overflow;  // some score exceeded m_ref + kRefSlackLog2 (this lane)
};

enum Pass { kPassMain = 0, kPassMax = 1, kPassFixed = 2 };

// QK, softmax weights and PV over one 32-row tile.  qk_base[c&3] and
// pv_base[d&7] are per-lane LDS byte offsets relative to the tile.
//   kPassMain:  m_ref is set at the row's first valid tile, later tiles only
//               flag scores above m_ref + kRefSlackLog2.
//   kPassMax:   QK only; m_ref becomes the exact running max.
//   kPassFixed: m_ref is already the exact max.
// The O accumulator is only ever touched by MFMAs here, never rescaled.
template <int PASS, bool P_HILO>
__device__ __forceinline__ void compute_tile(const uint8_t SMD_LDS *tile, const bf16x8 (&qreg)[16],
                                             const int (&qk_base)[4], const int (&pv_base)[8],
                                             uint64_t valid_t, int grp, float scale_log2,
                                             WaveState &w) {
  // ---- QK: S^T tiles for kv rows 0..15 (s0) and 16..31 (s1)
  // Operands are read kPre steps ahead of the MFMAs that consume them.
  constexpr int kPre = 4;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 k0[kPre], k1[kPre];
  auto qk_load = [&](int c) {
    const uint8_t SMD_LDS *p = tile + qk_base[c & 3] + 256 * (c >> 2);
    k0[c % kPre] = *(const bf16x8 SMD_LDS *)(p);
    k1[c % kPre] = *(const bf16x8 SMD_LDS *)(p + 16 * kLdsRow);
  };
#pragma unroll
  for (int c = 0; c < kPre; ++c) qk_load(c);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const bf16x8 a0 = k0[c % kPre], a1 = k1[c % kPre];
    if (c + kPre < 16) qk_load(c + kPre);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[c], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[c], s1, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads kPre steps ahead
  }

  // ---- scores; this lane holds kv rows 4grp+i (s0) and 16+4grp+i (s1)
  const uint32_t vbits = (uint32_t)valid_t;
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = ((vbits >> (4 * grp + i)) & 1) ? s0[i] * scale_log2 : -INFINITY;
    x[4 + i] = ((vbits >> (16 + 4 * grp + i)) & 1) ? s1[i] * scale_log2 : -INFINITY;
  }
  float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  tmax = fmaxf(tmax, wave_xor(tmax, 16));
  tmax = fmaxf(tmax, wave_xor(tmax, 32));
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

  // ---- PV: O^T[16d.., m] += V^T . P^T, V^T read transposed from LDS
  bf16x4 vlo[kPre], vhi[kPre];
  auto pv_load = [&](int d) {
    const uint8_t SMD_LDS *p = tile + pv_base[d & 7] + 256 * (d >> 3);
    vlo[d % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(p));
    vhi[d % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(p + 16 * kLdsRow));
  };
#pragma unroll
  for (int d = 0; d < kPre; ++d) pv_load(d);
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const bf16x8 av = __builtin_shufflevector(vlo[d % kPre], vhi[d % kPre], 0, 1, 2, 3, 4, 5, 6, 7);
    if (d + kPre < 32) pv_load(d + kPre);
    w.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, w.acc[d], 0, 0, 0);
    if constexpr (P_HILO) w.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl, w.acc[d], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Walk the split's tiles once: gather (double-buffered, the next tile's
// copies in flight during the current tile's math) and compute.
template <int WAVES, bool FP8, bool P_HILO, int PASS>
__device__ __forceinline__ void run_split(const DecodeArgs &a, uint8_t SMD_LDS *tile0,
                                          uint8_t SMD_LDS *tile1, uint8_t SMD_LDS *raw,
                                          const int32_t *row_idx, int p0, int p1, int wave,
                                          int lane, int grp, const bf16x8 (&qreg)[16],
                                          const int (&qk_base)[4], const int (&pv_base)[8],
                                          WaveState &w) {
  const int ntiles = (p1 - p0 + kBK - 1) / kBK;
  if (ntiles <= 0) return;
  int idx_cur = load_tile_indices(row_idx, p0, p1, 0, lane);
  uint64_t valid_cur = tile_valid_mask(idx_cur, a.num_rows);
  issue_tile<WAVES, FP8>(a, tile0, raw, wave, lane, idx_cur, valid_cur);
  int idx_next = (ntiles > 1) ? load_tile_indices(row_idx, p0, p1, 1, lane) : -1;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (FP8) {
    dequant_tile<WAVES>(tile0, raw);
    __syncthreads();
  }
  for (int t = 0; t < ntiles; ++t) {
    uint8_t SMD_LDS *cur = tile0 + (t & 1) * kTileBytes;
    uint8_t SMD_LDS *nxt = tile0 + ((t + 1) & 1) * kTileBytes;
    const uint64_t valid_t = valid_cur;
    uint64_t valid_nx = 0;
    int idx_nx2 = -1;
    const bool more = t + 1 < ntiles;
    if (more) {
      valid_nx = tile_valid_mask(idx_next, a.num_rows);
      issue_tile<WAVES, FP8>(a, nxt, raw, wave, lane, idx_next, valid_nx);
      if (t + 2 < ntiles) idx_nx2 = load_tile_indices(row_idx, p0, p1, t + 2, lane);
    }
    compute_tile<PASS, P_HILO>(cur, qreg, qk_base, pv_base, valid_t, grp, a.scale_log2, w);
    if (more) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (FP8) {
      if (more) {
        dequant_tile<WAVES>(nxt, raw);
        __syncthreads();
      }
    }
    valid_cur = valid_nx;
    idx_next = idx_nx2;
  }
}

template <int WAVES, bool FP8, bool P_HILO>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem<WAVES, FP8> sm;
  uint8_t SMD_LDS *tile0 = (uint8_t SMD_LDS *)sm.tile[0];
  uint8_t SMD_LDS *tile1 = (uint8_t SMD_LDS *)sm.tile[1];
  uint8_t SMD_LDS *raw = (uint8_t SMD_LDS *)sm.raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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
  const int m = g * (WAVES * 16) + wave * 16 + j;
  const int tok = b * a.qps + m / a.H;
  const int head = m % a.H;
  const int64_t qrow = (int64_t)tok * a.H + head;

  // Q^T as the B operand: chunk c holds dims 32c + 8*grp .. +7 of row m.
  bf16x8 qreg[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint16_t *src = (c < 14) ? a.q_nope + qrow * kNope + 32 * c + 8 * grp
                                   : a.q_rope + qrow * kRope + 32 * (c - 14) + 8 * grp;
    qreg[c] = *(const bf16x8 *)src;
  }

  // Per-lane LDS offsets.  QK: row j, logical chunk 4c+grp -> physical
  // (4c+grp) ^ swz(j); the xor only touches the low 4 chunk bits, so c>>2 is an
  // immediate 256-byte step.  PV: lanes 4t+q of a group supply row 4grp+t at
  // dims 16d+4q, logical chunk 2d+(q>>1), byte 8(q&1) within it.
  int qk_base[4], pv_base[8];
  {
    const int fj = swz(j);
#pragma unroll
    for (int c = 0; c < 4; ++c) qk_base[c] = j * kLdsRow + (((4 * c + grp) ^ fj) << 4);
    const int tq = j >> 2, qq = j & 3;
    const int tr_row = 4 * grp + tq;
    const int ftr = swz(tr_row);
#pragma unroll
    for (int d = 0; d < 8; ++d)
      pv_base[d] = tr_row * kLdsRow + (((2 * d + (qq >> 1)) ^ ftr) << 4) + ((qq & 1) << 3);
  }

  WaveState w;
#pragma unroll
  for (int d = 0; d < 32; ++d) w.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  w.m_ref = -INFINITY;
  w.l_run = 0.f;
  w.overflow = false;
  run_split<WAVES, FP8, P_HILO, kPassMain>(a, tile0, tile1, raw, row_idx, p0, p1, wave, lane, grp, qreg,
                                   qk_base, pv_base, w);
  if (__syncthreads_or(w.overflow)) {
    // Rare: a score ran far above its row's first-tile max.  Redo the split
    // with the exact max (found by a QK-only sweep) as the reference.
#pragma unroll
    for (int d = 0; d < 32; ++d) w.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    w.m_ref = -INFINITY;
    w.l_run = 0.f;
    run_split<WAVES, FP8, P_HILO, kPassMax>(a, tile0, tile1, raw, row_idx, p0, p1, wave, lane, grp, qreg,
                                    qk_base, pv_base, w);
    run_split<WAVES, FP8, P_HILO, kPassFixed>(a, tile0, tile1, raw, row_idx, p0, p1, wave, lane, grp,
                                      qreg, qk_base, pv_base, w);
  }

  // ---- epilogue: total sum per query row
  float l_tot = w.l_run;
  l_tot += wave_xor(l_tot, 16);
  l_tot += wave_xor(l_tot, 32);
  const float m_ref = w.m_ref;

  const int64_t orow = qrow;  // [T, H] row of this lane's query row
  if (a.S == 1 && a.out != nullptr) {
    const float sink2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
    const float mf = fmaxf(m_ref, sink2);
    float inv = 0.f, lse_v = -INFINITY;
    if (mf != -INFINITY) {
      const float e = exp2_fast(m_ref - mf);
      const float z = l_tot * e + exp2_fast(sink2 - mf);
      inv = e / z;
      lse_v = (mf + __log2f(z)) * kLn2;
    }
    uint16_t *dst = a.out + orow * kDim + 4 * grp;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      u32x2 v;
      v[0] = (uint32_t)f32_to_bf16_rne(w.acc[d][0] * inv) | ((uint32_t)f32_to_bf16_rne(w.acc[d][1] * inv) << 16);
      v[1] = (uint32_t)f32_to_bf16_rne(w.acc[d][2] * inv) | ((uint32_t)f32_to_bf16_rne(w.acc[d][3] * inv) << 16);
      *(u32x2 *)(dst + 16 * d) = v;
    }
    if (a.lse != nullptr && grp == 0) a.lse[orow] = lse_v;
  } else {
    float inv = 0.f, lse_v = -INFINITY;
    if (l_tot > 0.f) {
      inv = 1.f / l_tot;
      lse_v = (m_ref + __log2f(l_tot)) * kLn2;
    }
    float *dst = a.part_o + (orow * a.S + r) * kDim + 4 * grp;
#pragma unroll
    for (int d = 0; d < 32; ++d) *(f32x4 *)(dst + 16 * d) = w.acc[d] * inv;
    if (grp == 0) a.part_lse[orow * a.S + r] = lse_v;
  }
}

// Stage-2 merge: one wave per [T,H] row, 8 dims per lane.
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ po,
                                                    const float *__restrict__ plse, int rows, int H,
                                                    int S, const float *__restrict__ sink,
                                                    uint16_t *__restrict__ out, float *__restrict__ lse) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int head = row % H;
  const float *ls = plse + (int64_t)row * S;
  float mx = sink ? sink[head] : -INFINITY;
  for (int r = 0; r < S; ++r) mx = fmaxf(mx, ls[r]);
  uint16_t *dst = out + (int64_t)row * kDim + lane * 8;
  if (mx == -INFINITY) {
    *(u32x4 *)dst = u32x4{0u, 0u, 0u, 0u};
    if (lse && lane == 0) lse[row] = -INFINITY;
    return;
  }
  float z = sink ? exp2_fast((sink[head] - mx) * kLog2e) : 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float *src = po + (int64_t)row * S * kDim + lane * 8;
  for (int r = 0; r < S; ++r) {
    const float w = exp2_fast((ls[r] - mx) * kLog2e);
    z += w;
    const f32x4 v0 = *(const f32x4 *)(src + (int64_t)r * kDim);
    const f32x4 v1 = *(const f32x4 *)(src + (int64_t)r * kDim + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] += w * v0[i];
      o[4 + i] += w * v1[i];
    }
  }
  const float inv = 1.f / z;
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (uint32_t)f32_to_bf16_rne(o[2 * i] * inv) | ((uint32_t)f32_to_bf16_rne(o[2 * i + 1] * inv) << 16);
  *(u32x4 *)dst = v;
  if (lse && lane == 0) lse[row] = mx + logf(z);
}

template <int WAVES, bool FP8, bool P_HILO>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  const int blocks8 = (a.num_units + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.G));
  hipLaunchKernelGGL((decode_kernel<WAVES, FP8, P_HILO>), grid, dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}

template <bool P_HILO>
static hipError_t launch_decode_p(const DecodeArgs &a, int waves, bool fp8, hipStream_t stream) {
  switch (waves * 2 + (fp8 ? 1 : 0)) {
    case 2: return launch_decode_t<1, false, P_HILO>(a, stream);
    case 3: return launch_decode_t<1, true, P_HILO>(a, stream);
    case 4: return launch_decode_t<2, false, P_HILO>(a, stream);
    case 5: return launch_decode_t<2, true, P_HILO>(a, stream);
    case 8: return launch_decode_t<4, false, P_HILO>(a, stream);
    case 9: return launch_decode_t<4, true, P_HILO>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// Partials are written with the two-part P (FP32-partial precision); the
// direct bf16 output uses a single bf16 P.
hipError_t launch_decode(const DecodeArgs &a, int waves, bool fp8, hipStream_t stream) {
  return a.out != nullptr ? launch_decode_p<false>(a, waves, fp8, stream)
                          : launch_decode_p<true>(a, waves, fp8, stream);
}

hipError_t launch_merge(const float *part_o, const float *part_lse, int32_t rows, int32_t H,
                        int32_t S, const float *sink, uint16_t *out, float *lse,
                        hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, stream, part_o, part_lse, rows, H, S, sink,
                     out, lse);
  return hipGetLastError();
}

}  // namespace smd
