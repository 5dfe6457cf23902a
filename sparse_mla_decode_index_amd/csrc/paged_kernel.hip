// Dense paged GQA decode for gfx950 (the pa_decode workload of the aiter page
// "[FlyDSL] [Perf] pa_decode: K/V streaming, MTP query split and sparse
// split-major on gfx950": separate K and V caches read through a block
// table, grouped-query heads, MTP query positions, split plans).
//
// A workgroup of 4 waves owns one (sequence b, KV head g, split r) and the
// M = 64 query rows that share that KV head: MTP position i = m / R and head
// g R + m % R for row m (R = Hq / Hkv).  Wave w owns rows 16w .. 16w+15 and
// all 512 dims.  The split's positions are walked in half-tiles of 16: the K
// rows and the V rows of a half-tile (16 KiB each) arrive by direct-to-LDS
// loads, one 1 KiB row per load instruction, into a ring of 4 slots that all
// four waves share, so no VGPRs hold rows ("K/V streaming" without a
// register prefetch): two half-tiles are in flight while one is computed and
// the slot before it waits for its pair's PV.  With page sizes a power of two
// of at least 16, a half-tile lies in one page: one block-table entry per
// half-tile, read from an LDS copy of the split's slice of the table.
//
// Per half-tile and wave: QK S^T[16 kv x 16 q] on v_mfma_f32_16x16x32_bf16
// (Q in VGPRs, K from the ring) and the fixed-reference softmax of the other
// decode kernels (reference max per query row, exact-max redo on overflow).
// Per pair of half-tiles: PV O^T[512 x 16 q] += V^T . P^T on
// v_mfma_f32_16x16x32_bf16 with V^T from transposed LDS reads (the 16-row
// kernel's building blocks, ks_core.h / ks8_core.h, on the same swizzled
// 16-row layout).  The MTP tokens are causal among themselves: a lane masks
// the positions at or beyond its query row's limit, so the mask is per row,
// not per tile.
//
// One split writes bf16 out and lse; several write partials (FP32 when the
// caller reads them, else bf16 scratch) that the stage-2 merge reduces (aiter
// page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
// kernel", Summary part 1).
#include "ks8_core.h"
#include "wide_core.h"

namespace smd {
namespace {

constexpr int kPgWaves = 4;
constexpr int kPgRows = 16 * kPgWaves;          // query rows per workgroup
constexpr int kPgHalf = 16;                     // positions per half-tile
constexpr int kPgSlot = 2 * kPgHalf * 1024;     // K then V rows of a half-tile
constexpr int kPgSlots = 4;
// Half-tiles in flight ahead of the one computed: two, so that the slot of
// half-tile k - 1 stays until its V has gone through the pair's PV at step k
// (three measured no faster).
constexpr int kPgAhead = 2;

// Q of this lane's query row as QK B operands: k-step ks holds dims
// 32 ks + 8 (lane / 16) .. +8.
__device__ __forceinline__ f32x4 qk_regs(const bf16x8 (&q)[16], const uint8_t SMD_LDS *buf, const ks::Lane &L) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  constexpr int kPre = 3;
  bf16x8 ka[kPre];
  auto load = [&](int ks) { ka[ks % kPre] = *(const bf16x8 SMD_LDS *)(buf + L.wb[ks & 3] + 256 * (ks >> 2)); };
#pragma unroll
  for (int ks = 0; ks < kPre; ++ks) load(ks);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const bf16x8 k = ka[ks % kPre];
    if (ks + kPre < 16) load(ks + kPre);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, q[ks], s, 0, 0, 0);
  }
  return s;
}

// PV of a pair of half-tiles (V rows at va_buf, vb_buf) on
// v_mfma_f32_16x16x32_bf16, the rate of which is twice that of the 16-deep
// shape: the contraction index k = 8 (lane / 16) + e stands for row
// 4 (lane / 16) + e mod 4 of the first half-tile (e < 4) or of the second
// (e >= 4), the order in which the two half-tiles' P leave the lane, and the
// V^T operand is two transposed reads of 4 rows, one per half-tile.
template <bool P_HILO>
__device__ __forceinline__ void pv_pair(const uint8_t SMD_LDS *va_buf, const uint8_t SMD_LDS *vb_buf, bf16x4 pa,
                                        bf16x4 pb, bf16x4 pla, bf16x4 plb, const ks::Lane &L, ks::State &st) {
  const bf16x8 p = __builtin_shufflevector(pa, pb, 0, 1, 2, 3, 4, 5, 6, 7);
  bf16x8 pl;
  if constexpr (P_HILO) pl = __builtin_shufflevector(pla, plb, 0, 1, 2, 3, 4, 5, 6, 7);
  constexpr int kPre = 4;
  bf16x8 v[kPre];
  auto load = [&](int d) {
    const int off = L.pv[d & 7] + 256 * (d >> 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(va_buf + off));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMD_LDS *)(vb_buf + off));
    v[d % kPre] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
#pragma unroll
  for (int d = 0; d < kPre; ++d) load(d);
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const bf16x8 va = v[d % kPre];
    if (d + kPre < 32) load(d + kPre);
    st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, p, st.acc[d], 0, 0, 0);
    if constexpr (P_HILO) st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, st.acc[d], 0, 0, 0);
  }
}

// Valid-row bits of half-tile positions [pos0, pos0 + 16) for a query row
// that sees positions below lim.
__device__ __forceinline__ uint32_t limit_bits(int pos0, int lim) {
  const int n = lim - pos0;
  return n >= kPgHalf ? 0xffffu : (n <= 0 ? 0u : ((1u << n) - 1u));
}

// The walk of one pass over positions [p0, p1): bt holds the block-table
// entries of pages pg0 .. (already checked: -1 for an entry outside the
// cache), lim the positions this lane's query row sees (at most p1).
template <bool P_HILO, int PASS>
__device__ __forceinline__ void paged_walk(const PagedArgs &a, uint8_t SMD_LDS *ring, const int32_t SMD_LDS *bt,
                                           int pg0, int p0, int p1, int g, int wave, int lane,
                                           const bf16x8 (&q)[16], const ks::Lane &L, int lim, ks::State &st) {
  const int nh = (p1 - p0 + kPgHalf - 1) / kPgHalf;
  if (nh <= 0) return;
  auto slot = [&](int k) { return ring + (k % kPgSlots) * kPgSlot; };
  // this wave's 4 K rows and 4 V rows of half-tile k; lane x of a row's load
  // lands at chunk x and fetches logical chunk x ^ swz(r) (the 16-row layout)
  auto issue = [&](int k) {
    const int pos0 = p0 + kPgHalf * k;
    const int32_t blk = pos0 < p1 ? bt[(pos0 >> a.page_shift) - pg0] : -1;
    const uint8_t *zero = g_zero_row;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * wave + rr;
      const int pos = pos0 + r;
      const bool v = blk >= 0 && pos < p1;
      const int c = lane ^ swz(r);
      const uint64_t row = v ? ((uint64_t)blk * a.page + (uint64_t)(pos & (a.page - 1))) * a.Hkv + g : 0;
      const uint8_t *sk = v ? a.k_cache + row * 1024 + 16 * c : zero + 16 * c;
      const uint8_t *sv = v ? a.v_cache + row * 1024 + 16 * c : zero + 16 * c;
      lds_dma<16>(sk, slot(k) + r * 1024);
      lds_dma<16>(sv, slot(k) + kPgHalf * 1024 + r * 1024);
    }
  };
  // A real vmcnt(0): the compiler's wait bookkeeping starts the walk with
  // nothing in flight (as in the wide walks).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();  // the ring may still be read by a previous pass
#pragma unroll
  for (int k = 0; k < kPgAhead; ++k) issue(k);
  // one half-tile's QK and softmax (p, pl: its P)
  auto half = [&](int k, bf16x4 &p, bf16x4 &pl) {
    wait_vm<8 * (kPgAhead - 1)>();  // this wave's rows of half-tile k have landed
    barrier_lds();                  // everyone's have; the slot of k + 2 has been through its pair's PV
    issue(k + kPgAhead);
    const int pos0 = p0 + kPgHalf * k;
    // a half-tile in a page outside the cache reads zero rows; mask them
    const uint32_t vb = bt[(pos0 >> a.page_shift) - pg0] >= 0 ? limit_bits(pos0, lim) : 0u;
    const f32x4 s = qk_regs(q, slot(k), L);
    ks::softmax_step<PASS, P_HILO>(s, vb, a.scale_log2, L, st.m_ref, st.l_run, st.overflow, p, pl);
  };
  const int npairs = nh >> 1;
  for (int j = 0; j < npairs; ++j) {
    bf16x4 pa, pla, pb, plb;
    half(2 * j, pa, pla);
    half(2 * j + 1, pb, plb);
    if constexpr (PASS != kPassMax)
      pv_pair<P_HILO>(slot(2 * j) + kPgHalf * 1024, slot(2 * j + 1) + kPgHalf * 1024, pa, pb, pla, plb, L, st);
  }
  if (nh & 1) {  // the last half-tile has no pair: it goes with itself and a zero P
    bf16x4 pa, pla;
    half(nh - 1, pa, pla);
    const bf16x4 zero = {};
    if constexpr (PASS != kPassMax)
      pv_pair<P_HILO>(slot(nh - 1) + kPgHalf * 1024, slot(nh - 1) + kPgHalf * 1024, pa, zero, pla, zero, L, st);
  }
  wait_vm<0>();  // no load may land in LDS after the walk
}

constexpr int kBtMax = 4096;  // block-table entries of one split held in LDS

template <bool P_HILO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void paged_decode_kernel(PagedArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kPgSlots * kPgSlot];
  __shared__ int32_t s_bt[kBtMax];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = blockIdx.x;
  const int r = u % a.S;
  const int g = (u / a.S) % a.Hkv;
  const int b = u / (a.S * a.Hkv);
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int p0 = min(r * a.chunk, L);
  const int p1 = min(p0 + a.chunk, L);

  // the block-table entries of pages pg0 .. pg1 - 1, checked against the cache
  const int pg0 = p0 >> a.page_shift;
  const int npg = p1 > p0 ? ((p1 - 1) >> a.page_shift) - pg0 + 1 : 0;
  for (int e = threadIdx.x; e < npg; e += blockDim.x) {
    const int32_t blk = a.block_tables[(int64_t)b * a.bt_stride + pg0 + e];
    s_bt[e] = (uint32_t)blk < (uint64_t)a.num_blocks ? blk : -1;
  }

  // this lane's query row: m = 16 wave + lane % 16 -> MTP position i, head h
  const ks::Lane Lk = ks::make_lane(lane);
  const int m = 16 * wave + Lk.j;
  const int i = m / a.R;
  const int h = g * a.R + m % a.R;
  const int64_t t = (int64_t)b * a.mtp + i;
  const int64_t row = t * a.Hq + h;
  const int lim = min(p1, L - (a.mtp - 1 - i));  // the MTP tokens are causal among themselves
  bf16x8 q[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) q[ks] = *(const bf16x8 *)(a.q + row * kDim + 32 * ks + 8 * Lk.g);

  ks::State st;
  auto reset = [&]() {
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.l_run = 0.f;
  };
  uint8_t SMD_LDS *ring = (uint8_t SMD_LDS *)s_ring;
  const int32_t SMD_LDS *bt = (const int32_t SMD_LDS *)s_bt;
  reset();
  st.overflow = false;
  paged_walk<P_HILO, kPassMain>(a, ring, bt, pg0, p0, p1, g, wave, lane, q, Lk, lim, st);
  if (__syncthreads_or(st.overflow)) {  // rare: redo with each row's exact max
    reset();
    paged_walk<P_HILO, kPassMax>(a, ring, bt, pg0, p0, p1, g, wave, lane, q, Lk, lim, st);
    paged_walk<P_HILO, kPassFixed>(a, ring, bt, pg0, p0, p1, g, wave, lane, q, Lk, lim, st);
  }

  // epilogue: acc[d][e] holds dim 16d + 4(lane / 16) + e of this lane's row
  const float l_tot = group_sum(st.l_run);
  const bool lse_lane = Lk.g == 0;
  if (a.S == 1 && a.out != nullptr) {
    const OutScale sc = direct_scale(st.m_ref, l_tot, -INFINITY);
    uint16_t *dst = a.out + row * kDim + 4 * Lk.g;
#pragma unroll
    for (int d = 0; d < 32; ++d) *(u32x2 *)(dst + 16 * d) = pack_bf16x4(st.acc[d], sc.inv);
    if (a.lse != nullptr && lse_lane) a.lse[row] = sc.lse;
  } else if (a.hilo) {  // FP32 partials, returned to the caller
    const OutScale sc = partial_scale(st.m_ref, l_tot);
    float *dst = a.part_o + (row * a.S + r) * kDim + 4 * Lk.g;
#pragma unroll
    for (int d = 0; d < 32; ++d) *(f32x4 *)(dst + 16 * d) = st.acc[d] * sc.inv;
    if (lse_lane) a.part_lse[row * a.S + r] = sc.lse;
  } else {  // bf16 partials in the same buffer: they only feed the merge
    const OutScale sc = partial_scale(st.m_ref, l_tot);
    uint16_t *dst = (uint16_t *)a.part_o + (row * a.S + r) * kDim + 4 * Lk.g;
#pragma unroll
    for (int d = 0; d < 32; ++d) *(u32x2 *)(dst + 16 * d) = pack_bf16x4(st.acc[d], sc.inv);
    if (lse_lane) a.part_lse[row * a.S + r] = sc.lse;
  }
}

}  // namespace

hipError_t launch_paged_decode(const PagedArgs &a, hipStream_t stream) {
  if (a.R * a.mtp != kPgRows || a.page < kPgHalf || (a.page & (a.page - 1)) || a.S < 1 ||
      (a.chunk + a.page - 1) / a.page + 1 > kBtMax)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)a.num_seqs * a.Hkv * a.S));
  if (a.hilo)
    hipLaunchKernelGGL(paged_decode_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(paged_decode_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smd
