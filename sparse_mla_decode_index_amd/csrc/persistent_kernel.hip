// Persistent, graph-safe sparse MLA decode over ragged sequences (gfx950).
//
// The aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent
// decode kernel" (Summary, part 2) describes one launch with a fixed grid in
// which every workgroup derives the split plan inside the kernel from the live
// kv_indptr, unsplit rows are written as bf16 directly, and split rows are
// merged by the workgroup that arrives last.  The plan rule here (the pages do
// not print one): sequence b with tiles_b = ceil(K_b / 64) > 0 tiles takes
// tiles_b + 2 plan units, the first two charging the fixed cost of a piece
// (Q^T load, first round trips, epilogue) and the rest its tiles; the units of
// all sequences are concatenated in sequence order, partition p of P owns
// units [floor(p*total/P), floor((p+1)*total/P)), and a tile belongs to the
// partition that owns its unit.
//
// Grid: P partitions x G query-row groups of 16*RB rows, RB the largest of 8,
// 4, 2, 1 that divides M / 16 (8: the wide waves of wide_core.h, each wave
// 32 rows on 32x32 MFMAs, so one gathered tile serves 128 query rows).  Workgroup (p, g) walks the sequences of partition
// p and attends row group g of each over the piece of its index list that p
// owns.  A sequence inside one partition is
// written directly.  A sequence spread over partitions fp..lp is split: each
// piece writes a partial (o = O/l in bf16, lse = m + ln l in fp32; the merged
// result is bf16, so o needs no more) to its slot, releases
// it with an agent-scope fence and bumps the arrival counter of (g, fp); the
// workgroup that sees the count of the other pieces (the non-empty partitions
// of the span, minus one) merges the pieces in partition order
// (with the sink), writes bf16 out and lse, and resets the counter to zero, so
// the kernel can be replayed in a graph without any host-side reset.
// Sequences with K_b = 0 own no tile and are never written.
#include "wide_core.h"

#include <type_traits>

namespace smd {

PersistLayout persist_layout(int64_t M, int64_t P) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  PersistLayout l;
  l.plan_off = 0;
  l.ctr_off = up((size_t)P * 4 * sizeof(int32_t));
  l.slot_off = l.ctr_off + up((size_t)(M / 16) * (size_t)P * sizeof(uint32_t));
  l.total = l.slot_off + (size_t)2 * (size_t)P * (size_t)M * kSlotRowFloats * sizeof(float);
  return l;
}

// Inclusive prefix sum over the NT threads of the workgroup; `total` gets the
// sum of all NT values.  s_red holds NT / 64 ints and is free again on return.
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int *s_red, int &total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) s_red[wave] = v;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = s_red[w];
    off += w < wave ? x : 0;
    total += x;
  }
  __syncthreads();
  return v + off;
}

__device__ __forceinline__ int seq_tiles(const int32_t *ptr, int b) {
  return (max(ptr[b + 1] - ptr[b], 0) + kSplitAlign - 1) / kSplitAlign;  // decreasing: K_b = 0
}

// Plan units of a sequence: its tiles plus kSeqOverhead units charged for the
// fixed cost of a piece (none for K_b = 0).  Its tiles are its last tb units.
// (Measured on ragged MTP4 batches: a piece costs about two tiles more than
// its tiles, and charging it evens out the partitions' times.)
constexpr int kSeqOverhead = 2;
__device__ __forceinline__ int seq_units(int tb) { return tb > 0 ? tb + kSeqOverhead : 0; }

// The partition whose unit range holds unit x: the largest p with
// floor(p*total/P) <= x, i.e. floor(((x+1)*P - 1) / total).
__device__ __forceinline__ int tile_owner(int x, int total, int P) {
  return (int)(((int64_t)(x + 1) * P - 1) / total);
}

// Partition p owns no unit when floor(p*total/P) == floor((p+1)*total/P)
// (possible only when total < P).  Inside the span of a split sequence every
// unit is one of its tiles, so there a partition with a unit holds a piece.
__device__ __forceinline__ bool part_empty(int p, int total, int P) {
  return (int64_t)p * total / P == (int64_t)(p + 1) * total / P;
}

// Merge of the pieces of one split sequence for the workgroup's 16*RB query
// rows: LSE = ln(sum_q e^(lse_q) + e^(sink)), out = sum_q e^(lse_q - LSE) o_q.
// The pieces are held by the non-empty partitions among fp..lp, in that
// order.  The piece of partition q sits in slot 2q, except the first piece,
// which sits in slot 2fp+1 when the sequence is not the first of partition fp.
// A wave per query row (four rows of a wave at a time), 8 dims per lane;
// lane k looks at partition fp + k.
template <int NW>
__device__ __forceinline__ void merge_pieces(const PersistArgs &pa, int b, int g, int rows, int fp, int lp,
                                             int first_slot, int total) {
  // The slots were written by other workgroups, mostly on other XCDs, so
  // every load here is a long-latency miss: each wave keeps RU rows and up
  // to KP pieces per row in flight (16 loads of 16 bytes) instead of one
  // piece of one row.  (Larger batches spill at this point of the kernel,
  // and every spill reload waits for all loads in flight.)
  constexpr int RU = 4;
  const DecodeArgs &a = pa.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lp - fp + 1;  // partitions in the span (empty ones hold nothing)
  const size_t slot_floats = (size_t)a.M * kSlotRowFloats;
  auto slot_base = [&](int q) { return pa.slots + (size_t)(q == 0 ? first_slot : 2 * (fp + q)) * slot_floats; };
  for (int r0 = wave; r0 < rows; r0 += NW * RU) {
    int m[RU];
    int64_t qrow[RU];
    float sink[RU], mx[RU];
    bool live[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int r = r0 + NW * u;
      live[u] = r < rows;
      m[u] = g * rows + (live[u] ? r : r0);
      const int head = m[u] % a.H;
      qrow[u] = (int64_t)(b * a.qps + m[u] / a.H) * a.H + head;
      sink[u] = a.sink ? a.sink[head] : -INFINITY;
      mx[u] = sink[u];
    }
    // max over the pieces' lse and the sink
    for (int q0 = 0; q0 < n; q0 += 64) {
      const int q = q0 + lane;
      const bool held = q < n && !part_empty(fp + q, total, pa.P);
      const float *ls = slot_base(held ? q : 0) + (size_t)a.M * kSlotORowFloats;
      float l[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) l[u] = ls[m[u]];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        float v = held ? l[u] : -INFINITY;
        for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
        mx[u] = fmaxf(mx[u], v);
      }
    }
    float z[RU], o[RU][8];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      z[u] = mx[u] == -INFINITY ? 0.f : exp2_fast((sink[u] - mx[u]) * kLog2e);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[u][i] = 0.f;
    }
    for (int q0 = 0; q0 < n; q0 += 64) {
      const int ql = q0 + lane;
      const bool held = ql < n && !part_empty(fp + ql, total, pa.P);
      const float *ls = slot_base(held ? ql : 0) + (size_t)a.M * kSlotORowFloats;
      float wl[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const float l = ls[m[u]];
        wl[u] = (held && mx[u] != -INFINITY) ? exp2_fast((l - mx[u]) * kLog2e) : 0.f;
      }
      uint64_t mask = __ballot(held);  // wave-uniform
      while (mask) {
        // up to KP pieces per batch; absent ones repeat the first with weight 0
        constexpr int KP = 2;
        int kk[KP];
        bool has[KP];
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          has[i] = mask != 0;
          kk[i] = has[i] ? __builtin_ctzll(mask) : kk[0];
          if (has[i]) mask &= mask - 1;
        }
        u32x4 v[KP][RU];  // 8 bf16 dims per lane
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          const uint16_t *sp = (const uint16_t *)slot_base(q0 + kk[i]) + lane * 8;
#pragma unroll
          for (int u = 0; u < RU; ++u) v[i][u] = *(const u32x4 *)(sp + (size_t)m[u] * kDim);
        }
#pragma unroll
        for (int u = 0; u < RU; ++u) {
#pragma unroll
          for (int i = 0; i < KP; ++i) {
            const float wq = has[i] ? __shfl(wl[u], kk[i], 64) : 0.f;
            z[u] += wq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[u][2 * e] = __builtin_fmaf(wq, bf16_lo(v[i][u][e]), o[u][2 * e]);
              o[u][2 * e + 1] = __builtin_fmaf(wq, bf16_hi(v[i][u][e]), o[u][2 * e + 1]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      if (!live[u]) continue;
      uint16_t *dst = a.out + qrow[u] * kDim + lane * 8;
      if (mx[u] == -INFINITY) {
        *(u32x4 *)dst = u32x4{0u, 0u, 0u, 0u};
        if (a.lse != nullptr && lane == 0) a.lse[qrow[u]] = -INFINITY;
        continue;
      }
      const float inv = 1.f / z[u];
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = pack_bf16x2(o[u][2 * i] * inv, o[u][2 * i + 1] * inv);
      *(u32x4 *)dst = v;
      if (a.lse != nullptr && lane == 0) a.lse[qrow[u]] = mx[u] + logf(z[u]);
    }
  }
}

// merge_pieces for spans of at most 64 partitions (lane k holds piece k),
// with the rows a template constant: the lse of every row of the wave is
// loaded in one round trip up front, so the only serial misses left are one
// batch of slot loads per RU rows (instead of two lse trips per batch).
template <int NW, int ROWS>
__device__ __forceinline__ void merge_pieces_narrow(const PersistArgs &pa, int b, int g, int fp, int n,
                                                    int first_slot, int total) {
  constexpr int RPW = ROWS / NW;  // this wave's rows: wave, wave + NW, ...
  constexpr int RU = RPW < 4 ? RPW : 4, KP = 2;
  static_assert(ROWS % NW == 0 && RPW % RU == 0, "rows per wave");
  const DecodeArgs &a = pa.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t slot_floats = (size_t)a.M * kSlotRowFloats;
  auto slot_base = [&](int q) { return pa.slots + (size_t)(q == 0 ? first_slot : 2 * (fp + q)) * slot_floats; };
  const bool held = lane < n && !part_empty(fp + lane, total, pa.P);
  const uint64_t held_mask = __ballot(held);  // wave-uniform
  const float *ls = slot_base(held ? lane : 0) + (size_t)a.M * kSlotORowFloats;
  float l[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) l[i] = ls[g * ROWS + wave + NW * i];
#pragma unroll 1
  for (int i0 = 0; i0 < RPW; i0 += RU) {
    int m[RU];
    float mx[RU], wl[RU], z[RU], o[RU][8];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      m[u] = g * ROWS + wave + NW * (i0 + u);
      const float sink = a.sink ? a.sink[m[u] % a.H] : -INFINITY;
      float v = held ? l[u] : -INFINITY;
      for (int o2 = 32; o2 > 0; o2 >>= 1) v = fmaxf(v, __shfl_xor(v, o2, 64));
      mx[u] = fmaxf(v, sink);
      wl[u] = (held && mx[u] != -INFINITY) ? exp2_fast((l[u] - mx[u]) * kLog2e) : 0.f;
      z[u] = mx[u] == -INFINITY ? 0.f : exp2_fast((sink - mx[u]) * kLog2e);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[u][e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j + RU < RPW; ++j) l[j] = l[j + RU];  // the next batch's lse moves to the front
    uint64_t mask = held_mask;
    while (mask) {
      // up to KP pieces per batch; absent ones repeat the first with weight 0
      int kk[KP];
      bool has[KP];
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        has[i] = mask != 0;
        kk[i] = has[i] ? __builtin_ctzll(mask) : kk[0];
        if (has[i]) mask &= mask - 1;
      }
      u32x4 v[KP][RU];  // 8 bf16 dims per lane
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const uint16_t *sp = (const uint16_t *)slot_base(kk[i]) + lane * 8;
#pragma unroll
        for (int u = 0; u < RU; ++u) v[i][u] = *(const u32x4 *)(sp + (size_t)m[u] * kDim);
      }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          const float wq = has[i] ? __shfl(wl[u], kk[i], 64) : 0.f;
          z[u] += wq;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[u][2 * e] = __builtin_fmaf(wq, bf16_lo(v[i][u][e]), o[u][2 * e]);
            o[u][2 * e + 1] = __builtin_fmaf(wq, bf16_hi(v[i][u][e]), o[u][2 * e + 1]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int head = m[u] % a.H;
      const int64_t qrow = (int64_t)(b * a.qps + m[u] / a.H) * a.H + head;
      uint16_t *dst = a.out + qrow * kDim + lane * 8;
      if (mx[u] == -INFINITY) {
        *(u32x4 *)dst = u32x4{0u, 0u, 0u, 0u};
        if (a.lse != nullptr && lane == 0) a.lse[qrow] = -INFINITY;
        continue;
      }
      const float inv = 1.f / z[u];
      u32x4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vv[e] = pack_bf16x2(o[u][2 * e] * inv, o[u][2 * e + 1] * inv);
      *(u32x4 *)dst = vv;
      if (a.lse != nullptr && lane == 0) a.lse[qrow] = mx[u] + logf(z[u]);
    }
  }
}

// The plan of partition p from the live kv_indptr: total units, this
// partition's unit range [t0, t1), its first and last sequence with a tile in
// it and the first tile unit of that first sequence.  Row group 0 writes the
// descriptor.  Returns false (workgroup-uniform) when the partition owns no
// tile (no unit, or only units charged for a piece's fixed cost).
template <int NT>
__device__ __forceinline__ bool plan_partition(const PersistArgs &pa, int p, int g, int *s_red, int *s_last,
                                               int &total, int &t0, int &t1, int &b_first, int &b_last, int &start) {
  const int32_t *ptr = pa.kv_indptr;
  const int B = pa.B;
  {
    int loc = 0;
    for (int b = threadIdx.x; b < B; b += NT) loc += seq_units(seq_tiles(ptr, b));
    block_incl_scan<NT>(loc, s_red, total);
  }
  t0 = (int)((int64_t)p * total / pa.P);
  t1 = (int)((int64_t)(p + 1) * total / pa.P);
  __shared__ unsigned long long s_fst;  // (first sequence with a tile in [t0, t1)) << 32 | its first tile unit
  if (threadIdx.x == 0) {
    s_fst = ~0ull;
    *s_last = -1;
  }
  __syncthreads();
  if (t0 < t1) {
    int run = 0;
    for (int base = 0; base < B; base += NT) {
      const int b = base + (int)threadIdx.x;
      const int tb = b < B ? seq_tiles(ptr, b) : 0;
      const int ub = seq_units(tb);
      int chunk;
      const int st = run + block_incl_scan<NT>(ub, s_red, chunk) - ub + kSeqOverhead;  // first tile unit
      if (tb > 0 && st < t1 && st + tb > t0) {
        atomicMin(&s_fst, ((unsigned long long)b << 32) | (unsigned)st);
        atomicMax(s_last, b);
      }
      run += chunk;
      if (run >= t1) break;  // the same in every thread
    }
  }
  __syncthreads();
  b_first = s_fst == ~0ull ? -1 : (int)(s_fst >> 32);
  b_last = *s_last;
  start = (int)(s_fst & 0xffffffffu);
  if (g == 0 && threadIdx.x == 0) {
    int32_t *d = pa.plan + 4 * p;
    d[0] = t0;
    d[1] = t1;
    d[2] = b_first;
    d[3] = b_last;
  }
  return b_first >= 0;
}

// RB = 8 runs the wide waves of wide_core.h: wave w owns rows 32w .. 32w+31
// of the group's 128 rows, all 512 dims.
// QF8: the fp8 QK of wide_core.h (wide waves over an fp8 pool; options qk =
// SMD_QK_FP8).
template <int RB, bool FP8, bool PACKED, bool QF8 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void persistent_kernel(PersistArgs pa) {
  constexpr bool WIDE = RB == 8;
  static_assert(!QF8 || (WIDE && FP8), "the fp8 QK runs on the wide waves over an fp8 pool");
  constexpr int DS = WIDE ? 1 : 4 / RB;
  constexpr int NC = 16 / DS, ND = 32 / DS;
  constexpr int ROWS = 16 * RB;
  using SmemW = std::conditional_t<QF8, SmemWideQ<7>, SmemWide<wide_ring<FP8>()>>;
  __shared__ __attribute__((aligned(1024))) std::conditional_t<WIDE, SmemW, Smem<DS>> sm;
  __shared__ int s_red[4];
  __shared__ int s_last;
  __shared__ uint32_t s_arrived;
  const DecodeArgs &a = pa.d;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = WIDE ? wave : wave % RB, ds = WIDE ? 0 : wave / RB;
  const int j = lane & 15;
  const int grp = lane >> 4;

  // Workgroup -> (partition p, row group g); the G groups of a partition read
  // the same KV rows and are spaced 8 apart to share one XCD's L2.
  const int per = 8 * a.G;
  const int g = (int)(blockIdx.x % per) / 8;
  const int p = (int)(blockIdx.x / per) * 8 + (int)(blockIdx.x % 8);
  if (p >= pa.P) return;
  const int32_t *ptr = pa.kv_indptr;

  int total, t0, t1, b_first, b_last, start;
  if (!plan_partition<256>(pa, p, g, s_red, &s_last, total, t0, t1, b_first, b_last, start)) return;

  int qk_base[4], pv_base[8];
  if constexpr (!WIDE) lds_bases(j, grp, qk_base, pv_base);
  WideLanes wl;
  if constexpr (WIDE) wl = wide_lanes(lane);
  const int dcol = 16 * (ds * ND) + 4 * grp;
  const bool lse_lane = grp == 0 && ds == 0;
  const int m = g * ROWS + rb * 16 + j;  // this lane's query row within a sequence
  const int head = m % a.H;
  const size_t slot_floats = (size_t)a.M * kSlotRowFloats;

  for (int b = b_first; b <= b_last; ++b) {
    const int k0 = ptr[b];
    const int kb = max(ptr[b + 1] - k0, 0);
    const int tb = (kb + kSplitAlign - 1) / kSplitAlign;
    if (tb == 0) continue;
    if (b != b_first) start += kSeqOverhead;  // this sequence's first tile unit
    const int lo = max(t0, start), hi = min(t1, start + tb);
    const int pos0 = (lo - start) * kSplitAlign;
    const int pos1 = min((hi - start) * kSplitAlign, kb);
    const int fp = tile_owner(start, total, pa.P);
    const int lp = tile_owner(start + tb - 1, total, pa.P);

    const int slot = 2 * p + (lo == t0 ? 0 : 1);
    bool merged = false;  // this piece merged its row group from registers
    float *sb = pa.slots + slot * slot_floats;
    if constexpr (WIDE) {
      // wave w owns query rows 32w .. 32w+31 of the group: the consecutive
      // rows qbase .. qbase + 31 of the queries; this lane's row is
      // qbase + lane % 32 (query row mq of sequence b)
      const int mq0 = g * ROWS + 32 * wave;
      const int64_t qbase = (int64_t)b * a.M + mq0;
      const int64_t qrow = qbase + (lane & 31);
      const int hq = (int)(qrow % a.H);
      WideState w;
      WideDma dm = {nullptr, nullptr};
      if constexpr (WIDE && wide_ring<FP8>()) {
        __shared__ __attribute__((aligned(1024))) uint8_t s_raw[raw_slots<QF8>() * raw_slot<QF8>()];
        __shared__ __attribute__((aligned(16))) int32_t s_ibuf[2 * kIdxBlock];
        dm = WideDma{(uint8_t SMD_LDS *)s_raw, (int32_t SMD_LDS *)s_ibuf};
      }
      uint8_t SMD_LDS *stage;
      float SMD_LDS *tbl;  // merge weights: free until the next piece's walk
      if constexpr (QF8) {
        // the walk recomputes its lane offsets: this kernel's other live state
        // leaves no registers for them (kept, they spill inside the loop, even
        // with two of q's blocks moved to LDS)
        QF8Regs<7> q;  // loaded by attend_range_wide_qf8
        attend_range_wide_qf8<false, false, 7>(a, sm, dm, pa.kv_indices + k0, pos0, pos1, wave, lane, qbase, q, wl,
                                               w);
        stage = dm.raw + wave * kStageWave;
        tbl = (float SMD_LDS *)&sm.tile[0][0] + wave * 512;
      } else {
        bf16x8 qreg[wide_qreg<wide_ring<FP8>()>()];  // loaded by attend_range_wide
        attend_range_wide<FP8, PACKED, false>(a, sm, dm, pa.kv_indices + k0, pos0, pos1, wave, lane, qbase, qreg,
                                              wl, w);
        stage = wide_stage<wide_ring<FP8>()>(sm, dm, wave);
        tbl = (float SMD_LDS *)&sm.qs[wave][0][0];
      }
      const float l_tot = half_sum(w.l_run);
      const bool lse_lane = lane < 32;
      const int t0_fp = (int)((int64_t)fp * total / pa.P);
      // the k-th other piece of a merge: partition fp + k, skipping this one
      // (the register merge runs only when every partition of the span holds a piece)
      auto part = [&](int k) {
        const int qp = fp + k + (fp + k >= p ? 1 : 0);
        const int sl = qp == fp ? 2 * fp + (start == t0_fp ? 0 : 1) : 2 * qp;
        const float *base = pa.slots + (size_t)sl * slot_floats;
        return PiecePtrs{(const uint16_t *)base + (size_t)mq0 * kDim, base + (size_t)a.M * kSlotORowFloats + mq0};
      };
      const float sink_ln = a.sink ? a.sink[hq] : -INFINITY;
      float scale, lse_v;
      void *dst = a.out + qbase * kDim;
      float *lse_dst = (a.lse != nullptr && lse_lane) ? a.lse + qrow : nullptr;
      if (fp == lp) {
        const OutScale sc = direct_scale(w.m_ref, l_tot, sink_ln);
        scale = sc.inv;
        lse_v = sc.lse;
      } else {
        // When every other piece has arrived already (the usual case for the
        // piece that finishes last), this one merges from its registers and
        // writes no partial: nobody else can be last, since the count never
        // reaches the others' number of pieces from their side.  Both ways
        // of merging give the same bits.
        const int pieces = total >= pa.P ? lp - fp + 1 : tb;
        uint32_t *ctr = pa.counters + (size_t)g * pa.P + fp;
        if (threadIdx.x == 0) s_arrived = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        merged = pa.reg_merge && s_arrived == (uint32_t)(pieces - 1) && pieces - 1 <= kRegMergeMax &&
                 total >= pa.P;
        __syncthreads();  // s_arrived is rewritten below
        if (merged) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // acquire the other pieces
          merge_weights_wide(w, l_tot, sink_ln, part, pieces - 1, p - fp, tbl, scale, lse_v);
          if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const OutScale sc = partial_scale(w.m_ref, l_tot);
          scale = sc.inv;
          lse_v = sc.lse;
          dst = (uint16_t *)sb + (size_t)mq0 * kDim;
          lse_dst = lse_lane ? sb + (size_t)a.M * kSlotORowFloats + mq0 + (lane & 31) : nullptr;
        }
      }
      if (merged)
        store_rows_wide<true>(w, scale, false, dst, kDim, stage, part, lp - fp, p - fp, tbl);
      else
        store_rows_wide<false>(w, scale, false, dst, kDim, stage);  // bf16 out or a bf16 partial
      if (lse_dst != nullptr) *lse_dst = lse_v;
    } else {
      const int64_t qrow = (int64_t)(b * a.qps + m / a.H) * a.H + head;
      bf16x8 qreg[NC];
      load_q<DS>(a, qrow, ds, grp, qreg);
      WaveState<ND> w;
      attend_range<RB, FP8, PACKED, false>(a, sm, pa.kv_indices + k0, pos0, pos1, wave, lane, grp, ds, qreg,
                                           qk_base, pv_base, w);
      const float l_tot = row_total(w.l_run);
      if (fp == lp)
        write_direct(w, l_tot, a.sink ? a.sink[head] : -INFINITY, a.out + qrow * kDim + dcol,
                     (a.lse != nullptr && lse_lane) ? a.lse + qrow : nullptr);
      else
        write_partial_bf16(w, l_tot, (uint16_t *)sb + (size_t)m * kDim + dcol,
                           lse_lane ? sb + (size_t)a.M * kSlotORowFloats + m : nullptr);
    }
    if (fp != lp && !merged) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // release this piece (other XCDs read it)
      __syncthreads();
      uint32_t *ctr = pa.counters + (size_t)g * pa.P + fp;
      if (threadIdx.x == 0) s_arrived = atomicAdd(ctr, 1u);
      __syncthreads();
      // pieces = non-empty partitions of the span: all of them when total >= P,
      // otherwise every partition holds at most one tile, so one per tile
      const int pieces = total >= pa.P ? lp - fp + 1 : tb;
      if (s_arrived == (uint32_t)(pieces - 1)) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // acquire the other pieces
        const int t0_fp = (int)((int64_t)fp * total / pa.P);
        const int fs = 2 * fp + (start == t0_fp ? 0 : 1);
        if (lp - fp < 64)
          merge_pieces_narrow<4, ROWS>(pa, b, g, fp, lp - fp + 1, fs, total);
        else
          merge_pieces<4>(pa, b, g, ROWS, fp, lp, fs, total);
        if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();  // s_arrived is rewritten by the next piece
    }
    start += tb;
  }
}

template <int RB, bool FP8, bool PACKED, bool QF8 = false>
static hipError_t launch_persistent_t(const PersistArgs &a, hipStream_t stream) {
  const int blocks8 = (a.P + 7) / 8;
  const dim3 grid((unsigned)(blocks8 * 8 * a.d.G));
  hipLaunchKernelGGL((persistent_kernel<RB, FP8, PACKED, QF8>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int RB>
static hipError_t launch_persistent_rb(const PersistArgs &a, bool fp8, hipStream_t stream) {
  if constexpr (RB == 8) {
    if (a.d.qk_fp8) return fp8 ? launch_persistent_t<8, true, false, true>(a, stream) : hipErrorInvalidValue;
  } else {
    if (a.d.qk_fp8) return hipErrorInvalidValue;
  }
  if (fp8) return launch_persistent_t<RB, true, false>(a, stream);
  return a.d.packed ? launch_persistent_t<RB, false, true>(a, stream)
                    : launch_persistent_t<RB, false, false>(a, stream);
}

// rb query-row blocks of 16 per workgroup (8: wide waves), a.d.G = M / (16 rb).
hipError_t launch_persistent(const PersistArgs &a, int rb, bool fp8, hipStream_t stream) {
  switch (rb) {
    case 1: return launch_persistent_rb<1>(a, fp8, stream);
    case 2: return launch_persistent_rb<2>(a, fp8, stream);
    case 4: return launch_persistent_rb<4>(a, fp8, stream);
    case 8: return launch_persistent_rb<8>(a, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace smd
