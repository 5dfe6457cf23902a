// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/smd.h"

namespace smd {

constexpr int kNope = 448;
constexpr int kRope = 64;
constexpr int kDim = 512;
constexpr int kSplitAlign = 64;

// Arguments of the split-KV decode kernel.  Pointers are device pointers.
struct DecodeArgs {
  const uint16_t *q_nope;  // bf16 [T, H, 448]
  const uint16_t *q_rope;  // bf16 [T, H, 64]
  const uint8_t *kv_nope;  // row base; bf16 or e4m3 bytes
  int64_t nope_stride_b;   // bytes
  const uint8_t *kv_rope;  // bf16 rows
  int64_t rope_stride_b;   // bytes
  const uint8_t *kv_scale; // UE8M0 codes (fp8 pools)
  int64_t scale_stride_b;  // bytes
  int64_t num_rows;
  uint32_t num_rows32;     // min(num_rows, 2^31 - 1): int32 indices cannot exceed it
  int32_t packed;          // bf16 rows with RoPE right after NoPE (rope == nope + 896 B)
  uint32_t row_stride32;   // row stride in bytes when packed (< 2^32)
  const int32_t *indices;
  int64_t indices_stride;  // elements
  int32_t topk;
  int32_t chunk;           // index positions per split (multiple of 64)
  const float *sink;       // [H] or null
  float scale_log2;        // softmax_scale * log2(e)
  int32_t H, qps, M;       // heads, tokens per index row, M = H * qps
  int32_t S;               // splits
  int32_t num_units;       // index rows * S
  int32_t G;               // row groups per index row
  float *part_o;           // [T, H, S, 512] or null
  float *part_lse;         // [T, H, S] or null
  uint16_t *out;           // bf16 [T, H, 512] (direct output when S == 1)
  float *lse;              // [T, H] or null
  int32_t hilo;            // partials are returned to the caller: carry p as bf16 hi + lo
  bool qk_fp8;             // fp8 QK (options qk = SMD_QK_FP8): wide waves over an fp8 pool only
  // Second source (the sliding-window pool and its index list), same format
  // and strides as the first; indices2 null for one source.  Positions
  // [0, k_main) of an index row are entries of `indices`, [k_main, topk)
  // entries of `indices2`.
  const uint8_t *kv2_nope;
  const uint8_t *kv2_rope;
  const uint8_t *kv2_scale;
  uint32_t num_rows2_32;
  const int32_t *indices2;
  int64_t indices2_stride;  // elements
  int32_t k_main;
};

// Launch the split-KV decode: one workgroup per (index row, split, block of
// query rows).  Without pairs a block is 16 rows (a.G = M / 16); with pairs
// (the dim-split kernel, M a multiple of 32) it is 32 rows (a.G = M / 32).
hipError_t launch_decode(const DecodeArgs &a, bool fp8, bool pairs, hipStream_t stream);

// Launch the split-KV decode on the wide waves: one workgroup per (index row,
// split, group of 128 query rows); a.G = M / 128, one source only.
hipError_t launch_decode_wide(const DecodeArgs &a, bool fp8, hipStream_t stream);

// bf16_parts: the partials' o values are bf16 (the decode kernels write
// them so when the partials only feed this merge, i.e. hilo == 0); FP32
// otherwise.
hipError_t launch_merge(const float *part_o, const float *part_lse, int32_t rows, int32_t H,
                        int32_t S, const float *sink, uint16_t *out, float *lse,
                        hipStream_t stream, bool bf16_parts);

// Arguments of the dense paged GQA decode (smd_paged_decode).  Pointers are
// device pointers; caches are bf16 [num_blocks, page, Hkv, 512].
struct PagedArgs {
  const uint16_t *q;             // bf16 [num_seqs * mtp, Hq, 512]
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const int32_t *block_tables;   // [num_seqs, bt_stride]
  int64_t bt_stride;             // elements
  const int32_t *context_lens;   // [num_seqs]
  int64_t num_blocks;
  int32_t num_seqs, mtp, Hq, Hkv, R;  // R = Hq / Hkv; R * mtp == 64
  int32_t page, page_shift;      // page a power of two >= 16
  int32_t max_ctx;               // context lengths are clamped to it
  float scale_log2;
  int32_t S, chunk;              // split count and length (split r: [r chunk, (r+1) chunk))
  float *part_o, *part_lse;      // fp32 [T, Hq, S, 512], [T, Hq, S] when S > 1 or out is null
  uint16_t *out;                 // bf16 [T, Hq, 512] when S == 1
  float *lse;
  int32_t hilo;                  // partials are the result: carry p as bf16 hi + lo
};

hipError_t launch_paged_decode(const PagedArgs &a, hipStream_t stream);

// Arguments of the persistent kernel.  The decode fields carry the queries,
// pool, sink, scale, H, qps, M, G, out and lse (indices, chunk, S and the
// partial pointers are unused).
struct PersistArgs {
  DecodeArgs d;
  const int32_t *kv_indptr;   // [B + 1], non-decreasing; kv_indptr[0] may be > 0
  const int32_t *kv_indices;  // flat index array
  int32_t B;                  // sequences
  int32_t P;                  // partitions
  int32_t *plan;              // [P][4]: t0, t1, first and last sequence
  uint32_t *counters;         // [M / 16][P] arrival counters (row group g, first partition)
  float *slots;               // [2P][M * kSlotRowFloats]: per slot o [M][512] bf16, then lse [M] fp32
  bool reg_merge;             // SMD_MERGE_AUTO: the last piece may merge from its registers
};

// Workspace layout of the persistent kernel (byte offsets, 256-byte aligned).
struct PersistLayout {
  size_t plan_off, ctr_off, slot_off, total;
};
PersistLayout persist_layout(int64_t M, int64_t P);

// A persistent slot per query row: its o as 512 bf16 (256 floats' room) in
// the o region, its lse as one fp32 in the lse region that follows the M rows.
// The partials only feed the merge, whose result is bf16.
constexpr int kSlotORowFloats = 256;
constexpr int kSlotRowFloats = kSlotORowFloats + 1;

// rb in {1, 2, 4, 8} query-row blocks of 16 per workgroup; a.d.G = M / (16 rb).
hipError_t launch_persistent(const PersistArgs &a, int rb, bool fp8, hipStream_t stream);

// Arguments of the fp8/UE8M0 cache writer.  Pointers are device pointers.
struct WriterArgs {
  const uint16_t *kv;      // bf16 [num_rows, kv_stride]
  int64_t kv_stride;       // elements
  int32_t num_rows;
  const int32_t *slots;    // [num_rows] destination pool rows, or null (row r -> r)
  int64_t pool_rows;       // destination rows; slots outside [0, pool_rows) are skipped
  uint8_t *nope;           // e4m3 [pool_rows, nope_stride]
  int64_t nope_stride;     // bytes
  uint8_t *scale;          // codes [pool_rows, scale_stride]
  int64_t scale_stride;    // bytes
  uint16_t *rope;          // bf16 [pool_rows, rope_stride]
  int64_t rope_stride;     // elements
};

hipError_t launch_write_kv_fp8(const WriterArgs &a, hipStream_t stream);

// Error message of the calling thread's last failure (set by every entry point).
void set_error(const char *fmt, ...);

// The host planner's cost terms (plan.cpp; the formula is documented with
// smd_plan_model): the built-in coefficients, the narrow and wide kernels'
// modelled picoseconds at s splits, and whether the wide family is priced.
const smd_plan_model &default_plan_model();
int64_t narrow_cost(const smd_plan_model &m, int64_t num_seqs, int64_t M, int64_t kv_len, int64_t cus, int64_t s);
int64_t wide_cost(const smd_plan_model &m, int64_t num_seqs, int64_t M, int64_t kv_len, int32_t kv_dtype,
                  int64_t cus, int64_t s);
bool wide_priced(const smd_plan_model &m, int64_t M, bool two_source);

// Second source of a two-source decode (the sliding-window pool and its index
// list); null for one source.
struct SecondSource {
  const smd_kv_pool *kv;
  const int32_t *indices;
  int64_t indices_stride;
  int32_t count;
};

// The split-KV decode behind the public entry points (checks, kernel choice,
// decode launch and, for s > 1 with out, the merge); fn names the caller in
// error messages.
int decode_impl(const char *fn, const void *q_nope, const void *q_rope, int32_t num_tokens, int32_t num_heads,
                int32_t q_per_seq, const smd_kv_pool *kv, const int32_t *indices, int64_t indices_stride,
                int32_t topk, const SecondSource *two, const float *sink, float softmax_scale, int32_t num_splits,
                float *partial_o, float *partial_lse, void *out, float *lse, const smd_decode_options *opt,
                void *stream);

}  // namespace smd
