/*
 * smd.h -- C ABI of libsmd, sparse multi-head-latent-attention (MLA) decode
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
 * decode on gfx950", section Design): for every query token t and head h, a
 * list of indices selects rows of one latent KV pool that all heads share.
 * Each selected row is 512 wide: 448 NoPE dims followed by 64 RoPE dims.  The
 * score is one 512-wide dot product s_j = softmax_scale * <q[t,h], k_{i_j}>;
 * an online softmax over the selected rows also counts a per-head sink logit
 * in its denominator; the output is the probability-weighted sum of the same
 * 512-wide rows (V is the row itself).  Invalid indices contribute zero
 * probability.
 *
 *   Z      = sum_{valid j} exp(s_j) + exp(sink_h)
 *   out    = sum_{valid j} exp(s_j) / Z * row_{i_j}          (bf16, [T,H,512])
 *   lse    = ln Z                                            (fp32, [T,H])
 *
 * The work may be split along the index list into FP32 partials plus their
 * log-sum-exp and merged afterwards (aiter page "[ASM][HIP][MLA v4 nm] Split
 * plan helper and persistent decode kernel", Summary part 1: uniform split
 * plan, stage-2 merge that always reduces FP32 partials).
 *
 * Conventions for every entry point:
 *  - Every data pointer is device memory owned by the caller.  The library
 *    allocates no device memory and keeps no state between calls, so the
 *    launches may be captured into a HIP graph.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous; no entry point synchronises the device.
 *  - All arguments are checked on the host before any launch; on a failed
 *    check nothing is launched or written, the call returns a negative
 *    SMD_ERR_* code and smd_last_error() describes the failure.
 *  - Index values are data, not arguments: any index i < 0 or i >= num_rows
 *    is masked (contributes exactly zero), never an error.
 *  - bf16 is the 16-bit brain float format; fp32 is IEEE binary32.
 */
#ifndef SMD_H_
#define SMD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SMD_OK = 0,
  SMD_ERR_INVALID_ARG = -1, /* a pointer, size, stride or alignment is wrong */
  SMD_ERR_UNSUPPORTED = -2, /* a shape outside the supported set            */
  SMD_ERR_WORKSPACE = -3,   /* workspace missing or too small               */
  SMD_ERR_HIP = -4          /* a HIP launch reported an error               */
};

enum {
  SMD_KV_BF16 = 0,          /* rows are 512 bf16 values                                */
  SMD_KV_FP8_E4M3_UE8M0 = 1 /* 448 OCP E4M3FN bytes + 7 UE8M0 codes + 64 bf16 RoPE dims */
};

/* Largest split count of the split-KV entry points. */
#define SMD_MAX_SPLITS 256
/* Largest number of partials one merge (smd_merge_partials) combines, e.g.
 * the splits of several callers' partial decodes of one index list. */
#define SMD_MAX_MERGE_SPLITS 1024
/* Index positions of one split are a multiple of this (except the last). */
#define SMD_SPLIT_ALIGN 64
/* Largest partition count of the persistent entry point. */
#define SMD_MAX_PARTITIONS 16384

/* Message describing this thread's most recent failure ("" if none).  Not an
 * operation of the pages: the error channel of this C ABI.  The pointer stays
 * valid until this thread's next call into the library. */
const char *smd_last_error(void);

/*
 * A latent KV pool: num_rows rows, each 448 NoPE dims then 64 RoPE dims.
 *
 * SMD_KV_BF16:
 *   nope  bf16 [num_rows, >=448], row stride nope_stride ELEMENTS
 *   rope  bf16 [num_rows, >=64],  row stride rope_stride ELEMENTS
 *   scale must be NULL.  A packed [N,512] pool is nope = base,
 *   rope = base + 448, both strides 512.
 * SMD_KV_FP8_E4M3_UE8M0 (vLLM page, Design: UE8M0 codes, one per 64-dim block):
 *   nope  uint8 [num_rows, >=448] OCP E4M3FN, row stride nope_stride BYTES
 *   scale uint8 [num_rows, >=8]: 7 UE8M0 codes + 1 pad byte per row (all
 *         8 bytes are read), row stride scale_stride BYTES, a multiple of 4,
 *         base 4-byte aligned; NoPE dim d decodes to
 *         e4m3(byte_d) * 2^(scale[d/64] - 127)
 *   rope  bf16 [num_rows, >=64], row stride rope_stride ELEMENTS (not scaled)
 * Alignment: nope and rope base addresses and row strides in bytes must be
 * multiples of 16.  The struct itself is read during the call only.
 */
typedef struct smd_kv_pool {
  int32_t dtype; /* SMD_KV_* */
  int32_t reserved;
  int64_t num_rows;
  const void *nope;
  int64_t nope_stride;
  const void *rope;
  int64_t rope_stride;
  const uint8_t *scale;
  int64_t scale_stride;
} smd_kv_pool;

/*
 * Cost model of the host split planner.  The aiter page "[ASM][HIP][MLA v4
 * nm] Split plan helper and persistent decode kernel", Summary part 1, picks
 * the split count from the call's sizes alone by minimising a modelled time
 * that grows with the rounds of workgroups the GPU must run and with the
 * extra partial traffic and merge that each split adds.  This library's
 * formula, all times in picoseconds (the terms are ours; the page prints no
 * formula or coefficients), prices its two kinds of split-KV workgroup:
 *
 * Narrow (SMD_KERNEL_ROWS16 / PAIRS): a workgroup owns rows_per_wg query rows
 * of one index row and one split, and its waves_per_wg waves share the
 * split's positions in steps of 16.
 *
 *   M         = num_heads * q_per_seq,   G = ceil(M / rows_per_wg)
 *   slots     = num_cus * wg_per_cu
 *   wgs(s)    = num_seqs * G * s
 *   waves(s)  = ceil(wgs(s) / slots),    busy(s) = min(wgs(s), slots)
 *   chunk(s)  = roundup(ceil(kv_len / s), 64)   (the split length)
 *   steps(s)  = ceil(ceil(min(chunk(s), kv_len) / 16) / waves_per_wg)
 *   tail(s)   = (s > 1) * (merge + part * num_seqs * M * s)
 *   narrow(s) = waves(s) * (fixed + steps(s) * (step + floor(step_load * busy(s) / slots))) + tail(s)
 *
 * Wide (SMD_KERNEL_WIDE), when wide_rows > 0, M % wide_rows == 0 and the call
 * has one source: a workgroup owns wide_rows query rows and walks the split in
 * tiles of wide_tile positions, one workgroup per CU.
 *
 *   wgs_w(s)  = num_seqs * (M / wide_rows) * s
 *   waves_w(s)= ceil(wgs_w(s) / num_cus),   busy_w(s) = min(wgs_w(s), num_cus)
 *   tiles(s)  = ceil(min(chunk(s), kv_len) / wide_tile)
 *   tile      = wide_tile_fp8 for an fp8 pool, else wide_tile
 *   wide(s)   = waves_w(s) * (wide_fixed + tiles(s) * (tile + floor(wide_tile_load * busy_w(s) / num_cus)))
 *               + tail(s)
 *
 * Caps, each also at most ceil(kv_len / 64): below long_kv indices both
 * families take s <= short_cap; from there on narrow takes s <= long_cap and
 * wide s <= wide_cap (0: long_cap).  All caps are <= SMD_MAX_SPLITS.
 * cost(s) = min of the families that take s; the smallest s of minimum cost
 * wins, and its family is wide when wide(s) is below narrow(s) or narrow does
 * not take s.  (A wide workgroup covers 8 narrow ones' query rows, so the
 * wide family reaches the same grid size with up to 8 times the splits.)
 */
typedef struct smd_plan_model {
  int64_t fixed_ps;     /* per workgroup wave: prologue, wave merge, epilogue */
  int64_t step_ps;      /* per 16-position step of a wave, GPU otherwise idle */
  int64_t step_load_ps; /* added per step with every slot busy (pro rata)     */
  int64_t merge_ps;     /* fixed cost of the stage-2 merge                    */
  int64_t part_ps;      /* per query row and split (partial write + read)     */
  int32_t rows_per_wg;  /* query rows per decode workgroup                    */
  int32_t waves_per_wg; /* waves sharing one workgroup's positions            */
  int32_t wg_per_cu;    /* resident decode workgroups per CU                  */
  int32_t short_cap;    /* split cap when kv_len < long_kv                    */
  int32_t long_cap;     /* split cap otherwise                                */
  int32_t long_kv;      /* threshold between the two caps                     */
  int32_t wide_rows;    /* query rows per wide workgroup; 0: no wide family   */
  int32_t wide_tile;    /* positions per wide tile                            */
  int64_t wide_fixed_ps;     /* per wide workgroup round                      */
  int64_t wide_tile_ps;      /* per wide tile, bf16 pool, GPU otherwise idle  */
  int64_t wide_tile_fp8_ps;  /* per wide tile, fp8 pool, GPU otherwise idle   */
  int64_t wide_tile_load_ps; /* added per wide tile with every CU busy        */
  int32_t wide_cap;          /* wide split cap from long_kv on; 0: long_cap   */
  int32_t reserved;          /* must be 0                                     */
} smd_plan_model;

/*
 * Host split planner: the number of KV splits s in [1, SMD_MAX_SPLITS] for the
 * split-KV decode of `num_seqs` index rows, each shared by q_per_seq tokens
 * of num_heads heads, with kv_len indices per row.  Pure host integer
 * arithmetic with the library's fitted MI355X coefficients; touches no
 * device and depends on nothing but its arguments (aiter page, Summary
 * part 1).  num_cus <= 0 means 256 (MI355X).  Returns s, or a negative
 * SMD_ERR_* code for negative sizes or an unsupported kv_dtype.
 * num_seqs == 0 or kv_len == 0 returns 1.
 */
int smd_plan_num_kv_splits(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq, int32_t kv_len,
                           int32_t kv_dtype, int32_t num_cus);

/* The same planner with explicit coefficients (model must not be NULL). */
int smd_plan_num_kv_splits_model(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq,
                                 int32_t kv_len, int32_t kv_dtype, int32_t num_cus,
                                 const smd_plan_model *model);

/*
 * The planner with the kernel family it priced: returns s like
 * smd_plan_num_kv_splits_model and, when `kernel` is not NULL, stores
 * SMD_KERNEL_WIDE if the wide family won at that s, else SMD_KERNEL_AUTO (a
 * narrow family; smd_decode_kernel_choice names which).  two_source != 0
 * prices the two-source entry points, which have no wide family.  model ==
 * NULL uses the built-in coefficients.  Host only, pure.
 */
int smd_plan_decode(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq, int32_t kv_len,
                    int32_t kv_dtype, int32_t num_cus, int32_t two_source, const smd_plan_model *model,
                    int32_t *kernel);

/* Copy the library's built-in coefficient table into *model. */
int smd_plan_default_model(smd_plan_model *model);

/*
 * Bytes of FP32 partials for num_splits pieces per (token, head): partial_o
 * [num_tokens, num_heads, num_splits, 512] plus partial_lse [num_tokens,
 * num_heads, num_splits], i.e. num_tokens * num_heads * num_splits * 513 * 4.
 * These are the split partials of the aiter page "[ASM][HIP][MLA v4 nm] Split
 * plan helper and persistent decode kernel", Summary part 1 (FP32 partials
 * that a stage-2 merge reduces).  Valid for num_splits in [1,
 * SMD_MAX_MERGE_SPLITS], the range smd_merge_partials accepts (a split-KV
 * call itself takes at most SMD_MAX_SPLITS).  Returns 0 for negative sizes or
 * num_splits outside that range (smd_last_error() says which).
 */
size_t smd_partials_bytes(int32_t num_tokens, int32_t num_heads, int32_t num_splits);

/*
 * Index positions [*begin, *end) of split `split` out of num_splits over a
 * list of kv_len indices: chunk = roundup(ceil(kv_len / num_splits), 64),
 * split r covers [min(r*chunk, kv_len), min((r+1)*chunk, kv_len)).  Trailing
 * splits may be empty.  This is the rule the decode kernels apply.  It is a
 * reading of the aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and
 * persistent decode kernel", Summary part 1, which describes a uniform split
 * of each index list into contiguous ranges without printing the rounding;
 * the 64-position alignment is this library's tile size.  Host only; returns
 * SMD_ERR_INVALID_ARG for NULL outputs or kv_len < 0, num_splits < 1, split
 * outside [0, num_splits).
 */
int smd_split_bounds(int32_t kv_len, int32_t num_splits, int32_t split, int32_t *begin,
                     int32_t *end);

/*
 * Kernel families of the split-KV decode (the results agree to the documented
 * tolerances, not bit for bit).  M = num_heads * q_per_seq.
 *   SMD_KERNEL_ROWS16  16 query rows per workgroup; 8 waves share the split's
 *                      positions and merge their states at the end.
 *   SMD_KERNEL_PAIRS   32 query rows per workgroup, dims split over wave pairs
 *                      (M a multiple of 32).
 *   SMD_KERNEL_WIDE    128 query rows per workgroup, 4 waves of 32 rows on
 *                      32x32 MFMAs sharing every gathered row (M a multiple of
 *                      128, one source).
 * SMD_KERNEL_AUTO picks WIDE when it fits and either the built-in planner
 * model prices it below the narrow kernels at the call's split count (wide(s)
 * < narrow(s) in the model above, with num_seqs = num_tokens / q_per_seq and
 * kv_len = the index count) or that count exceeds the narrow family's cap
 * (short_cap below long_kv indices, long_cap from there on); otherwise PAIRS when M is a multiple of 32 and,
 * with W = (num_tokens / q_per_seq) * num_splits * (M / 32), 7 * ceil(W /
 * 256) < 4 * ceil(2W / 256); otherwise ROWS16.  A named family that does not
 * fit the shape is SMD_ERR_UNSUPPORTED.
 */
enum {
  SMD_KERNEL_AUTO = 0,
  SMD_KERNEL_ROWS16 = 1,
  SMD_KERNEL_PAIRS = 2,
  SMD_KERNEL_WIDE = 3
};

/*
 * How the persistent decode merges a split row group (the split-KV entry
 * points take SMD_MERGE_AUTO only).  Both give the same bits.
 *   SMD_MERGE_AUTO       a piece that finds every other piece of its row
 *                        group arrived (and at most 8 of them) merges straight
 *                        from its registers and writes no partial of its own;
 *                        the rest write FP32 partials and the last to arrive
 *                        merges from the workspace.
 *   SMD_MERGE_WORKSPACE  every piece writes its partial and the last to
 *                        arrive merges from the workspace.
 */
enum {
  SMD_MERGE_AUTO = 0,
  SMD_MERGE_WORKSPACE = 1
};

/* The kernel family a split-KV call with these shapes runs (SMD_KERNEL_ROWS16,
 * SMD_KERNEL_PAIRS or SMD_KERNEL_WIDE): `requested` is options->kernel, and
 * SMD_KERNEL_AUTO applies the rule above.  kv_len is the index count per index
 * row (topk), kv_dtype the pool's SMD_KV_*, two_source != 0 for the two-source
 * entry points.  SMD_ERR_UNSUPPORTED for a named family that does not fit or
 * an unknown kv_dtype, SMD_ERR_INVALID_ARG for bad shapes.  Host only. */
int32_t smd_decode_kernel_choice(int32_t num_tokens, int32_t num_heads, int32_t q_per_seq, int32_t num_splits,
                                 int32_t kv_len, int32_t kv_dtype, int32_t two_source, int32_t requested);

/*
 * How QK runs (options->qk):
 *   SMD_QK_BF16  exact: an fp8 pool's NoPE is dequantised to bf16 (exact,
 *                e4m3 x 2^(code - 127)) and QK runs on bf16 MFMAs.
 *   SMD_QK_FP8   "a8w8" (the persistent decode object of the aiter page
 *                "[ASM][HIP][MLA v4 nm] Split plan helper and persistent
 *                decode kernel", Summary part 2): q_nope is quantised the way
 *                the cache writer quantises a latent row's NoPE (per 64-dim
 *                block, code c = clamp(ceil(log2(amax / 448)) + 127, 0, 254),
 *                each value the E4M3FN byte nearest to x * 2^(127 - c), ties
 *                to even; c = 0 for an all-zero block), and the NoPE part of QK
 *                runs on the block-scaled fp8 MFMA straight from the pool's
 *                bytes and codes.  RoPE, P and PV stay bf16.  The result is the
 *                exact decode's with q_nope replaced by its quantised values,
 *                up to rounding order.  For fp8 pools, one source, M a
 *                multiple of 128: the wide kernel of the split-KV entry points
 *                (with options->kernel SMD_KERNEL_AUTO or SMD_KERNEL_WIDE) and
 *                the persistent decode.  Anything else is SMD_ERR_UNSUPPORTED.
 */
enum {
  SMD_QK_BF16 = 0,
  SMD_QK_FP8 = 1
};

/* Options of the _ex entry points; NULL means all defaults (zero). */
typedef struct smd_decode_options {
  int32_t kernel;      /* SMD_KERNEL_* (SMD_KERNEL_AUTO for the persistent decode) */
  int32_t merge;       /* SMD_MERGE_* */
  int32_t qk;          /* SMD_QK_* */
  int32_t reserved[5]; /* must be zero */
} smd_decode_options;

/*
 * Split-KV sparse MLA decode over dense index rows.
 *
 *  q_nope   bf16 [num_tokens, num_heads, 448], contiguous, 16-byte aligned
 *  q_rope   bf16 [num_tokens, num_heads, 64],  contiguous, 16-byte aligned
 *  num_heads in {16, 32, 64, 128}; q_per_seq in [1, 8]; num_tokens a
 *           multiple of q_per_seq.  Token t uses index row t / q_per_seq
 *           (multi-token prediction positions share their row; no causal
 *           mask among them).
 *  kv       the pool (see smd_kv_pool).
 *  indices  int32 [num_tokens / q_per_seq, >= topk], row stride
 *           indices_stride elements; topk >= 0.
 *  sink     fp32 [num_heads] logits in the scaled score domain, or NULL.
 *  softmax_scale multiplies every dot product.
 *  num_splits in [1, SMD_MAX_SPLITS]; split r covers the positions
 *           smd_split_bounds() gives.
 *  partial_o   fp32 [num_tokens, num_heads, num_splits, 512]
 *  partial_lse fp32 [num_tokens, num_heads, num_splits]
 *           Required when num_splits > 1 or out == NULL.  With out == NULL
 *           they are the result: partial r holds
 *           o_r = sum_{j in r} e^{s_j - lse_r} row_j and
 *           lse_r = ln sum_{j in r} e^{s_j} (no sink); an empty or
 *           all-invalid split holds o_r = 0, lse_r = -inf.  With out they
 *           are scratch for the merge (o_r kept as bf16 in the buffer's
 *           first half; contents afterwards unspecified).
 *  out      bf16 [num_tokens, num_heads, 512] or NULL (partials only)
 *  lse      fp32 [num_tokens, num_heads] or NULL; ln Z including the sink.
 *  With num_splits > 1 and out != NULL the call also launches the merge
 *  (smd_merge_partials' operation, on the bf16 scratch partials).  A row with no valid index gets out = 0 and
 *  lse = sink_h (-inf without a sink).  topk == 0 or num_tokens == 0
 *  launches nothing.
 *  The kernel family is SMD_KERNEL_AUTO's choice (see above).
 */
int smd_sparse_mla_decode(const void *q_nope, const void *q_rope, int32_t num_tokens,
                          int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv,
                          const int32_t *indices, int64_t indices_stride, int32_t topk,
                          const float *sink, float softmax_scale, int32_t num_splits,
                          float *partial_o, float *partial_lse, void *out, float *lse,
                          void *stream);

/* smd_sparse_mla_decode with explicit options (options may be NULL); an
 * unknown kernel or qk value or a non-zero reserved field is
 * SMD_ERR_INVALID_ARG, a qk choice the call cannot take SMD_ERR_UNSUPPORTED. */
int smd_sparse_mla_decode_ex(const void *q_nope, const void *q_rope, int32_t num_tokens,
                             int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv,
                             const int32_t *indices, int64_t indices_stride, int32_t topk,
                             const float *sink, float softmax_scale, int32_t num_splits,
                             float *partial_o, float *partial_lse, void *out, float *lse,
                             const smd_decode_options *options, void *stream);

/*
 * Two-source decode: the compressed main cache and the sliding-window (SWA)
 * cache, each with its own index list, as ordered segments of one softmax
 * (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on
 * gfx950", Design: main and SWA work run in guarded tiles of one kernel).
 *
 *  Index row b has K = k_main + k_swa positions: position p < k_main is
 *  main_indices[b][p], a row of main_kv; position p >= k_main is
 *  swa_indices[b][p - k_main], a row of swa_kv.  Each index is valid
 *  against its own pool's num_rows (anything else contributes nothing).
 *  Every valid row is a term of one softmax with the sink; out, lse and the
 *  split partials are those of smd_sparse_mla_decode over the K positions
 *  (split r covers smd_split_bounds(K, num_splits, r) of them, so a split
 *  may hold main and SWA rows).
 *  main_kv, swa_kv  both required; same dtype, same row strides and (bf16)
 *           the same RoPE placement, else SMD_ERR_UNSUPPORTED.  They may be
 *           the same pool.
 *  main_indices int32 [num_tokens / q_per_seq, >= k_main], row stride
 *           main_stride; swa_indices int32 [.., >= k_swa], row stride
 *           swa_stride.  A list with count 0 may be NULL.
 *  All other arguments, errors and outputs as smd_sparse_mla_decode; the
 *  planner's kv_len for this call is k_main + k_swa.
 */
int smd_sparse_mla_decode_two_source(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                     int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *main_kv,
                                     const int32_t *main_indices, int64_t main_stride, int32_t k_main,
                                     const smd_kv_pool *swa_kv, const int32_t *swa_indices,
                                     int64_t swa_stride, int32_t k_swa, const float *sink,
                                     float softmax_scale, int32_t num_splits, float *partial_o,
                                     float *partial_lse, void *out, float *lse, void *stream);

/* The two-source decode with explicit options (options may be NULL).  With
 * both lists non-empty SMD_KERNEL_WIDE does not fit (one source only). */
int smd_sparse_mla_decode_two_source_ex(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                        int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *main_kv,
                                        const int32_t *main_indices, int64_t main_stride, int32_t k_main,
                                        const smd_kv_pool *swa_kv, const int32_t *swa_indices,
                                        int64_t swa_stride, int32_t k_swa, const float *sink,
                                        float softmax_scale, int32_t num_splits, float *partial_o,
                                        float *partial_lse, void *out, float *lse,
                                        const smd_decode_options *options, void *stream);

/*
 * Allocation-free split-KV decode, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): smd_sparse_mla_decode_ex with the
 * FP32 partials of a split plan kept in a library-owned device array of
 * SMD_NOALLOC_SCRATCH_BYTES per GPU instead of caller buffers.
 *  - out (bf16 [num_tokens, num_heads, 512]) is required; lse may be NULL.
 *  - num_splits == 1 needs no scratch; num_splits > 1 needs
 *    smd_partials_bytes(num_tokens, num_heads, num_splits) <=
 *    SMD_NOALLOC_SCRATCH_BYTES, else SMD_ERR_WORKSPACE (nothing launched).
 *  - The array belongs to the device current at the call; each GPU the
 *    library runs on holds its own copy until the process ends.  The first
 *    call on a device looks its address up (no allocation, no launch).
 *  - Calls that overlap on one GPU (concurrent streams, or threads without
 *    ordering) race on that GPU's array; order them on the GPU.
 * Everything else (arguments, checks, results, options) as
 * smd_sparse_mla_decode_ex.  Calls no hipMalloc / hipFree.
 */
#define SMD_NOALLOC_SCRATCH_BYTES (32u << 20)
int smd_sparse_mla_decode_noalloc(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                  int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv,
                                  const int32_t *indices, int64_t indices_stride, int32_t topk,
                                  const float *sink, float softmax_scale, int32_t num_splits, void *out,
                                  float *lse, const smd_decode_options *options, void *stream);

/*
 * Stage-2 merge (aiter page, Summary part 1: always reduce the FP32
 * partials, even with one split per row):
 *   LSE = ln(sum_r e^{lse_r} + e^{sink_h}),  out = sum_r e^{lse_r - LSE} o_r.
 *  partial_o fp32 [num_tokens, num_heads, num_splits, 512], partial_lse fp32
 *  [num_tokens, num_heads, num_splits]; sink fp32 [num_heads] or NULL;
 *  out bf16 [num_tokens, num_heads, 512] (required); lse fp32
 *  [num_tokens, num_heads] or NULL.  num_splits in [1, SMD_MAX_MERGE_SPLITS].  No finite
 *  term and no sink gives out = 0, lse = -inf.
 */
int smd_merge_partials(const float *partial_o, const float *partial_lse, int32_t num_tokens,
                       int32_t num_heads, int32_t num_splits, const float *sink, void *out,
                       float *lse, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Persistent, graph-safe decode over ragged sequences
 * ---------------------------------------------------------------------------
 * The aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent
 * decode kernel" (Summary, part 2): one launch with a fixed grid; every
 * workgroup computes the split plan inside the kernel from the live
 * kv_indptr; rows held by one partition are written as bf16 directly, split
 * rows write partials into the workspace (o in bf16, lse in fp32: the merged
 * result is bf16) and the workgroup that arrives last merges them; sequences with no index are left unwritten.  (Here the
 * piece that finds all the others arrived merges without writing a partial
 * of its own when the row group has 128 rows; see SMD_MERGE_*.)  Because the
 * plan is read from device memory on every launch, a captured graph stays
 * correct when kv_indptr and kv_indices change between replays.
 *
 * Plan rule: sequence b with tiles_b = ceil(K_b / 64) > 0 tiles of 64 index
 * positions (K_b = kv_indptr[b+1] - kv_indptr[b]) takes tiles_b + 2 plan
 * units, two charged for the fixed cost of a piece and then one per tile; the
 * units of all sequences are concatenated in sequence order, partition p of
 * num_partitions owns units [floor(p*total/P), floor((p+1)*total/P)), and a
 * tile belongs to the partition owning its unit.  The plan descriptor of
 * partition p is (first unit, end unit, first and last sequence with a tile
 * in it, or -1 and -1).
 * The kernel runs P x G workgroups, G = M / R query-row groups of R rows
 * (M = num_heads * q_per_seq; R = 128 when 128 divides M, else 64, 32 or 16,
 * the largest that divides M).
 */

/* P that fills num_cus CUs once: num_cus / G (G as above), at least 1
 * (num_cus <= 0 means 256).  Host only.  Negative SMD_ERR_* on bad shapes. */
int32_t smd_persistent_default_partitions(int32_t num_heads, int32_t q_per_seq, int32_t num_cus);

/* Bytes of workspace the persistent decode needs for these shapes: the plan
 * (16 bytes per partition), arrival counters (4 bytes per partition and
 * 16-row group) and 2 * num_partitions partial slots of M * 1028 bytes (o of
 * M rows as 512 bf16, then the M lse as fp32).
 * Returns 0 for unsupported shapes (smd_last_error says why).  Host only. */
size_t smd_persistent_workspace_bytes(int32_t num_heads, int32_t q_per_seq, int32_t num_partitions);

/* Zero a persistent workspace (an asynchronous memset of `bytes` bytes on
 * `stream`).  Call once after allocating it, outside any graph capture; the
 * kernel returns every counter to zero itself, so later calls (any batch
 * size, any plan) need no further reset. */
int smd_persistent_workspace_reset(void *workspace, size_t bytes, void *stream);

/*
 * Persistent decode.
 *  q_nope   bf16 [num_seqs * q_per_seq, num_heads, 448], contiguous
 *  q_rope   bf16 [num_seqs * q_per_seq, num_heads, 64], contiguous
 *           Tokens b*q_per_seq .. (b+1)*q_per_seq - 1 belong to sequence b
 *           and share its index list (no causal mask among them).
 *  num_seqs >= 0 (0 launches nothing); q_per_seq in [1, 8];
 *  num_heads in {16, 32, 64, 128}.
 *  kv       the pool (see smd_kv_pool).
 *  kv_indptr  int32 device [num_seqs + 1], non-decreasing; sequence b owns
 *           kv_indices[kv_indptr[b] .. kv_indptr[b+1]); kv_indptr[0] may be
 *           > 0.  (A decreasing pair is read as K_b = 0.)
 *  kv_indices int32 device, flat; i < 0 or i >= num_rows is masked.
 *  sink, softmax_scale as for smd_sparse_mla_decode.
 *  workspace  device memory, 256-byte aligned, >= smd_persistent_workspace_bytes
 *           (num_heads, q_per_seq, num_partitions) bytes, zeroed once by
 *           smd_persistent_workspace_reset.  Calls that share a workspace
 *           must be ordered on the GPU (same stream or synchronised); after
 *           a call the plan region holds int32 [num_partitions][4] =
 *           (t0, t1, first sequence, last sequence) of each partition
 *           (-1, -1 for an empty one).
 *  num_partitions in [1, SMD_MAX_PARTITIONS].
 *  out      bf16 [num_seqs * q_per_seq, num_heads, 512] (required)
 *  lse      fp32 [num_seqs * q_per_seq, num_heads] or NULL; ln Z with the sink.
 *  Rows of sequences with K_b = 0 are not written.
 */
int smd_sparse_mla_decode_persistent(const void *q_nope, const void *q_rope, int32_t num_seqs,
                                     int32_t q_per_seq, int32_t num_heads, const smd_kv_pool *kv,
                                     const int32_t *kv_indptr, const int32_t *kv_indices,
                                     const float *sink, float softmax_scale, void *workspace,
                                     size_t workspace_bytes, int32_t num_partitions, void *out,
                                     float *lse, void *stream);

/* The same with options (NULL = defaults): options->kernel must be
 * SMD_KERNEL_AUTO; options->merge selects SMD_MERGE_*. */
int smd_sparse_mla_decode_persistent_ex(const void *q_nope, const void *q_rope, int32_t num_seqs,
                                        int32_t q_per_seq, int32_t num_heads, const smd_kv_pool *kv,
                                        const int32_t *kv_indptr, const int32_t *kv_indices,
                                        const float *sink, float softmax_scale, void *workspace,
                                        size_t workspace_bytes, int32_t num_partitions, void *out,
                                        float *lse, const smd_decode_options *options, void *stream);

/*
 * fp8/UE8M0 KV-cache writer: quantises bf16 latent rows into an fp8 pool
 * (vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on
 * gfx950", Design: writers cap the UE8M0 codes at 254 and canonicalise RoPE
 * NaNs).  For each 64-dim NoPE block b of a row: code c = clamp(ceil(log2(
 * amax / 448)) + 127, 0, 254) with amax the largest |x| of the block (NaN
 * ignored; c = 0 for a block of zeros), stored at scale[row][b]; each value
 * becomes the OCP E4M3FN byte nearest to x * 2^(127 - c), ties to the even
 * mantissa, non-saturating (values past 464 and infinities give NaN with
 * their sign).  scale[row][7] = 0.  RoPE dims are copied, every NaN replaced
 * by 0x7FC0.
 *  kv        bf16 [num_rows, kv_stride]: NoPE dims 0..447, RoPE 448..511;
 *            16-byte aligned, kv_stride >= 512 and a multiple of 8
 *  slots     int32 [num_rows]: the pool row each input row is written to, or
 *            NULL (row r -> pool row r).  Slots outside [0, pool->num_rows)
 *            are skipped; valid slots must be distinct.
 *  pool      an fp8 pool as the decode takes it (nope, rope, scale arrays and
 *            strides); the writer writes into its arrays.
 * Checks as the decode's pool checks; SMD_ERR_UNSUPPORTED for a bf16 pool.
 * num_rows == 0 launches nothing.  Device memory only; no allocation.
 */
int smd_write_kv_fp8(const void *kv, int64_t kv_stride, int32_t num_rows, const int32_t *slots,
                     const smd_kv_pool *pool, void *stream);

/*
 * Dense paged GQA decode: the pa_decode workload of the aiter page "[FlyDSL]
 * [Perf] pa_decode: K/V streaming, MTP query split and sparse split-major on
 * gfx950" (Summary, Performance: paged grouped-query attention with separate
 * K and V rows, MTP query positions and split plans).  The page prints no
 * definition; this is the usual paged decode:
 *
 *  q        bf16 [num_seqs * mtp, num_q_heads, 512], contiguous, 16-byte
 *           aligned; token t = b * mtp + i is MTP position i of sequence b.
 *  k_cache, v_cache  bf16 [num_blocks, page_size, num_kv_heads, 512],
 *           contiguous, 16-byte aligned.  Position p of sequence b is slot
 *           p % page_size of block block_tables[b * block_tables_stride +
 *           p / page_size].
 *  Query head h reads KV head h / (num_q_heads / num_kv_heads).  Supported:
 *  (num_q_heads / num_kv_heads) * mtp == 64 (e.g. GQA 16 x MTP 4, GQA 64 x
 *  MTP 1), page_size a power of two >= 16; otherwise SMD_ERR_UNSUPPORTED.
 *  context_lens int32 [num_seqs] (device), each clamped to [0,
 *           max_context_len]; block_tables_stride >= ceil(max_context_len /
 *           page_size).  The last mtp positions of a context are its MTP
 *           tokens, causal among themselves: token i attends to positions
 *           p < context_lens[b] - (mtp - 1 - i).
 *  A block-table entry outside [0, num_blocks) reads nothing: its positions
 *  are masked (not an error the call reports).
 *  s_p = softmax_scale * <q, k_p>; out = sum_p softmax(s)_p v_p (bf16
 *  [num_seqs * mtp, num_q_heads, 512]); lse = ln sum_p e^{s_p} (fp32, natural
 *  log, no sink); a token with no position gets out = 0, lse = -inf.
 *  num_splits in [1, SMD_MAX_SPLITS]: split r covers positions [r c, (r+1) c)
 *  with c = smd_split_bounds' chunk of max_context_len (a split may span at
 *  most 4095 pages, else SMD_ERR_INVALID_ARG).  partial_o fp32 [tokens,
 *  num_q_heads, s, 512] and partial_lse [tokens, num_q_heads, s] are required
 *  when s > 1 or out == NULL (then they are the result; with out they are
 *  scratch, o kept as bf16, and the call also merges them without a sink).  num_seqs == 0 or
 *  max_context_len == 0 launches nothing.  Returns SMD_OK or SMD_ERR_*.
 */
int smd_paged_decode(const void *q, int32_t num_seqs, int32_t mtp, int32_t num_q_heads, const void *k_cache,
                     const void *v_cache, int64_t num_blocks, int32_t page_size, int32_t num_kv_heads,
                     const int32_t *block_tables, int64_t block_tables_stride, const int32_t *context_lens,
                     int32_t max_context_len, float softmax_scale, int32_t num_splits, float *partial_o,
                     float *partial_lse, void *out, float *lse, void *stream);

/*
 * A split count for smd_paged_decode: enough splits for num_seqs *
 * num_kv_heads * s workgroups to cover num_cus (<= 0: 256) once, capped at 32
 * and ceil(max_context_len / 64), raised (up to SMD_MAX_SPLITS) until a split
 * spans at most 4095 pages.  A heuristic of this library (the page's planner and
 * budgets are not printed).  Host only, pure; SMD_ERR_* on bad sizes.
 */
int32_t smd_paged_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len, int32_t page_size,
                             int32_t num_cus);

#ifdef __cplusplus
}
#endif

#endif /* SMD_H_ */
