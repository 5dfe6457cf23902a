// C ABI entry points of libsmd: argument checks on the host, then kernel
// launches on the caller's stream.  Nothing is allocated and nothing is
// launched when a check fails.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/smd.h"
#include "smd_internal.h"

namespace smd {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static bool heads_ok(int32_t h) { return h == 16 || h == 32 || h == 64 || h == 128; }

// Checks shared by the decode entry points.  On success fills the pool part of `a`.
static int check_pool(const char *fn, const smd_kv_pool *kv, DecodeArgs &a) {
  if (!kv) {
    set_error("%s: kv pool is NULL", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (kv->dtype != SMD_KV_BF16 && kv->dtype != SMD_KV_FP8_E4M3_UE8M0) {
    set_error("%s: unknown kv dtype %d", fn, kv->dtype);
    return SMD_ERR_UNSUPPORTED;
  }
  if (kv->num_rows < 0) {
    set_error("%s: negative num_rows", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (!kv->nope || !kv->rope) {
    set_error("%s: kv nope/rope pointer is NULL", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (!aligned16(kv->nope) || !aligned16(kv->rope)) {
    set_error("%s: kv nope/rope base must be 16-byte aligned", fn);
    return SMD_ERR_INVALID_ARG;
  }
  const bool fp8 = kv->dtype == SMD_KV_FP8_E4M3_UE8M0;
  const int64_t nope_b = fp8 ? kv->nope_stride : kv->nope_stride * 2;
  const int64_t rope_b = kv->rope_stride * 2;
  if (kv->nope_stride < kNope || kv->rope_stride < kRope) {
    set_error("%s: kv row strides (%lld, %lld) below the row widths (448, 64)", fn,
              (long long)kv->nope_stride, (long long)kv->rope_stride);
    return SMD_ERR_INVALID_ARG;
  }
  if ((nope_b & 15) || (rope_b & 15)) {
    set_error("%s: kv row strides must be multiples of 16 bytes", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (fp8) {
    if (!kv->scale) {
      set_error("%s: fp8 pool needs a scale (UE8M0 code) array", fn);
      return SMD_ERR_INVALID_ARG;
    }
    if (kv->scale_stride < 8 || (kv->scale_stride & 3) || ((uintptr_t)kv->scale & 3)) {
      set_error("%s: scale rows must hold 8 bytes (7 codes + pad) with a stride that is a multiple "
                "of 4 and a 4-byte aligned base (stride %lld)", fn, (long long)kv->scale_stride);
      return SMD_ERR_INVALID_ARG;
    }
  } else if (kv->scale) {
    set_error("%s: bf16 pool must not pass a scale array", fn);
    return SMD_ERR_INVALID_ARG;
  }
  a.kv_nope = (const uint8_t *)kv->nope;
  a.nope_stride_b = nope_b;
  a.kv_rope = (const uint8_t *)kv->rope;
  a.rope_stride_b = rope_b;
  a.kv_scale = kv->scale;
  a.scale_stride_b = kv->scale_stride;
  a.num_rows = kv->num_rows;
  a.num_rows32 = (uint32_t)(kv->num_rows < INT32_MAX ? kv->num_rows : INT32_MAX);
  a.packed = !fp8 && (const uint8_t *)kv->rope == (const uint8_t *)kv->nope + 2 * kNope && nope_b == rope_b &&
             nope_b < (int64_t)UINT32_MAX;
  a.row_stride32 = a.packed ? (uint32_t)nope_b : 0u;
  return SMD_OK;
}

// The split-KV kernel families (include/smd.h, SMD_KERNEL_*).
enum Kern { kKernRows16 = 1, kKernPairs = 2, kKernWide = 3 };

// The dim-split kernel (32 query rows per workgroup) moves less through LDS
// per unit of work but has half as many workgroups, each taking about 7/4 of
// the time of a 16-row one (measured on full GPUs).  With one workgroup per
// CU on 256 CUs it wins when 7/4 x its rounds of workgroups is below the
// 16-row kernel's rounds: a full grid, and not a grid that spills a small
// last round.
static bool pairs_pay(int32_t M, int64_t units) {
  if (M % 32 != 0) return false;
  const int64_t w = units * (M / 32);
  const int64_t rounds_pairs = (w + 255) / 256, rounds_rows = (2 * w + 255) / 256;
  return 7 * rounds_pairs < 4 * rounds_rows;
}

// The wide kernel (128 query rows per workgroup on 32x32 MFMAs) shares each
// gathered row among 128 query rows; it needs M % 128 == 0 and one source.
// It runs when the planner's cost model prices it below the narrow kernels at
// the call's split count: it pays once its grid fills the GPU and each
// workgroup has enough tiles to hide its fixed cost.
constexpr int32_t kWideRowsPerGroup = 128;
static bool wide_fits(int32_t M, bool two) { return M % kWideRowsPerGroup == 0 && !two; }

// Kernel of a split-KV call of `rows` index rows, s splits and kv_len indices
// per row: the caller's choice when it names one (checked against the shape),
// else the rule above.  Returns 0 for an impossible choice.
static int pick_kernel(int32_t requested, int32_t M, int64_t rows, int32_t s, int64_t kv_len, int32_t kv_dtype,
                       bool two) {
  switch (requested) {
    case SMD_KERNEL_ROWS16: return kKernRows16;
    case SMD_KERNEL_PAIRS: return M % 32 == 0 ? kKernPairs : 0;
    case SMD_KERNEL_WIDE: return wide_fits(M, two) ? kKernWide : 0;
    default: break;
  }
  const smd_plan_model &pm = default_plan_model();
  static_assert(kWideRowsPerGroup == 128, "the planner's wide_rows");
  // the planner prices the narrow family up to its cap only: beyond it a
  // split count is a wide plan
  const int64_t narrow_cap = kv_len < pm.long_kv ? pm.short_cap : pm.long_cap;
  if (wide_fits(M, two) && rows > 0 && kv_len > 0 && wide_priced(pm, M, two) &&
      (s > narrow_cap ||
       wide_cost(pm, rows, M, kv_len, kv_dtype, 256, s) < narrow_cost(pm, rows, M, kv_len, 256, s)))
    return kKernWide;
  return pairs_pay(M, rows * s) ? kKernPairs : kKernRows16;
}

}  // namespace smd

using namespace smd;

extern "C" int32_t smd_decode_kernel_choice(int32_t num_tokens, int32_t num_heads, int32_t q_per_seq,
                                            int32_t num_splits, int32_t kv_len, int32_t kv_dtype,
                                            int32_t two_source, int32_t requested) {
  static const char *fn = "smd_decode_kernel_choice";
  g_err[0] = 0;
  if (num_tokens < 0 || num_heads <= 0 || q_per_seq < 1 || num_splits < 1 || kv_len < 0 ||
      num_tokens % q_per_seq != 0 || requested < SMD_KERNEL_AUTO || requested > SMD_KERNEL_WIDE) {
    set_error("%s: bad shapes or kernel choice", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (kv_dtype != SMD_KV_BF16 && kv_dtype != SMD_KV_FP8_E4M3_UE8M0) {
    set_error("%s: unknown kv_dtype %d", fn, kv_dtype);
    return SMD_ERR_UNSUPPORTED;
  }
  const int32_t M = num_heads * q_per_seq;
  const int k = pick_kernel(requested, M, num_tokens / q_per_seq, num_splits, kv_len, kv_dtype, two_source != 0);
  if (k == 0) {
    set_error("%s: kernel choice %d does not fit M = %d query rows per index row", fn, requested, M);
    return SMD_ERR_UNSUPPORTED;
  }
  return k == kKernWide ? SMD_KERNEL_WIDE : k == kKernPairs ? SMD_KERNEL_PAIRS : SMD_KERNEL_ROWS16;
}

extern "C" const char *smd_last_error(void) { return g_err; }

namespace smd {
int decode_impl(const char *fn, const void *q_nope, const void *q_rope, int32_t num_tokens,
                       int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv, const int32_t *indices,
                       int64_t indices_stride, int32_t topk, const SecondSource *two, const float *sink,
                       float softmax_scale, int32_t num_splits, float *partial_o, float *partial_lse, void *out,
                       float *lse, const smd_decode_options *opt, void *stream) {
  g_err[0] = 0;
  if (opt != nullptr) {
    if (opt->kernel < SMD_KERNEL_AUTO || opt->kernel > SMD_KERNEL_WIDE) {
      set_error("%s: unknown kernel choice %d", fn, opt->kernel);
      return SMD_ERR_INVALID_ARG;
    }
    if (opt->merge != SMD_MERGE_AUTO) {
      set_error("%s: options.merge applies to the persistent decode only", fn);
      return SMD_ERR_INVALID_ARG;
    }
    if (opt->qk != SMD_QK_BF16 && opt->qk != SMD_QK_FP8) {
      set_error("%s: unknown qk choice %d", fn, opt->qk);
      return SMD_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 5; ++i) {
      if (opt->reserved[i] != 0) {
        set_error("%s: options.reserved must be zero", fn);
        return SMD_ERR_INVALID_ARG;
      }
    }
  }
  const bool qk_fp8 = opt != nullptr && opt->qk == SMD_QK_FP8;
  if (num_tokens < 0 || topk < 0 || indices_stride < 0 ||
      (two && (two->count < 0 || two->indices_stride < 0))) {
    set_error("%s: negative size (num_tokens=%d counts=%d,%d strides=%lld,%lld)", fn, num_tokens, topk,
              two ? two->count : 0, (long long)indices_stride, (long long)(two ? two->indices_stride : 0));
    return SMD_ERR_INVALID_ARG;
  }
  if (!heads_ok(num_heads)) {
    set_error("%s: num_heads=%d not in {16,32,64,128}", fn, num_heads);
    return SMD_ERR_UNSUPPORTED;
  }
  if (q_per_seq < 1 || q_per_seq > 8) {
    set_error("%s: q_per_seq=%d not in [1,8]", fn, q_per_seq);
    return SMD_ERR_UNSUPPORTED;
  }
  if (num_tokens % q_per_seq) {
    set_error("%s: num_tokens=%d is not a multiple of q_per_seq=%d", fn, num_tokens, q_per_seq);
    return SMD_ERR_INVALID_ARG;
  }
  if (num_splits < 1 || num_splits > SMD_MAX_SPLITS) {
    set_error("%s: num_splits=%d not in [1,%d]", fn, num_splits, SMD_MAX_SPLITS);
    return SMD_ERR_INVALID_ARG;
  }
  if (!isfinite(softmax_scale)) {
    set_error("%s: softmax_scale is not finite", fn);
    return SMD_ERR_INVALID_ARG;
  }
  DecodeArgs a = {};
  int rc = check_pool(fn, kv, a);
  if (rc) return rc;
  const int32_t k2 = two ? two->count : 0;
  if (two) {
    DecodeArgs b = {};
    rc = check_pool(fn, two->kv, b);
    if (rc) return rc;
    if (two->kv->dtype != kv->dtype || b.nope_stride_b != a.nope_stride_b || b.rope_stride_b != a.rope_stride_b ||
        b.scale_stride_b != a.scale_stride_b || b.packed != a.packed) {
      set_error("%s: the main and SWA pools must have the same dtype, row strides and RoPE placement", fn);
      return SMD_ERR_UNSUPPORTED;
    }
    if ((int64_t)topk + k2 > INT32_MAX) {
      set_error("%s: main + SWA index counts exceed 2^31 - 1", fn);
      return SMD_ERR_INVALID_ARG;
    }
    a.kv2_nope = b.kv_nope;
    a.kv2_rope = b.kv_rope;
    a.kv2_scale = b.kv_scale;
    a.num_rows2_32 = b.num_rows32;
  }
  const int32_t rows = num_tokens / q_per_seq;
  if (num_tokens > 0 && topk + k2 > 0) {
    if (!q_nope || !q_rope || (topk > 0 && !indices) || (k2 > 0 && !two->indices)) {
      set_error("%s: q_nope, q_rope and the index lists are required", fn);
      return SMD_ERR_INVALID_ARG;
    }
    if (!aligned16(q_nope) || !aligned16(q_rope)) {
      set_error("%s: q_nope/q_rope must be 16-byte aligned", fn);
      return SMD_ERR_INVALID_ARG;
    }
    if (topk > 0 && indices_stride < topk && rows > 1) {
      set_error("%s: indices_stride=%lld below its count %d", fn, (long long)indices_stride, topk);
      return SMD_ERR_INVALID_ARG;
    }
    if (k2 > 0 && two->indices_stride < k2 && rows > 1) {
      set_error("%s: swa indices stride=%lld below k_swa=%d", fn, (long long)two->indices_stride, k2);
      return SMD_ERR_INVALID_ARG;
    }
  }
  const bool need_partials = num_splits > 1 || out == nullptr;
  if (need_partials && (!partial_o || !partial_lse)) {
    set_error("%s: partial_o and partial_lse are required when num_splits > 1 or out is NULL", fn);
    return SMD_ERR_WORKSPACE;
  }
  if (partial_o && !aligned16(partial_o)) {
    set_error("%s: partial_o must be 16-byte aligned", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (out && !aligned16(out)) {
    set_error("%s: out must be 16-byte aligned", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (num_tokens == 0 || topk + k2 == 0) return SMD_OK;

  const int32_t K = topk + k2;
  const int32_t M = num_heads * q_per_seq;
  // chunk = roundup(ceil(K / s), 64), as smd_split_bounds.
  const int64_t per = ((int64_t)K + num_splits - 1) / num_splits;
  const int64_t chunk = (per + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
  a.q_nope = (const uint16_t *)q_nope;
  a.q_rope = (const uint16_t *)q_rope;
  if (k2 == 0 || topk == 0) {  // one list holds every position: a one-source launch over its pool
    if (topk == 0) {
      DecodeArgs b = {};
      check_pool(fn, two->kv, b);  // passed above
      a.kv_nope = b.kv_nope;
      a.kv_rope = b.kv_rope;
      a.kv_scale = b.kv_scale;
      a.num_rows = b.num_rows;
      a.num_rows32 = b.num_rows32;
      indices = two->indices;
      indices_stride = two->indices_stride;
    }
    a.indices2 = nullptr;
  } else {
    a.indices2 = two->indices;
    a.indices2_stride = two->indices_stride;
  }
  a.indices = indices;
  a.indices_stride = indices_stride;
  a.k_main = topk;
  a.topk = K;
  a.chunk = (int32_t)(chunk < INT32_MAX ? chunk : INT32_MAX);
  a.sink = sink;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.H = num_heads;
  a.qps = q_per_seq;
  a.M = M;
  a.S = num_splits;
  a.num_units = rows * num_splits;
  const bool fp8 = kv->dtype == SMD_KV_FP8_E4M3_UE8M0;
  if (qk_fp8) {  // the fp8 QK exists on the wide kernel over one fp8 source
    if (!fp8 || two != nullptr || !wide_fits(M, false) ||
        (opt->kernel != SMD_KERNEL_AUTO && opt->kernel != SMD_KERNEL_WIDE)) {
      set_error("%s: qk = SMD_QK_FP8 needs an fp8 pool, one source, M = %d a multiple of 128 and the wide "
                "kernel (kernel choice %d)", fn, M, opt->kernel);
      return SMD_ERR_UNSUPPORTED;
    }
  }
  const int kern = qk_fp8 ? kKernWide
                          : pick_kernel(opt ? opt->kernel : SMD_KERNEL_AUTO, M, rows, num_splits, K, kv->dtype,
                                        a.indices2 != nullptr);
  if (kern == 0) {
    set_error("%s: kernel choice %d does not fit M = %d query rows per index row%s", fn, opt->kernel, M,
              a.indices2 ? " with two sources" : "");
    return SMD_ERR_UNSUPPORTED;
  }
  a.G = M / (kern == kKernWide ? 128 : (kern == kKernPairs ? 32 : 16));
  a.part_o = need_partials ? partial_o : nullptr;
  a.part_lse = need_partials ? partial_lse : nullptr;
  a.out = need_partials ? nullptr : (uint16_t *)out;
  a.lse = need_partials ? nullptr : lse;
  a.hilo = out == nullptr;  // FP32 partials are the result only without out
  a.qk_fp8 = qk_fp8;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = kern == kKernWide ? launch_decode_wide(a, fp8, st) : launch_decode(a, fp8, kern == kKernPairs, st);
  if (e != hipSuccess) {
    set_error("%s: decode launch failed: %s", fn, hipGetErrorString(e));
    return SMD_ERR_HIP;
  }
  if (need_partials && out) {
    e = launch_merge(partial_o, partial_lse, num_tokens * num_heads, num_heads, num_splits, sink,
                     (uint16_t *)out, lse, st, /*bf16_parts=*/true);
    if (e != hipSuccess) {
      set_error("%s: merge launch failed: %s", fn, hipGetErrorString(e));
      return SMD_ERR_HIP;
    }
  }
  return SMD_OK;
}

}  // namespace smd

extern "C" int smd_sparse_mla_decode_ex(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                        int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv,
                                        const int32_t *indices, int64_t indices_stride, int32_t topk,
                                        const float *sink, float softmax_scale, int32_t num_splits,
                                        float *partial_o, float *partial_lse, void *out, float *lse,
                                        const smd_decode_options *options, void *stream) {
  return decode_impl("smd_sparse_mla_decode", q_nope, q_rope, num_tokens, num_heads, q_per_seq, kv, indices,
                     indices_stride, topk, nullptr, sink, softmax_scale, num_splits, partial_o, partial_lse, out,
                     lse, options, stream);
}

extern "C" int smd_sparse_mla_decode(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                     int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv,
                                     const int32_t *indices, int64_t indices_stride, int32_t topk,
                                     const float *sink, float softmax_scale, int32_t num_splits,
                                     float *partial_o, float *partial_lse, void *out, float *lse,
                                     void *stream) {
  return smd_sparse_mla_decode_ex(q_nope, q_rope, num_tokens, num_heads, q_per_seq, kv, indices, indices_stride,
                                  topk, sink, softmax_scale, num_splits, partial_o, partial_lse, out, lse, nullptr,
                                  stream);
}

extern "C" int smd_sparse_mla_decode_two_source_ex(
    const void *q_nope, const void *q_rope, int32_t num_tokens, int32_t num_heads, int32_t q_per_seq,
    const smd_kv_pool *main_kv, const int32_t *main_indices, int64_t main_stride, int32_t k_main,
    const smd_kv_pool *swa_kv, const int32_t *swa_indices, int64_t swa_stride, int32_t k_swa, const float *sink,
    float softmax_scale, int32_t num_splits, float *partial_o, float *partial_lse, void *out, float *lse,
    const smd_decode_options *options, void *stream) {
  const SecondSource two{swa_kv, swa_indices, swa_stride, k_swa};
  return decode_impl("smd_sparse_mla_decode_two_source", q_nope, q_rope, num_tokens, num_heads, q_per_seq, main_kv,
                     main_indices, main_stride, k_main, &two, sink, softmax_scale, num_splits, partial_o,
                     partial_lse, out, lse, options, stream);
}

extern "C" int smd_sparse_mla_decode_two_source(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                                int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *main_kv,
                                                const int32_t *main_indices, int64_t main_stride, int32_t k_main,
                                                const smd_kv_pool *swa_kv, const int32_t *swa_indices,
                                                int64_t swa_stride, int32_t k_swa, const float *sink,
                                                float softmax_scale, int32_t num_splits, float *partial_o,
                                                float *partial_lse, void *out, float *lse, void *stream) {
  return smd_sparse_mla_decode_two_source_ex(q_nope, q_rope, num_tokens, num_heads, q_per_seq, main_kv,
                                             main_indices, main_stride, k_main, swa_kv, swa_indices, swa_stride,
                                             k_swa, sink, softmax_scale, num_splits, partial_o, partial_lse, out,
                                             lse, nullptr, stream);
}

extern "C" int smd_merge_partials(const float *partial_o, const float *partial_lse,
                                  int32_t num_tokens, int32_t num_heads, int32_t num_splits,
                                  const float *sink, void *out, float *lse, void *stream) {
  static const char *fn = "smd_merge_partials";
  g_err[0] = 0;
  if (num_tokens < 0 || num_heads < 1) {
    set_error("%s: invalid num_tokens=%d num_heads=%d", fn, num_tokens, num_heads);
    return SMD_ERR_INVALID_ARG;
  }
  if (num_splits < 1 || num_splits > SMD_MAX_MERGE_SPLITS) {
    set_error("%s: num_splits=%d not in [1,%d]", fn, num_splits, SMD_MAX_MERGE_SPLITS);
    return SMD_ERR_INVALID_ARG;
  }
  if (num_tokens == 0) return SMD_OK;
  if (!partial_o || !partial_lse || !out) {
    set_error("%s: partial_o, partial_lse and out are required", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (!aligned16(partial_o) || !aligned16(out)) {
    set_error("%s: partial_o and out must be 16-byte aligned", fn);
    return SMD_ERR_INVALID_ARG;
  }
  hipError_t e = launch_merge(partial_o, partial_lse, num_tokens * num_heads, num_heads, num_splits,
                              sink, (uint16_t *)out, lse, (hipStream_t)stream, /*bf16_parts=*/false);
  if (e != hipSuccess) {
    set_error("%s: merge launch failed: %s", fn, hipGetErrorString(e));
    return SMD_ERR_HIP;
  }
  return SMD_OK;
}

// ----------------------------------------------------------------------------
// persistent, graph-safe variant
// ----------------------------------------------------------------------------
// Row blocks per workgroup of the persistent kernel: the largest of 8, 4, 2, 1
// that divides M / 16, so the 16*rb-row groups cover every query row.
static int persist_rb(int32_t M) { return M % 128 == 0 ? 8 : (M % 64 == 0 ? 4 : (M % 32 == 0 ? 2 : 1)); }
static int32_t persist_groups(int32_t M) { return M / (16 * persist_rb(M)); }

extern "C" int32_t smd_persistent_default_partitions(int32_t num_heads, int32_t q_per_seq, int32_t num_cus) {
  g_err[0] = 0;
  if (!heads_ok(num_heads) || q_per_seq < 1 || q_per_seq > 8) {
    set_error("smd_persistent_default_partitions: unsupported num_heads=%d / q_per_seq=%d", num_heads, q_per_seq);
    return SMD_ERR_UNSUPPORTED;
  }
  const int32_t cus = num_cus > 0 ? num_cus : 256;
  const int32_t M = num_heads * q_per_seq;
  const int32_t groups = persist_groups(M);
  const int32_t p = cus / groups;
  return p < 1 ? 1 : (p > SMD_MAX_PARTITIONS ? SMD_MAX_PARTITIONS : p);
}

extern "C" size_t smd_persistent_workspace_bytes(int32_t num_heads, int32_t q_per_seq, int32_t num_partitions) {
  g_err[0] = 0;
  if (!heads_ok(num_heads) || q_per_seq < 1 || q_per_seq > 8 || num_partitions < 1 ||
      num_partitions > SMD_MAX_PARTITIONS) {
    set_error("smd_persistent_workspace_bytes: unsupported num_heads=%d q_per_seq=%d num_partitions=%d",
              num_heads, q_per_seq, num_partitions);
    return 0;
  }
  return persist_layout((int64_t)num_heads * q_per_seq, num_partitions).total;
}

extern "C" int smd_persistent_workspace_reset(void *workspace, size_t bytes, void *stream) {
  static const char *fn = "smd_persistent_workspace_reset";
  g_err[0] = 0;
  if (!workspace || bytes == 0) {
    set_error("%s: workspace is NULL or empty", fn);
    return SMD_ERR_INVALID_ARG;
  }
  hipError_t e = hipMemsetAsync(workspace, 0, bytes, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("%s: hipMemsetAsync failed: %s", fn, hipGetErrorString(e));
    return SMD_ERR_HIP;
  }
  return SMD_OK;
}

extern "C" int smd_sparse_mla_decode_persistent_ex(const void *q_nope, const void *q_rope, int32_t num_seqs,
                                                   int32_t q_per_seq, int32_t num_heads, const smd_kv_pool *kv,
                                                   const int32_t *kv_indptr, const int32_t *kv_indices,
                                                   const float *sink, float softmax_scale, void *workspace,
                                                   size_t workspace_bytes, int32_t num_partitions, void *out,
                                                   float *lse, const smd_decode_options *opt, void *stream) {
  static const char *fn = "smd_sparse_mla_decode_persistent";
  g_err[0] = 0;
  if (opt != nullptr) {
    if (opt->kernel != SMD_KERNEL_AUTO) {
      set_error("%s: the persistent decode takes SMD_KERNEL_AUTO only (got %d)", fn, opt->kernel);
      return SMD_ERR_INVALID_ARG;
    }
    if (opt->merge != SMD_MERGE_AUTO && opt->merge != SMD_MERGE_WORKSPACE) {
      set_error("%s: unknown merge choice %d", fn, opt->merge);
      return SMD_ERR_INVALID_ARG;
    }
    if (opt->qk != SMD_QK_BF16 && opt->qk != SMD_QK_FP8) {
      set_error("%s: unknown qk choice %d", fn, opt->qk);
      return SMD_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 5; ++i) {
      if (opt->reserved[i] != 0) {
        set_error("%s: options.reserved must be zero", fn);
        return SMD_ERR_INVALID_ARG;
      }
    }
  }
  if (num_seqs < 0) {
    set_error("%s: negative num_seqs=%d", fn, num_seqs);
    return SMD_ERR_INVALID_ARG;
  }
  if (!heads_ok(num_heads)) {
    set_error("%s: num_heads=%d not in {16,32,64,128}", fn, num_heads);
    return SMD_ERR_UNSUPPORTED;
  }
  if (q_per_seq < 1 || q_per_seq > 8) {
    set_error("%s: q_per_seq=%d not in [1,8]", fn, q_per_seq);
    return SMD_ERR_UNSUPPORTED;
  }
  if (num_partitions < 1 || num_partitions > SMD_MAX_PARTITIONS) {
    set_error("%s: num_partitions=%d not in [1,%d]", fn, num_partitions, SMD_MAX_PARTITIONS);
    return SMD_ERR_INVALID_ARG;
  }
  if (!isfinite(softmax_scale)) {
    set_error("%s: softmax_scale is not finite", fn);
    return SMD_ERR_INVALID_ARG;
  }
  DecodeArgs a = {};
  int rc = check_pool(fn, kv, a);
  if (rc) return rc;
  const int32_t M = num_heads * q_per_seq;
  const PersistLayout lay = persist_layout(M, num_partitions);
  if (!workspace || ((uintptr_t)workspace & 255u)) {
    set_error("%s: workspace must be a non-NULL 256-byte aligned device buffer", fn);
    return SMD_ERR_WORKSPACE;
  }
  if (workspace_bytes < lay.total) {
    set_error("%s: workspace of %zu bytes is below the %zu bytes needed for num_heads=%d q_per_seq=%d "
              "num_partitions=%d", fn, workspace_bytes, lay.total, num_heads, q_per_seq, num_partitions);
    return SMD_ERR_WORKSPACE;
  }
  if (num_seqs > 0) {
    if (!q_nope || !q_rope || !kv_indptr || !kv_indices || !out) {
      set_error("%s: q_nope, q_rope, kv_indptr, kv_indices and out are required", fn);
      return SMD_ERR_INVALID_ARG;
    }
    if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(out)) {
      set_error("%s: q_nope, q_rope and out must be 16-byte aligned", fn);
      return SMD_ERR_INVALID_ARG;
    }
    if (((uintptr_t)kv_indptr & 3) || ((uintptr_t)kv_indices & 3) || (lse && ((uintptr_t)lse & 3))) {
      set_error("%s: kv_indptr, kv_indices and lse must be 4-byte aligned", fn);
      return SMD_ERR_INVALID_ARG;
    }
  }
  if (num_seqs == 0) return SMD_OK;

  const int rb = persist_rb(M);
  const bool qk_fp8 = opt != nullptr && opt->qk == SMD_QK_FP8;
  if (qk_fp8 && (kv->dtype != SMD_KV_FP8_E4M3_UE8M0 || rb != 8)) {
    set_error("%s: qk = SMD_QK_FP8 needs an fp8 pool and M = %d a multiple of 128", fn, M);
    return SMD_ERR_UNSUPPORTED;
  }
  PersistArgs pa = {};
  a.q_nope = (const uint16_t *)q_nope;
  a.q_rope = (const uint16_t *)q_rope;
  a.sink = sink;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.H = num_heads;
  a.qps = q_per_seq;
  a.M = M;
  a.S = 1;
  a.G = persist_groups(M);
  a.out = (uint16_t *)out;
  a.lse = lse;
  a.qk_fp8 = qk_fp8;
  pa.d = a;
  pa.kv_indptr = kv_indptr;
  pa.kv_indices = kv_indices;
  pa.B = num_seqs;
  pa.P = num_partitions;
  uint8_t *ws = (uint8_t *)workspace;
  pa.plan = (int32_t *)(ws + lay.plan_off);
  pa.counters = (uint32_t *)(ws + lay.ctr_off);
  pa.slots = (float *)(ws + lay.slot_off);
  pa.reg_merge = opt == nullptr || opt->merge == SMD_MERGE_AUTO;
  hipError_t e = launch_persistent(pa, rb, kv->dtype == SMD_KV_FP8_E4M3_UE8M0, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", fn, hipGetErrorString(e));
    return SMD_ERR_HIP;
  }
  return SMD_OK;
}

extern "C" int smd_sparse_mla_decode_persistent(const void *q_nope, const void *q_rope, int32_t num_seqs,
                                                int32_t q_per_seq, int32_t num_heads, const smd_kv_pool *kv,
                                                const int32_t *kv_indptr, const int32_t *kv_indices,
                                                const float *sink, float softmax_scale, void *workspace,
                                                size_t workspace_bytes, int32_t num_partitions, void *out,
                                                float *lse, void *stream) {
  return smd_sparse_mla_decode_persistent_ex(q_nope, q_rope, num_seqs, q_per_seq, num_heads, kv, kv_indptr,
                                             kv_indices, sink, softmax_scale, workspace, workspace_bytes,
                                             num_partitions, out, lse, nullptr, stream);
}

// ----------------------------------------------------------------------------
// fp8/UE8M0 cache writer
// ----------------------------------------------------------------------------
extern "C" int smd_write_kv_fp8(const void *kv, int64_t kv_stride, int32_t num_rows, const int32_t *slots,
                                const smd_kv_pool *pool, void *stream) {
  static const char *fn = "smd_write_kv_fp8";
  g_err[0] = 0;
  if (num_rows < 0) {
    set_error("%s: negative num_rows", fn);
    return SMD_ERR_INVALID_ARG;
  }
  DecodeArgs d = {};
  int rc = check_pool(fn, pool, d);
  if (rc) return rc;
  if (pool->dtype != SMD_KV_FP8_E4M3_UE8M0) {
    set_error("%s: the destination pool must be fp8 (SMD_KV_FP8_E4M3_UE8M0)", fn);
    return SMD_ERR_UNSUPPORTED;
  }
  if (num_rows == 0) return SMD_OK;
  if (!kv || !aligned16(kv) || kv_stride < kDim || ((kv_stride * 2) & 15)) {
    set_error("%s: kv must be non-NULL bf16 rows, 16-byte aligned, with a stride >= 512 elements and a "
              "multiple of 8 (stride %lld)", fn, (long long)kv_stride);
    return SMD_ERR_INVALID_ARG;
  }
  if (slots && ((uintptr_t)slots & 3)) {
    set_error("%s: slots must be 4-byte aligned", fn);
    return SMD_ERR_INVALID_ARG;
  }
  WriterArgs a = {};
  a.kv = (const uint16_t *)kv;
  a.kv_stride = kv_stride;
  a.num_rows = num_rows;
  a.slots = slots;
  a.pool_rows = pool->num_rows;
  a.nope = (uint8_t *)pool->nope;
  a.nope_stride = d.nope_stride_b;
  a.scale = (uint8_t *)pool->scale;
  a.scale_stride = d.scale_stride_b;
  a.rope = (uint16_t *)pool->rope;
  a.rope_stride = d.rope_stride_b / 2;
  hipError_t e = launch_write_kv_fp8(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", fn, hipGetErrorString(e));
    return SMD_ERR_HIP;
  }
  return SMD_OK;
}

// ---------------------------------------------------------------------------
// dense paged GQA decode
// ---------------------------------------------------------------------------
namespace smd {
constexpr int32_t kPagedRows = 64;     // (Hq / Hkv) * mtp query rows per workgroup
constexpr int32_t kPagedBtMax = 4096;  // block-table entries a split may span
constexpr int32_t kPagedMaxSplits = 32;  // smd_paged_num_splits' cap

static int64_t paged_chunk(int32_t max_ctx, int32_t s) {
  const int64_t per = ((int64_t)max_ctx + s - 1) / s;
  return (per + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
}

static bool paged_chunk_fits(int64_t chunk, int32_t page) { return (chunk + page - 1) / page + 1 <= kPagedBtMax; }
}  // namespace smd

extern "C" int32_t smd_paged_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                        int32_t page_size, int32_t num_cus) {
  g_err[0] = 0;
  if (num_seqs < 0 || num_kv_heads < 1 || max_context_len < 0 || page_size < 16 || (page_size & (page_size - 1))) {
    set_error("smd_paged_num_splits: bad sizes");
    return SMD_ERR_INVALID_ARG;
  }
  if (num_seqs == 0 || max_context_len == 0) return 1;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int64_t cap_len = (max_context_len + kSplitAlign - 1) / kSplitAlign;
  int64_t s = (cus + units - 1) / units;  // fill the GPU once
  if (s > cap_len) s = cap_len;
  if (s > kPagedMaxSplits) s = kPagedMaxSplits;
  if (s < 1) s = 1;
  while (s < SMD_MAX_SPLITS && !paged_chunk_fits(paged_chunk(max_context_len, (int32_t)s), page_size)) ++s;
  if (!paged_chunk_fits(paged_chunk(max_context_len, (int32_t)s), page_size)) {
    set_error("smd_paged_num_splits: max_context_len %d needs more than %d splits at page size %d", max_context_len,
              SMD_MAX_SPLITS, page_size);
    return SMD_ERR_UNSUPPORTED;
  }
  return (int32_t)s;
}

extern "C" int smd_paged_decode(const void *q, int32_t num_seqs, int32_t mtp, int32_t num_q_heads,
                                const void *k_cache, const void *v_cache, int64_t num_blocks, int32_t page_size,
                                int32_t num_kv_heads, const int32_t *block_tables, int64_t block_tables_stride,
                                const int32_t *context_lens, int32_t max_context_len, float softmax_scale,
                                int32_t num_splits, float *partial_o, float *partial_lse, void *out, float *lse,
                                void *stream) {
  static const char *fn = "smd_paged_decode";
  g_err[0] = 0;
  if (num_seqs < 0 || mtp < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 0 || max_context_len < 0 ||
      block_tables_stride < 0) {
    set_error("%s: negative or zero size", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (num_q_heads % num_kv_heads != 0 || (num_q_heads / num_kv_heads) * mtp != kPagedRows) {
    set_error("%s: (num_q_heads / num_kv_heads) * mtp must be %d (got %d / %d, mtp %d)", fn, kPagedRows, num_q_heads,
              num_kv_heads, mtp);
    return SMD_ERR_UNSUPPORTED;
  }
  if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1))) {
    set_error("%s: page_size=%d must be a power of two >= 16", fn, page_size);
    return SMD_ERR_UNSUPPORTED;
  }
  if (num_splits < 1 || num_splits > SMD_MAX_SPLITS) {
    set_error("%s: num_splits=%d not in [1,%d]", fn, num_splits, SMD_MAX_SPLITS);
    return SMD_ERR_INVALID_ARG;
  }
  if (!isfinite(softmax_scale)) {
    set_error("%s: softmax_scale is not finite", fn);
    return SMD_ERR_INVALID_ARG;
  }
  const int64_t chunk = paged_chunk(max_context_len, num_splits);
  if (!paged_chunk_fits(chunk, page_size)) {
    set_error("%s: a split of %lld positions spans more than %d pages of %d; use more splits "
              "(smd_paged_num_splits)", fn, (long long)chunk, kPagedBtMax - 1, page_size);
    return SMD_ERR_INVALID_ARG;
  }
  const int64_t pages = ((int64_t)max_context_len + page_size - 1) / page_size;
  if (num_seqs > 0 && max_context_len > 0 && block_tables_stride < pages) {
    set_error("%s: block_tables_stride=%lld below the %lld pages of max_context_len", fn,
              (long long)block_tables_stride, (long long)pages);
    return SMD_ERR_INVALID_ARG;
  }
  const bool need_partials = num_splits > 1 || out == nullptr;
  if (num_seqs == 0 || max_context_len == 0) return SMD_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || (need_partials && (!partial_o || !partial_lse))) {
    set_error("%s: q, the caches, block_tables, context_lens%s are required", fn,
              need_partials ? " and the partials" : "");
    return SMD_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || (out && !aligned16(out)) ||
      (partial_o && !aligned16(partial_o)) || ((uintptr_t)block_tables & 3) || ((uintptr_t)context_lens & 3) ||
      (lse && ((uintptr_t)lse & 3)) || (partial_lse && ((uintptr_t)partial_lse & 3))) {
    set_error("%s: q, caches, out and partial_o must be 16-byte aligned; tables, lengths and lse 4-byte", fn);
    return SMD_ERR_INVALID_ARG;
  }
  PagedArgs a = {};
  a.q = (const uint16_t *)q;
  a.k_cache = (const uint8_t *)k_cache;
  a.v_cache = (const uint8_t *)v_cache;
  a.block_tables = block_tables;
  a.bt_stride = block_tables_stride;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.mtp = mtp;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.R = num_q_heads / num_kv_heads;
  a.page = page_size;
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  a.page_shift = sh;
  a.max_ctx = max_context_len;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.S = num_splits;
  a.chunk = (int32_t)chunk;
  a.part_o = need_partials ? partial_o : nullptr;
  a.part_lse = need_partials ? partial_lse : nullptr;
  a.out = need_partials ? nullptr : (uint16_t *)out;
  a.lse = need_partials ? nullptr : lse;
  a.hilo = out == nullptr;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_paged_decode(a, st);
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", fn, hipGetErrorString(e));
    return SMD_ERR_HIP;
  }
  if (need_partials && out) {
    e = launch_merge(partial_o, partial_lse, num_seqs * mtp * num_q_heads, num_q_heads, num_splits, nullptr,
                     (uint16_t *)out, lse, st, /*bf16_parts=*/true);
    if (e != hipSuccess) {
      set_error("%s: merge launch failed: %s", fn, hipGetErrorString(e));
      return SMD_ERR_HIP;
    }
  }
  return SMD_OK;
}
