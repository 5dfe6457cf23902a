// Host split planner (aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and
// persistent decode kernel", Summary part 1): the split count is chosen from
// the call's sizes alone by minimising a modelled time, the rounds of decode
// workgroups times one workgroup's time plus what each extra split adds in
// partial traffic and merge work.  Two kinds of workgroup are priced: the
// narrow kernels' (16 query rows, eight waves, one step per 16 positions of
// each wave's share) and the wide kernel's (128 query rows, one workgroup per
// CU, one tile per 32 positions); a step or tile costs more the fuller the
// GPU.  The caps are model fields (short_cap below long_kv indices,
// long_cap from there on).  The vLLM page "[ROCm][DSV4][Perf] Optimize Triton
// sparse-MLA decode on gfx950", Design, caps its kernel at four splits for
// short workloads and 32 for long ones; here the model prices what each
// split adds, and grids of few query rows fill the GPU only with more
// splits, so both defaults are 128.
//
// Pure integer arithmetic in picoseconds; no device access, so it may run
// during graph capture.
#include <stdint.h>
#include <string.h>

#include "../../include/smd.h"
#include "smd_internal.h"

// MI355X coefficients.  Narrow terms: fitted (log-time least squares) to
// graph-timed decode + merge over T in {1, 4, 16, 64}, H in {16, 64, 128},
// 384 to 65664 indices and s in {1, 2, 4, 8, 16, 32}, bf16 and fp8 pools.
// Wide terms: fitted the same way, with the merge terms held at the narrow
// values, to the wide kernel over T in {1, 4, 16, 32, 64}, H = 128, 384 to
// 65664 indices and s in {1, 2, 4, 8, 16, 32} (model/measured 0.94-1.07 for
// the middle 80% of 240 points).
static const smd_plan_model kDefaultModel = {
    /*fixed_ps=*/7194000,
    /*step_ps=*/1971000,
    /*step_load_ps=*/569000,
    /*merge_ps=*/4065000,
    /*part_ps=*/287,
    /*rows_per_wg=*/16,
    /*waves_per_wg=*/8,
    /*wg_per_cu=*/1,
    /*short_cap=*/128,
    /*long_cap=*/128,
    /*long_kv=*/4096,
    /*wide_rows=*/128,
    /*wide_tile=*/32,
    /*wide_fixed_ps=*/13648000,
    /*wide_tile_ps=*/1774000,
    /*wide_tile_fp8_ps=*/2192000,
    /*wide_tile_load_ps=*/536000,
    /*wide_cap=*/256,
    /*reserved=*/0,
};

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FP32 values per (token, head, split): 512 of o and one lse.
static const int64_t kPartialFloats = 513;

namespace smd {

const smd_plan_model &default_plan_model() { return kDefaultModel; }

static int64_t split_len(int64_t kv_len, int64_t s) {
  const int64_t chunk = ceil_div(ceil_div(kv_len, s), SMD_SPLIT_ALIGN) * SMD_SPLIT_ALIGN;
  return chunk < kv_len ? chunk : kv_len;
}

static int64_t tail_cost(const smd_plan_model &m, int64_t num_seqs, int64_t M, int64_t s) {
  return s > 1 ? m.merge_ps + m.part_ps * num_seqs * M * s : 0;
}

int64_t narrow_cost(const smd_plan_model &m, int64_t num_seqs, int64_t M, int64_t kv_len, int64_t cus,
                    int64_t s) {
  const int64_t slots = cus * m.wg_per_cu;
  const int64_t wgs = num_seqs * ceil_div(M, m.rows_per_wg) * s;
  const int64_t waves = ceil_div(wgs, slots);
  const int64_t busy = wgs < slots ? wgs : slots;
  const int64_t steps = ceil_div(ceil_div(split_len(kv_len, s), 16), m.waves_per_wg);
  const int64_t step = m.step_ps + m.step_load_ps * busy / slots;
  return waves * (m.fixed_ps + steps * step) + tail_cost(m, num_seqs, M, s);
}

bool wide_priced(const smd_plan_model &m, int64_t M, bool two_source) {
  return !two_source && m.wide_rows > 0 && M % m.wide_rows == 0;
}

int64_t wide_cost(const smd_plan_model &m, int64_t num_seqs, int64_t M, int64_t kv_len, int32_t kv_dtype,
                  int64_t cus, int64_t s) {
  const int64_t wgs = num_seqs * (M / m.wide_rows) * s;
  const int64_t waves = ceil_div(wgs, cus);
  const int64_t busy = wgs < cus ? wgs : cus;
  const int64_t tiles = ceil_div(split_len(kv_len, s), m.wide_tile);
  const int64_t tile = (kv_dtype == SMD_KV_FP8_E4M3_UE8M0 ? m.wide_tile_fp8_ps : m.wide_tile_ps) +
                       m.wide_tile_load_ps * busy / cus;
  return waves * (m.wide_fixed_ps + tiles * tile) + tail_cost(m, num_seqs, M, s);
}

}  // namespace smd

using namespace smd;

static bool model_ok(const smd_plan_model *model, const char *fn) {
  if (!model) {
    set_error("%s: model is NULL", fn);
    return false;
  }
  if (model->wg_per_cu < 1 || model->rows_per_wg < 1 || model->waves_per_wg < 1 || model->short_cap < 1 ||
      model->long_cap < 1 || model->short_cap > SMD_MAX_SPLITS || model->long_cap > SMD_MAX_SPLITS ||
      model->wide_cap < 0 || model->wide_cap > SMD_MAX_SPLITS || model->reserved != 0 ||
      model->wide_rows < 0 || (model->wide_rows > 0 && model->wide_tile < 1)) {
    set_error("%s: invalid model (sizes and caps must be >= 1, caps <= %d, wide_cap in [0, %d], reserved 0, "
              "wide_rows >= 0, wide_tile >= 1 when wide_rows > 0)", fn, SMD_MAX_SPLITS, SMD_MAX_SPLITS);
    return false;
  }
  return true;
}

extern "C" int smd_plan_default_model(smd_plan_model *model) {
  if (!model) {
    set_error("smd_plan_default_model: model is NULL");
    return SMD_ERR_INVALID_ARG;
  }
  *model = kDefaultModel;
  return SMD_OK;
}

extern "C" int smd_plan_decode(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq, int32_t kv_len,
                               int32_t kv_dtype, int32_t num_cus, int32_t two_source,
                               const smd_plan_model *model, int32_t *kernel) {
  static const char *fn = "smd_plan_num_kv_splits";
  if (!model) model = &kDefaultModel;
  if (num_seqs < 0 || num_heads < 0 || q_per_seq < 0 || kv_len < 0) {
    set_error("%s: negative size", fn);
    return SMD_ERR_INVALID_ARG;
  }
  if (kv_dtype != SMD_KV_BF16 && kv_dtype != SMD_KV_FP8_E4M3_UE8M0) {
    set_error("%s: unknown kv_dtype %d", fn, kv_dtype);
    return SMD_ERR_UNSUPPORTED;
  }
  if (!model_ok(model, fn)) return SMD_ERR_INVALID_ARG;
  if (kernel) *kernel = SMD_KERNEL_AUTO;
  if (num_seqs == 0 || kv_len == 0 || num_heads == 0 || q_per_seq == 0) return 1;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t M = (int64_t)num_heads * q_per_seq;
  const bool wide = wide_priced(*model, M, two_source != 0);
  const bool is_short = kv_len < model->long_kv;
  const int64_t cap_tiles = ceil_div(kv_len, SMD_SPLIT_ALIGN);
  const int64_t cap_n0 = is_short ? model->short_cap : model->long_cap;
  const int64_t cap_w0 = is_short ? model->short_cap : (model->wide_cap > 0 ? model->wide_cap : model->long_cap);
  const int64_t cap_n = cap_n0 < cap_tiles ? cap_n0 : cap_tiles;
  const int64_t cap_w = wide ? (cap_w0 < cap_tiles ? cap_w0 : cap_tiles) : 0;
  const int64_t cap = cap_n > cap_w ? cap_n : cap_w;
  int best_s = 1;
  bool best_wide = false;
  int64_t best_cost = INT64_MAX;
  for (int64_t s = 1; s <= cap; ++s) {
    int64_t cost = s <= cap_n ? narrow_cost(*model, num_seqs, M, kv_len, cus, s) : INT64_MAX;
    bool w = false;
    if (s <= cap_w) {
      const int64_t cw = wide_cost(*model, num_seqs, M, kv_len, kv_dtype, cus, s);
      if (cw < cost) {
        cost = cw;
        w = true;
      }
    }
    if (cost < best_cost) {
      best_cost = cost;
      best_s = (int)s;
      best_wide = w;
    }
  }
  if (kernel) *kernel = best_wide ? SMD_KERNEL_WIDE : SMD_KERNEL_AUTO;
  return best_s;
}

extern "C" int smd_plan_num_kv_splits_model(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq,
                                            int32_t kv_len, int32_t kv_dtype, int32_t num_cus,
                                            const smd_plan_model *model) {
  if (!model) {
    set_error("smd_plan_num_kv_splits: model is NULL");
    return SMD_ERR_INVALID_ARG;
  }
  return smd_plan_decode(num_seqs, num_heads, q_per_seq, kv_len, kv_dtype, num_cus, 0, model, nullptr);
}

extern "C" int smd_plan_num_kv_splits(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq,
                                      int32_t kv_len, int32_t kv_dtype, int32_t num_cus) {
  return smd_plan_decode(num_seqs, num_heads, q_per_seq, kv_len, kv_dtype, num_cus, 0, &kDefaultModel,
                         nullptr);
}

extern "C" int smd_split_bounds(int32_t kv_len, int32_t num_splits, int32_t split, int32_t *begin,
                                int32_t *end) {
  if (!begin || !end) {
    smd::set_error("smd_split_bounds: NULL output pointer");
    return SMD_ERR_INVALID_ARG;
  }
  if (kv_len < 0 || num_splits < 1 || split < 0 || split >= num_splits) {
    smd::set_error("smd_split_bounds: kv_len=%d num_splits=%d split=%d out of range", kv_len,
                   num_splits, split);
    return SMD_ERR_INVALID_ARG;
  }
  const int64_t per = ceil_div(kv_len, num_splits);
  const int64_t chunk = ceil_div(per, SMD_SPLIT_ALIGN) * SMD_SPLIT_ALIGN;
  int64_t a = (int64_t)split * chunk, e = a + chunk;
  if (a > kv_len) a = kv_len;
  if (e > kv_len) e = kv_len;
  *begin = (int32_t)a;
  *end = (int32_t)e;
  return SMD_OK;
}

extern "C" size_t smd_partials_bytes(int32_t num_tokens, int32_t num_heads, int32_t num_splits) {
  if (num_tokens < 0 || num_heads < 0 || num_splits < 1 || num_splits > SMD_MAX_MERGE_SPLITS) {
    smd::set_error("smd_partials_bytes: num_tokens=%d num_heads=%d num_splits=%d out of range", num_tokens,
                   num_heads, num_splits);
    return 0;
  }
  return (size_t)num_tokens * (size_t)num_heads * (size_t)num_splits * (size_t)(kPartialFloats * 4);
}
