// Host split planner (aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and
// persistent decode kernel", Summary part 1): the split count is chosen from
// the call's sizes alone by minimising a modelled time, the rounds of decode
// workgroups times one workgroup's time plus what each extra split adds in
// partial traffic and merge work.  The per-wave time is that of this
// library's decode workgroup: a fixed part plus one step per 16 positions of
// each wave's share, a step costing more the fuller the GPU.  The caps follow the vLLM page
// "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on gfx950", Design:
// at most four splits for short index lists, up to 32 for long ones.
//
// Pure integer arithmetic in picoseconds; no device access, so it may run
// during graph capture.
#include <stdint.h>
#include <string.h>

#include "../../include/smd.h"

namespace smd {
void set_error(const char *fmt, ...);
}

// MI355X coefficients, fitted (log-time least squares) to graph-timed decode
// + merge over T in {1, 4, 16, 64}, H in {16, 64, 128}, 384 to 65664 indices
// and s in {1, 2, 4, 8, 16, 32}, bf16 and fp8 pools.
static const smd_plan_model kDefaultModel = {
    /*fixed_ps=*/7194000,
    /*step_ps=*/1971000,
    /*step_load_ps=*/569000,
    /*merge_ps=*/4065000,
    /*part_ps=*/287,
    /*rows_per_wg=*/16,
    /*waves_per_wg=*/8,
    /*wg_per_cu=*/1,
    /*short_cap=*/4,
    /*long_cap=*/32,
    /*long_kv=*/4096,
};

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FP32 values per (token, head, split): 512 of o and one lse.
static const int64_t kPartialFloats = 513;

extern "C" int smd_plan_default_model(smd_plan_model *model) {
  if (!model) {
    smd::set_error("smd_plan_default_model: model is NULL");
    return SMD_ERR_INVALID_ARG;
  }
  *model = kDefaultModel;
  return SMD_OK;
}

extern "C" int smd_plan_num_kv_splits_model(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq,
                                            int32_t kv_len, int32_t kv_dtype, int32_t num_cus,
                                            const smd_plan_model *model) {
  if (!model) {
    smd::set_error("smd_plan_num_kv_splits: model is NULL");
    return SMD_ERR_INVALID_ARG;
  }
  if (num_seqs < 0 || num_heads < 0 || q_per_seq < 0 || kv_len < 0) {
    smd::set_error("smd_plan_num_kv_splits: negative size");
    return SMD_ERR_INVALID_ARG;
  }
  if (kv_dtype != SMD_KV_BF16 && kv_dtype != SMD_KV_FP8_E4M3_UE8M0) {
    smd::set_error("smd_plan_num_kv_splits: unknown kv_dtype %d", kv_dtype);
    return SMD_ERR_UNSUPPORTED;
  }
  if (model->wg_per_cu < 1 || model->rows_per_wg < 1 || model->waves_per_wg < 1 || model->short_cap < 1 ||
      model->long_cap < 1 || model->short_cap > SMD_MAX_SPLITS || model->long_cap > SMD_MAX_SPLITS) {
    smd::set_error("smd_plan_num_kv_splits: invalid model (sizes and caps must be >= 1, caps <= %d)",
                   SMD_MAX_SPLITS);
    return SMD_ERR_INVALID_ARG;
  }
  if (num_seqs == 0 || kv_len == 0 || num_heads == 0 || q_per_seq == 0) return 1;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t M = (int64_t)num_heads * q_per_seq;
  const int64_t G = ceil_div(M, model->rows_per_wg);
  const int64_t slots = cus * model->wg_per_cu;
  const int64_t cap_len = kv_len < model->long_kv ? model->short_cap : model->long_cap;
  const int64_t cap_tiles = ceil_div(kv_len, SMD_SPLIT_ALIGN);
  const int64_t cap = cap_len < cap_tiles ? cap_len : cap_tiles;
  int best_s = 1;
  int64_t best_cost = INT64_MAX;
  for (int64_t s = 1; s <= cap; ++s) {
    const int64_t wgs = (int64_t)num_seqs * G * s;
    const int64_t waves = ceil_div(wgs, slots);
    const int64_t busy = wgs < slots ? wgs : slots;
    const int64_t chunk = ceil_div(ceil_div(kv_len, s), SMD_SPLIT_ALIGN) * SMD_SPLIT_ALIGN;
    const int64_t len = chunk < kv_len ? chunk : kv_len;
    const int64_t steps = ceil_div(ceil_div(len, 16), model->waves_per_wg);
    const int64_t step = model->step_ps + model->step_load_ps * busy / slots;
    int64_t cost = waves * (model->fixed_ps + steps * step);
    if (s > 1) cost += model->merge_ps + model->part_ps * (int64_t)num_seqs * M * s;
    if (cost < best_cost) {
      best_cost = cost;
      best_s = (int)s;
    }
  }
  return best_s;
}

extern "C" int smd_plan_num_kv_splits(int32_t num_seqs, int32_t num_heads, int32_t q_per_seq,
                                      int32_t kv_len, int32_t kv_dtype, int32_t num_cus) {
  return smd_plan_num_kv_splits_model(num_seqs, num_heads, q_per_seq, kv_len, kv_dtype, num_cus,
                                      &kDefaultModel);
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
