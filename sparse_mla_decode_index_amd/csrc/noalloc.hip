// Allocation-free split-KV decode: the FP32 partials of a split plan live in a
// library-owned device array instead of caller buffers, for callers that
// cannot allocate device memory.  The decode itself is the library's usual one
// (decode_impl in api.cpp); only where the partials go differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/smd.h"
#include "smd_internal.h"

namespace smd {

// The partials of one call: o [T, H, s, 512] then lse [T, H, s], fp32.  In host
// code this name stands for the device array but is not its address: host
// code uses the per-device address from hipGetSymbolAddress (scratch_ptr).
static __device__ __attribute__((aligned(256))) float scratch[SMD_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;

// Address of the current device's copy of `scratch`, looked up once per
// device with that device current; nullptr (error set) on failure.
static float *scratch_ptr(const char *fn) {
  static std::mutex mu;
  static float *ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("%s: no usable current device (%s, device %d)", fn, hipGetErrorString(e), dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = (float *)p;
  }
  return ptrs[dev];
}

}  // namespace smd

using namespace smd;

extern "C" int smd_sparse_mla_decode_noalloc(const void *q_nope, const void *q_rope, int32_t num_tokens,
                                             int32_t num_heads, int32_t q_per_seq, const smd_kv_pool *kv,
                                             const int32_t *indices, int64_t indices_stride, int32_t topk,
                                             const float *sink, float softmax_scale, int32_t num_splits, void *out,
                                             float *lse, const smd_decode_options *options, void *stream) {
  static const char *fn = "smd_sparse_mla_decode_noalloc";
  set_error("");
  if (out == nullptr) {
    set_error("%s: out is required (the partials are not returned)", fn);
    return SMD_ERR_INVALID_ARG;
  }
  float *po = nullptr, *pl = nullptr;
  if (num_splits > 1 && num_splits <= SMD_MAX_SPLITS && num_tokens > 0 && num_heads > 0) {
    const size_t need = (size_t)num_tokens * (size_t)num_heads * (size_t)num_splits * 513 * sizeof(float);
    if (need > SMD_NOALLOC_SCRATCH_BYTES) {
      set_error("%s: %d tokens x %d heads x %d splits need %zu bytes of FP32 partials, above the %u-byte "
                "scratch array (use fewer splits or smd_sparse_mla_decode with caller buffers)",
                fn, num_tokens, num_heads, num_splits, need, (unsigned)SMD_NOALLOC_SCRATCH_BYTES);
      return SMD_ERR_WORKSPACE;
    }
    float *base = scratch_ptr(fn);
    if (base == nullptr) return SMD_ERR_HIP;
    po = base;
    pl = base + (size_t)num_tokens * num_heads * num_splits * kDim;
  }
  return decode_impl(fn, q_nope, q_rope, num_tokens, num_heads, q_per_seq, kv, indices, indices_stride, topk, nullptr,
                     sink, softmax_scale, num_splits, po, pl, out, lse, options, stream);
}
