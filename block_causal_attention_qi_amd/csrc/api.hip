// C-ABI entry points that enqueue device work: workspace upload, the step-0 prefix build,
// the denoising step and the full recompute.  Every argument is checked on the host
// before anything is enqueued; a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include "qi_internal.h"

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool ok_ptr(const void *p) { return p != nullptr && aligned16(p); }

}  // namespace

extern "C" {

qi_status qi_plan_upload(qi_plan *p, void *d_ws, size_t bytes, void *stream) {
  if (!p || !ok_ptr(d_ws)) return QI_ERR_INVALID_ARG;
  if (bytes < p->ws_bytes) return QI_ERR_BUFFER_TOO_SMALL;
  if (!p->ws_image.empty()) {
    if (hipMemcpyAsync(d_ws, p->ws_image.data(), p->ws_image.size(), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
      return QI_ERR_HIP;
  }
  p->d_ws = d_ws;
  return QI_OK;
}

// Step 0 of a request (prefix side): write the cache, then prefix attention.  The
// prompt and reference KV computed at the first step is what every later step reuses
// (ThakiCloud blog "Qwen-Image-2.1 vLLM-Omni day 0", section "Serving architecture: the
// cross-step prefix KV cache"; the prefill runs eagerly, vLLM recipe
// "Qwen/Qwen-Image-2.1", section "CUDA graphs").
qi_status qi_prefix_kv_build(qi_plan *p, const void *q_pre, const void *k_pre,
                             const void *v_pre, void *o_pre, void *d_cache,
                             size_t cache_bytes, void *stream) {
  if (!p || !ok_ptr(q_pre) || !ok_ptr(k_pre) || !ok_ptr(v_pre) || !ok_ptr(o_pre) ||
      !ok_ptr(d_cache))
    return QI_ERR_INVALID_ARG;
  if (!p->d_ws) return QI_ERR_STATE;
  if (cache_bytes < p->cache_bytes) return QI_ERR_BUFFER_TOO_SMALL;
  qi_status st = qi_launch_cache_write(p, k_pre, v_pre, d_cache, nullptr, stream);
  if (st != QI_OK) return st;
  st = qi_launch_attention(p, QI_CALL_PREFIX, q_pre, k_pre, v_pre, o_pre, nullptr, stream);
  if (st != QI_OK) return st;
  p->built = true;
  return QI_OK;
}

// The same step-0 build for callers that cannot allocate device memory: the fp8 absmax
// partials go to the library's static scratch array of this device instead of the
// workspace (the workspace still holds the plan's tables, uploaded beforehand).  Nothing
// in the scratch has to start at zero: the first fp8 pass writes every partial that the
// later passes read.  Calls that overlap in time on one device share the array and race.
qi_status qi_prefix_kv_build_noalloc(qi_plan *p, const void *q_pre, const void *k_pre,
                                     const void *v_pre, void *o_pre, void *d_cache,
                                     size_t cache_bytes, void *stream) {
  if (!p || !ok_ptr(q_pre) || !ok_ptr(k_pre) || !ok_ptr(v_pre) || !ok_ptr(o_pre) ||
      !ok_ptr(d_cache))
    return QI_ERR_INVALID_ARG;
  if (p->part_floats > QI_NOALLOC_MAX_PARTIALS) return QI_ERR_BUFFER_TOO_SMALL;
  if (!p->d_ws) return QI_ERR_STATE;
  if (cache_bytes < p->cache_bytes) return QI_ERR_BUFFER_TOO_SMALL;
  float *part = nullptr;
  if (p->part_floats > 0) {
    const qi_status st = qi_scratch_partials(&part);
    if (st != QI_OK) return st;
  }
  qi_status st = qi_launch_cache_write(p, k_pre, v_pre, d_cache, part, stream);
  if (st != QI_OK) return st;
  st = qi_launch_attention(p, QI_CALL_PREFIX, q_pre, k_pre, v_pre, o_pre, nullptr, stream);
  if (st != QI_OK) return st;
  p->built = true;
  return QI_OK;
}

// Denoising step: image rows over the cached prefix plus the live image KV (exact reuse:
// vLLM recipe "Qwen/Qwen-Image-2.1", section "Prefix KV cache").
qi_status qi_denoise_attn_step(const qi_plan *p, const void *d_cache, size_t cache_bytes,
                               const void *q_img, const void *k_img, const void *v_img,
                               void *o_img, void *stream) {
  if (!p || !ok_ptr(d_cache) || !ok_ptr(q_img) || !ok_ptr(k_img) || !ok_ptr(v_img) ||
      !ok_ptr(o_img))
    return QI_ERR_INVALID_ARG;
  if (!p->d_ws || !p->built) return QI_ERR_STATE;
  if (cache_bytes < p->cache_bytes) return QI_ERR_BUFFER_TOO_SMALL;
  return qi_launch_attention(p, QI_CALL_DENOISE, q_img, k_img, v_img, o_img, d_cache, stream);
}

// Full recompute without the cache (the baseline the prefix cache saves against).
qi_status qi_attn_full_reference_step(const qi_plan *p, const void *q_all, const void *k_all,
                                      const void *v_all, void *o_all, void *stream) {
  if (!p || !ok_ptr(q_all) || !ok_ptr(k_all) || !ok_ptr(v_all) || !ok_ptr(o_all))
    return QI_ERR_INVALID_ARG;
  if (!p->d_ws) return QI_ERR_STATE;
  return qi_launch_attention(p, QI_CALL_FULL, q_all, k_all, v_all, o_all, nullptr, stream);
}

}  // extern "C"
