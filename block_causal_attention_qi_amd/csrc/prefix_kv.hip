// Prefix KV cache write for step 0 (gfx950).
//
// The prompt and reference-image K/V computed at the first denoising step is stored and
// reused by every later step of the same request, and rebuilt for the next request
// (ThakiCloud blog "Qwen-Image-2.1 vLLM-Omni day 0", section "Serving architecture: the
// cross-step prefix KV cache").  The cache may be kept in FP8 for long-prompt or
// multi-image work (vLLM recipe "Qwen/Qwen-Image-2.1", section "Prefix KV cache").
//
// Source: packed token-major bf16 [sum L_p][H][D].  Destination, per request: K
// [H][L_p][D], V [H][L_p][D], head-major so that each (request, head) key stream is one
// contiguous run for the attention kernel's tile loads.
//
// bf16 cache: one pass, a re-layout copy (16 bytes per lane, contiguous writes).
// fp8 caches (OCP E4M3FN, one float32 scale per (request, head, K|V); the V-only cache
// keeps K in bf16 with scale 1):
//   pass 1  every workgroup takes 64 tokens of one (request, head) and writes the max |x|
//           of K and of V over them to the workspace (no atomics: max is exact, so the
//           result does not depend on any order);
//   pass 2  one workgroup per (request, head) reduces its partials to the absmax a;
//   pass 3  every workgroup derives scale = a/448 and inv = 448/a (correctly rounded
//           float32 divisions; a == 0 gives 1 and 1), the first workgroup of a (request,
//           head) stores the scales, and all quantise their tokens: code = nearest E4M3FN
//           value to x*inv (float32 product), ties to the even code, saturating at 448.
// The copy and passes 1 and 3 run one workgroup per (64-token chunk, request, head).
#include <hip/hip_runtime.h>

#include <mutex>

#include "qi_internal.h"

// Scratch of the allocation-free build (qi_prefix_kv_build_noalloc): the absmax partials
// of the fp8 passes live here instead of in the caller's workspace.  Each GPU the library
// runs on holds its own copy until the process ends.  Host code must never pass the name
// `scratch` to a kernel or a copy (on the host it is only a stand-in symbol): it uses the
// device address qi_scratch_partials() obtained with hipGetSymbolAddress on that device.
static __device__ __align__(256) float scratch[QI_NOALLOC_MAX_PARTIALS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

constexpr int NT = 256;
constexpr int CHUNK = QI_CACHE_CHUNK;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> E4M3FN code: round to nearest, ties to even, saturate to +-448, keep the sign
// of zero.  Integer arithmetic on the float32 bit pattern, exact for every input.
__device__ __forceinline__ uint32_t e4m3fn_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {                 // |y| >= 448 (and inf): saturate
    code = 0x7eu;
  } else if (a < 0x3c800000u) {           // |y| < 2^-6: subnormal codes m * 2^-9
    // |y| * 2^9 < 8 is exact in float32; rint rounds to nearest even; 8 encodes 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {                                // normal: keep 3 of the 23 mantissa bits
    const uint32_t e = (a >> 23) - 127u + 7u;          // biased E4M3 exponent, 1..15
    const uint32_t mant = a & 0x7fffffu;
    const uint32_t keep = mant >> 20, rest = mant & 0xfffffu;
    uint32_t c = (e << 3) | keep;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) c += 1u;   // carry may bump e
    code = c > 0x7eu ? 0x7eu : c;
  }
  return sign | code;
}

// Workgroup (chunk x, request y, head z): tokens [64 x, 64 x + 64) of one request and one
// head.  Item i of the workgroup is 16-byte chunk i % (D/8) of token i / (D/8): the writes
// are one contiguous run of the head-major destination.
__global__ __launch_bounds__(NT) void cache_copy_bf16(const qi_req_dev *__restrict__ reqs,
                                                      int H, int D,
                                                      const uint4 *__restrict__ k_pre,
                                                      const uint4 *__restrict__ v_pre,
                                                      uint8_t *__restrict__ cache) {
  const qi_req_dev r = reqs[blockIdx.y];
  const int t0 = blockIdx.x * CHUNK, h = blockIdx.z;
  if (t0 >= r.lp) return;
  const int nt = min(CHUNK, r.lp - t0);
  const int ch = D / 8;   // 16-byte chunks per (token, head)
  for (int i = threadIdx.x; i < nt * ch; i += NT) {
    const int tok = t0 + i / ch, c = i % ch;
    const int64_t src = ((int64_t)(r.pre_tok + tok) * H + h) * ch + c;
    const int64_t dst = ((int64_t)h * r.lp + tok) * D * 2 + c * 16;
    *reinterpret_cast<uint4 *>(cache + r.k_off + dst) = k_pre[src];
    *reinterpret_cast<uint4 *>(cache + r.v_off + dst) = v_pre[src];
  }
}

// max over the workgroup of a non-negative float (every thread passes its value)
__device__ __forceinline__ float block_max(float m, float *red) {
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

// Pass 1, workgroup (chunk x, request y, head z): max |x| of K and of V over the chunk's
// tokens of head z -> partials[part_idx + (x * 2 + K|V) * H + z].
__global__ __launch_bounds__(NT) void cache_absmax_fp8(const qi_req_dev *__restrict__ reqs,
                                                       int H, int D,
                                                       const uint4 *__restrict__ k_pre,
                                                       const uint4 *__restrict__ v_pre,
                                                       float *__restrict__ partials) {
  __shared__ float red[NT / 64];
  const qi_req_dev r = reqs[blockIdx.y];
  const int t0 = blockIdx.x * CHUNK, h = blockIdx.z;
  if (t0 >= r.lp) return;
  const int nt = min(CHUNK, r.lp - t0);
  const int ch = D / 8;
  float m[2] = {0.0f, 0.0f};
  for (int i = threadIdx.x; i < nt * ch; i += NT) {
    const int tok = t0 + i / ch, c = i % ch;
    const int64_t src = ((int64_t)(r.pre_tok + tok) * H + h) * ch + c;
    const uint4 kv[2] = {k_pre[src], v_pre[src]};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t x[4] = {kv[w].x, kv[w].y, kv[w].z, kv[w].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) m[w] = fmaxf(m[w], fmaxf(fabsf(bf16_lo(x[j])), fabsf(bf16_hi(x[j]))));
    }
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const float a = block_max(m[w], red);
    if (threadIdx.x == 0) partials[r.part_idx + (blockIdx.x * 2 + w) * H + h] = a;
  }
}

// Pass 2, workgroup (request x, head y): reduce the request's per-chunk partials of head y
// to its absmax of K and of V, written over the chunk-0 partials (read by pass 3).
__global__ __launch_bounds__(NT) void cache_absmax_reduce(const qi_req_dev *__restrict__ reqs,
                                                          int H, float *__restrict__ partials) {
  __shared__ float red[NT / 64];
  const qi_req_dev r = reqs[blockIdx.x];
  const int h = blockIdx.y;
  float m[2] = {0.0f, 0.0f};
  for (int c = threadIdx.x; c < r.n_chunks; c += NT) {
#pragma unroll
    for (int w = 0; w < 2; ++w) m[w] = fmaxf(m[w], partials[r.part_idx + (c * 2 + w) * H + h]);
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const float a = block_max(m[w], red);   // every read above precedes its barriers
    if (threadIdx.x == 0) partials[r.part_idx + w * H + h] = a;
  }
}

// Pass 3, workgroup (chunk x, request y, head z): turn the request's absmax of head z into
// the scales, store them (chunk 0), quantise the chunk's tokens of head z.  K8 false (the
// V-only cache): K is copied as bf16 and its scale stored as 1.
template <bool K8>
__global__ __launch_bounds__(NT) void cache_quant_fp8(const qi_req_dev *__restrict__ reqs,
                                                      int H, int D,
                                                      const uint4 *__restrict__ k_pre,
                                                      const uint4 *__restrict__ v_pre,
                                                      const float *__restrict__ partials,
                                                      uint8_t *__restrict__ cache) {
  const qi_req_dev r = reqs[blockIdx.y];
  const int t0 = blockIdx.x * CHUNK, h = blockIdx.z;
  if (t0 >= r.lp) return;
  float inv[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const float a = partials[r.part_idx + w * H + h];   // reduced by pass 2
    inv[w] = a > 0.0f ? __fdiv_rn(448.0f, a) : 1.0f;
    const float scale = (w == 0 && !K8) ? 1.0f : a > 0.0f ? __fdiv_rn(a, 448.0f) : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0)
      reinterpret_cast<float *>(cache + r.s_off)[w * H + h] = scale;
  }
  const int nt = min(CHUNK, r.lp - t0);
  const int ch = D / 8;
  for (int i = threadIdx.x; i < nt * ch; i += NT) {
    const int tok = t0 + i / ch, c = i % ch;
    const int64_t src = ((int64_t)(r.pre_tok + tok) * H + h) * ch + c;
    const int64_t dst = ((int64_t)h * r.lp + tok) * D + c * 8;
    const uint4 kv[2] = {k_pre[src], v_pre[src]};
    if (!K8) *reinterpret_cast<uint4 *>(cache + r.k_off + dst * 2) = kv[0];
#pragma unroll
    for (int w = K8 ? 0 : 1; w < 2; ++w) {
      const uint32_t x[4] = {kv[w].x, kv[w].y, kv[w].z, kv[w].w};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = e4m3fn_from_f32(bf16_lo(x[j]) * inv[w]);
        const uint32_t hi = e4m3fn_from_f32(bf16_hi(x[j]) * inv[w]);
        out[j >> 1] |= (lo | (hi << 8)) << (16 * (j & 1));
      }
      *reinterpret_cast<uint2 *>(cache + (w == 0 ? r.k_off : r.v_off) + dst) =
          make_uint2(out[0], out[1]);
    }
  }
}

}  // namespace

qi_status qi_scratch_partials(float **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QI_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return QI_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<float *>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return QI_OK;
}

qi_status qi_launch_cache_write(const qi_plan *p, const void *k_pre, const void *v_pre,
                                void *cache, float *partials, void *stream) {
  if (p->max_chunks == 0) return QI_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = static_cast<uint8_t *>(p->d_ws);
  const qi_req_dev *reqs = reinterpret_cast<const qi_req_dev *>(ws + p->reqs_off);
  const dim3 grid(p->max_chunks, p->n_req, p->H);
  const uint4 *k = static_cast<const uint4 *>(k_pre);
  const uint4 *v = static_cast<const uint4 *>(v_pre);
  uint8_t *c = static_cast<uint8_t *>(cache);
  if (p->kv == QI_KV_BF16) {
    hipLaunchKernelGGL(cache_copy_bf16, grid, dim3(NT), 0, s, reqs, p->H, p->D, k, v, c);
  } else {
    float *part = partials ? partials : reinterpret_cast<float *>(ws + p->part_off);
    hipLaunchKernelGGL(cache_absmax_fp8, grid, dim3(NT), 0, s, reqs, p->H, p->D, k, v, part);
    if (hipGetLastError() != hipSuccess) return QI_ERR_HIP;
    hipLaunchKernelGGL(cache_absmax_reduce, dim3(p->n_req, p->H), dim3(NT), 0, s, reqs, p->H, part);
    if (hipGetLastError() != hipSuccess) return QI_ERR_HIP;
    auto quant = p->kv == QI_KV_FP8_E4M3 ? cache_quant_fp8<true> : cache_quant_fp8<false>;
    hipLaunchKernelGGL(quant, grid, dim3(NT), 0, s, reqs, p->H, p->D, k, v, (const float *)part, c);
  }
  return hipGetLastError() == hipSuccess ? QI_OK : QI_ERR_HIP;
}
