// Block-causal attention forward for gfx950 (CDNA4), bf16 MFMA, fp32 online softmax.
//
// One workgroup (4 wavefronts, 256 lanes) owns one (request, head, row tile of <= 128
// rows); each wavefront owns 32 query rows and keeps its Q fragments and its O
// accumulator in registers for the whole key loop.  Row tiles never cross a block, so
// every row of a tile sees the same key prefix [0, kend) (block-causal rule: a row of
// block b sees keys of blocks 0..b; ThakiCloud blog "Qwen-Image-2.1 vLLM-Omni day 0",
// section "Serving architecture: the cross-step prefix KV cache").  Key tiles past kend
// are never visited (EMPTY tiles skipped), the one straddling kend is masked (PARTIAL),
// the others run unmasked (FULL).
//
// Key sources.  In the full and prefix calls K/V come from one token-major tensor.  In
// the denoising call keys [0, lp) come from the prefix cache (head-major, bf16 or E4M3FN
// codes with a per-head scale, dequantised while staging) and keys [lp, kend) from the
// live image K/V; a key tile straddling lp gathers from both.  Key tiles start at key 0
// in every call and the arithmetic does not depend on where a key came from, so on a
// bf16 cache the denoising call reproduces the full call's image rows bit for bit -- the
// exact reuse the vLLM recipe "Qwen/Qwen-Image-2.1" states in its "Prefix KV cache"
// section.
//
// Per key tile (64 keys) and wavefront:
//   S^T = K Q^T      16 x v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q in VGPRs)
//   lane (query j = lane%32, half g = lane/32) then holds 32 scores of its query row
//   online softmax in the log2 domain: x = s * log2(e)/sqrt(D) - m, p = 2^x.  The
//   running max m is only raised when a row's tile max exceeds it by more than 8 (then
//   every row of the wavefront is rescaled exactly); otherwise p <= 2^8, which bf16 and
//   fp32 hold without loss of relative precision.  The result is the same softmax.
//   O^T += V^T P^T   16 x MFMA (A = V^T from LDS, B = P packed to bf16 in VGPRs); the
//   key order inside each 16-key MFMA step is permuted consistently on both operands so
//   that P never leaves the lane that computed it.
// LDS: K tile [64 keys][D] and V^T tile [D][64 keys], bf16, XOR-swizzled in 16-byte
// chunks, double-buffered; the next tile is prefetched into registers during compute.
#include <hip/hip_runtime.h>
#include <math.h>

#include "qi_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = QI_KERNEL_BM;
constexpr int BN = QI_KERNEL_BN;
constexpr int NT = 256;
constexpr float TAU = 8.0f;   // lazy-rescale threshold, log2 units

enum { SRC_ONE = 0, SRC_CACHE_BF16 = 1, SRC_CACHE_FP8 = 2 };

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;           // 16-byte chunks per K row
  static constexpr int KROWS = NT / CH;      // K rows staged per pass
  static constexpr int KPASS = BN / KROWS;   // passes per K tile
  static constexpr int KPT = BN * CH / NT;   // consecutive keys per lane in V staging
  static constexpr int QS = D / 16;          // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;          // 32-wide blocks of the output
  static constexpr int TILE = BN * D;        // bf16 elements per staged K (or V) tile
  static_assert(KPASS * KROWS == BN && (KPT == 2 || KPT == 4), "tile shape");
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};   // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, v);
}

// 8 E4M3FN codes -> 8 bf16 of code * scale (value * scale in fp32, rounded once to bf16)
__device__ __forceinline__ uint4 dequant8(uint32_t lo, uint32_t hi, float scale) {
  f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  uint4 r;
  r.x = pack_bf16(a[0] * scale, a[1] * scale);
  r.y = pack_bf16(b[0] * scale, b[1] * scale);
  r.z = pack_bf16(c[0] * scale, c[1] * scale);
  r.w = pack_bf16(d[0] * scale, d[1] * scale);
  return r;
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Physical position of key k inside a V^T row: bits 2 and 3 swapped, so that the 8 keys
// one lane feeds to a 16-key PV step are contiguous.
__device__ __forceinline__ int vpos(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

struct TileArgs {
  const __bf16 *k, *v;       // live K/V (token-major [tokens][H][D])
  const uint8_t *cache;      // prefix cache arena (denoise) or null
  int H, h, kend, kv_tok, lp;
  int64_t k_off, v_off;
  float k_scale, v_scale;    // fp8 dequantisation scales of this (request, head)
};

template <int D, int SRC>
struct Stage {
  uint4 kr[Cfg<D>::KPASS];
  uint4 vr[Cfg<D>::KPT];

  __device__ __forceinline__ static uint4 fetch(const __bf16 *live, int64_t coff, int key,
                                                int chunk, const TileArgs &a) {
    if (key >= a.kend) return make_uint4(0, 0, 0, 0);
    if (SRC != SRC_ONE && key < a.lp) {
      if (SRC == SRC_CACHE_BF16) {
        const uint8_t *p = a.cache + coff + ((int64_t)(a.h * a.lp + key) * D + chunk * 8) * 2;
        return *reinterpret_cast<const uint4 *>(p);
      } else {
        const uint8_t *p = a.cache + coff + (int64_t)(a.h * a.lp + key) * D + chunk * 8;
        const uint2 raw = *reinterpret_cast<const uint2 *>(p);
        return make_uint4(raw.x, raw.y, 0, 0);
      }
    }
    const __bf16 *p = live + ((int64_t)(a.kv_tok + key - a.lp) * a.H + a.h) * D + chunk * 8;
    return *reinterpret_cast<const uint4 *>(p);
  }

  __device__ __forceinline__ void load(int kt, const TileArgs &a) {
    using C = Cfg<D>;
    const int t = threadIdx.x;
    const int kc = t % C::CH, kr0 = t / C::CH;
#pragma unroll
    for (int i = 0; i < C::KPASS; ++i)
      kr[i] = fetch(a.k, a.k_off, kt * BN + kr0 + i * C::KROWS, kc, a);
    const int dg = t % C::CH, kg = t / C::CH;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) vr[i] = fetch(a.v, a.v_off, kt * BN + kg * C::KPT + i, dg, a);
  }

  __device__ __forceinline__ void store(int kt, const TileArgs &a, __bf16 *Ks, __bf16 *Vt) {
    using C = Cfg<D>;
    const int t = threadIdx.x;
    const int kc = t % C::CH, kr0 = t / C::CH;
#pragma unroll
    for (int i = 0; i < C::KPASS; ++i) {
      const int row = kr0 + i * C::KROWS;
      uint4 val = kr[i];
      if (SRC == SRC_CACHE_FP8 && kt * BN + row < a.lp) val = dequant8(val.x, val.y, a.k_scale);
      *reinterpret_cast<uint4 *>(Ks + row * D + ((kc ^ (row & (C::CH - 1))) << 3)) = val;
    }
    const int dg = t % C::CH, kg = t / C::CH;
    uint4 vals[C::KPT];
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      vals[i] = vr[i];
      if (SRC == SRC_CACHE_FP8 && kt * BN + kg * C::KPT + i < a.lp)
        vals[i] = dequant8(vals[i].x, vals[i].y, a.v_scale);
    }
    const int pos = vpos(kg * C::KPT);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int j = d >> 1;
      uint32_t w[C::KPT / 2];
#pragma unroll
      for (int q = 0; q < C::KPT / 2; ++q) {
        const uint32_t A = word(vals[2 * q], j), B = word(vals[2 * q + 1], j);
        w[q] = (d & 1) ? ((A >> 16) | (B & 0xffff0000u)) : ((A & 0xffffu) | (B << 16));
      }
      const int dim = dg * 8 + d;
      __bf16 *dst = Vt + dim * BN + (((pos >> 3) ^ (dim & 7)) << 3) + (pos & 7);
      if (C::KPT == 4)
        *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1 % (C::KPT / 2)]);
      else
        *reinterpret_cast<uint32_t *>(dst) = w[0];
    }
  }
};

// One key tile for one wavefront: scores, online softmax, PV.
template <int D>
__device__ __forceinline__ void compute_tile(const __bf16 *Ks, const __bf16 *Vt,
                                             const bf16x8_t (&qf)[Cfg<D>::QS],
                                             f32x16_t (&o)[Cfg<D>::DB], float &m_run,
                                             float &l_run, int kt, int kend, float c) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;

  f32x16_t s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int st = 0; st < C::QS; ++st) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kb * 32 + j;
      const int chunk = 2 * st + g;
      const bf16x8_t a =
          *reinterpret_cast<const bf16x8_t *>(Ks + row * D + ((chunk ^ (row & (C::CH - 1))) << 3));
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
    }
  }

  if ((kt + 1) * BN > kend) {   // the PARTIAL tile: keys at or past kend do not exist
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * BN + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= kend) s[kb][r] = -INFINITY;
      }
  }

  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mc = mx * c;
  if (__any(mc > m_run + TAU)) {
    const float mn = fmaxf(m_run, mc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }

  bf16x8_t p[2][2];
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * cc + 2 * t], c, -m_run));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * cc + 2 * t + 1], c, -m_run));
        w[t] = pack_bf16(x0, x1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[t]), ones, l_run,
                                                false);
      }
      uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
      p[kb][cc] = __builtin_bit_cast(bf16x8_t, u);
    }

#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int dim = db * 32 + j;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int chunk = 4 * kb + 2 * cc + g;
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t *>(Vt + dim * BN + ((chunk ^ (dim & 7)) << 3));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[kb][cc], o[db], 0, 0, 0);
      }
  }
}

template <int D, int SRC>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(
    const int32_t *__restrict__ sched, const qi_tile *__restrict__ tiles, int H,
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ o, const uint8_t *__restrict__ cache, float c) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2 * C::TILE];

  const int item = sched[blockIdx.x];
  if (item < 0) return;   // schedule padding
  const qi_tile tl = tiles[item / H];
  const int h = item % H;

  TileArgs a;
  a.k = k;
  a.v = v;
  a.cache = cache;
  a.H = H;
  a.h = h;
  a.kend = tl.kend;
  a.kv_tok = tl.kv_tok;
  a.lp = tl.lp;
  a.k_off = tl.k_off;
  a.v_off = tl.v_off;
  a.k_scale = 1.0f;
  a.v_scale = 1.0f;
  if (SRC == SRC_CACHE_FP8) {
    const float *sc = reinterpret_cast<const float *>(cache + tl.s_off);
    a.k_scale = sc[h];
    a.v_scale = sc[H + h];
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  const int row = wave * 32 + j;               // row inside the tile
  const bool active = wave * 32 < tl.nrows;    // wavefront has at least one real row

  bf16x8_t qf[C::QS];
  {
    const bool valid = row < tl.nrows;
    const __bf16 *qp = q + ((int64_t)(tl.q_tok + row) * H + h) * D + 8 * g;
#pragma unroll
    for (int st = 0; st < C::QS; ++st) {
      uint4 u = valid ? *reinterpret_cast<const uint4 *>(qp + 16 * st) : make_uint4(0, 0, 0, 0);
      qf[st] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  f32x16_t acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int ntiles = (tl.kend + BN - 1) / BN;
  Stage<D, SRC> st;
  st.load(0, a);
  st.store(0, a, lds[0], lds[0] + C::TILE);
  if (ntiles > 1) st.load(1, a);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    if (active)
      compute_tile<D>(lds[cur], lds[cur] + C::TILE, qf, acc, m_run, l_run, kt, tl.kend, c);
    if (kt + 1 < ntiles) st.store(kt + 1, a, lds[cur ^ 1], lds[cur ^ 1] + C::TILE);
    if (kt + 2 < ntiles) st.load(kt + 2, a);
    __syncthreads();
  }

  if (!active) return;
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / lt;
  if (row < tl.nrows) {
    __bf16 *op = o + ((int64_t)(tl.q_tok + row) * H + h) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int dim = db * 32 + 8 * aa + 4 * g;
        uint2 u;
        u.x = pack_bf16(acc[db][4 * aa] * inv, acc[db][4 * aa + 1] * inv);
        u.y = pack_bf16(acc[db][4 * aa + 2] * inv, acc[db][4 * aa + 3] * inv);
        *reinterpret_cast<uint2 *>(op + dim) = u;
      }
  }
}

template <int D, int SRC>
qi_status launch(const qi_plan *p, int call, const void *q, const void *k, const void *v,
                 void *o, const void *cache, hipStream_t s) {
  const uint8_t *ws = static_cast<const uint8_t *>(p->d_ws);
  const float c = (float)(1.4426950408889634 / std::sqrt((double)D));   // log2(e)/sqrt(D)
  hipLaunchKernelGGL((attn_fwd_kernel<D, SRC>), dim3(p->sched_len[call]), dim3(NT), 0, s,
                     reinterpret_cast<const int32_t *>(ws + p->sched_off[call]),
                     reinterpret_cast<const qi_tile *>(ws + p->tiles_off[call]), p->H,
                     static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k),
                     static_cast<const __bf16 *>(v), static_cast<__bf16 *>(o),
                     static_cast<const uint8_t *>(cache), c);
  return hipGetLastError() == hipSuccess ? QI_OK : QI_ERR_HIP;
}

}  // namespace

qi_status qi_launch_attention(const qi_plan *p, int call, const void *q, const void *k,
                              const void *v, void *o, const void *cache, void *stream) {
  if (p->sched_len[call] == 0) return QI_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int src = call != QI_CALL_DENOISE ? SRC_ONE
                                          : (p->kv == QI_KV_BF16 ? SRC_CACHE_BF16 : SRC_CACHE_FP8);
  if (p->D == 128) {
    if (src == SRC_ONE) return launch<128, SRC_ONE>(p, call, q, k, v, o, cache, s);
    if (src == SRC_CACHE_BF16) return launch<128, SRC_CACHE_BF16>(p, call, q, k, v, o, cache, s);
    return launch<128, SRC_CACHE_FP8>(p, call, q, k, v, o, cache, s);
  }
  if (src == SRC_ONE) return launch<64, SRC_ONE>(p, call, q, k, v, o, cache, s);
  if (src == SRC_CACHE_BF16) return launch<64, SRC_CACHE_BF16>(p, call, q, k, v, o, cache, s);
  return launch<64, SRC_CACHE_FP8>(p, call, q, k, v, o, cache, s);
}
