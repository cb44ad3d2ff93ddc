// Block-causal attention forward for gfx950 (CDNA4), bf16 MFMA, fp32 online softmax.
//
// One workgroup owns one (request, head, row tile); each wavefront owns 32 query rows and
// keeps its Q fragments and its O accumulator in registers for the whole key loop.  Row
// tiles never cross a block, so every row of a tile sees the same key prefix [0, kend)
// (block-causal rule: a row of block b sees keys of blocks 0..b; ThakiCloud blog
// "Qwen-Image-2.1 vLLM-Omni day 0", section "Serving architecture: the cross-step prefix
// KV cache").  Key tiles past kend are never visited (EMPTY tiles skipped), the one
// straddling kend is masked (PARTIAL), the others run unmasked (FULL).
//
// Key sources.  In the full and prefix calls K/V come from one token-major tensor.  In
// the denoising call keys [0, lp) come from the prefix cache (head-major, bf16 or E4M3FN
// codes with a per-head scale) and keys [lp, kend) from the live image K/V; a key tile
// straddling lp gathers from both.  Key tiles start at key 0 in every call and the
// arithmetic does not depend on where a key came from, so on a bf16 cache the denoising
// call reproduces the full call's image rows bit for bit -- the exact reuse the vLLM
// recipe "Qwen/Qwen-Image-2.1" states in its "Prefix KV cache" section.
//
// Per key tile (64 keys) and wavefront:
//   S^T = K Q^T      16 x v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q in VGPRs)
//   lane (query j = lane%32, half g = lane/32) then holds 32 scores of its query row
//   online softmax in the log2 domain: x = s * log2(e)/sqrt(D) - m, p = 2^x.  The
//   running max m is only raised when a row's tile max exceeds it by more than 8 (then
//   every row of the wavefront is rescaled exactly); otherwise p <= 2^8, which bf16 and
//   fp32 hold without loss of relative precision.  The result is the same softmax.
//   O^T += V^T P^T   16 x MFMA (A = V^T, read from the natural [key][dim] V tile with
//   the gfx950 LDS transpose read ds_read_b64_tr_b16; B = P packed to bf16 in VGPRs);
//   the key order inside each 16-key MFMA step is permuted consistently on both
//   operands so that P never leaves the lane that computed it.
// LDS: K and V tiles [64 keys][D] bf16, XOR-swizzled in 16-byte chunks so that every LDS
// access of the kernel is free of bank conflicts on the 64-bank gfx950 LDS (16 lanes per
// cycle for 16-byte reads, 32 lanes per cycle for 8-byte reads).
//
// Every call and cache type: a workgroup of 8 wavefronts (two per SIMD) in two groups of
// four that alternate an MFMA phase and a VALU phase (softmax, tile loads) between
// workgroup barriers ("ping-pong"), so each SIMD always has one wavefront feeding the
// matrix core and one feeding the vector ALU.  Row tiles of 256 rows give each wavefront
// its own 32 rows; row tiles of 128 rows give two wavefronts the same rows, the two
// groups split the key tiles, and the two partial softmax states are merged through LDS
// in a fixed order.  bf16 rows go straight from global memory into LDS; tiles wholly in
// an E4M3FN cache land there as codes and are converted to bf16 code values by the
// wavefront that loaded them, one VALU phase later, with the per-head scales folded into
// the logit scale (K) and into P (V).
#include <hip/hip_runtime.h>
#include <math.h>

#include "qi_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BN = QI_KERNEL_BN;
constexpr int NT = 512;                 // 8 wavefronts
constexpr float TAU = 8.0f;   // lazy-rescale threshold, log2 units

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;
// MFMA operands read ahead of their MFMA in the MFMA phase
#ifndef QI_QK_AHEAD
#define QI_QK_AHEAD 4
#endif
#ifndef QI_PV_AHEAD
#define QI_PV_AHEAD 2
#endif
constexpr int QK_AHEAD = QI_QK_AHEAD, PV_AHEAD = QI_PV_AHEAD;

enum { SRC_ONE = 0, SRC_CACHE_BF16 = 1, SRC_CACHE_FP8 = 2, SRC_CACHE_FP8V = 3 };

// Whether cached K (which = 0) or V (which = 1) rows are E4M3FN codes for a source kind.
__host__ __device__ constexpr bool coded(int src, int which) {
  return src == SRC_CACHE_FP8 || (src == SRC_CACHE_FP8V && which == 1);
}

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;           // 16-byte chunks per K/V row
  static constexpr int QS = D / 16;          // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;          // 32-wide blocks of the output
  static constexpr int IPW = D / 32;         // 1 KiB direct V loads per wavefront per tile
  static constexpr int RPK = 512 / D;        // V rows per 1 KiB
  static_assert(IPW * RPK * 4 == BN, "tile shape");
  // K tile: rows of 2D bytes; logical 16-byte chunk c of row r sits at chunk c ^ ks(r), so
  // the 16 consecutive rows one 16-byte MFMA-operand read touches (one chunk each) fall in
  // 16 distinct bank groups.
  static constexpr int KHALF_N = D / 16;                 // 1 KiB loads per 32-row half
  static constexpr int KHALF = KHALF_N * 1024;           // bytes per half
  static constexpr int KTILE = BN * D;                   // bf16 elements per K tile
  static constexpr int VTILE = BN * D;                   // bf16 elements per V tile
  static_assert(2 * KHALF == KTILE * 2, "two 32-row halves make a K tile");
  __device__ static constexpr int ks(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // V tile: rows of 2D bytes; the 64-byte quarter q of row r sits at quarter q ^ vq(r), so
  // the transpose reads (32 lanes: 64 bytes of one quarter in each of 4 consecutive rows)
  // hit 64 distinct banks and a lane needs one base address per quarter.
  __device__ static constexpr int vq(int r) { return D == 128 ? (r & 3) : ((r >> 1) & 1); }
  // byte offsets of 16-byte chunk c of row r
  __device__ static constexpr int koff(int r, int c) { return r * 2 * D + ((c ^ ks(r)) << 4); }
  __device__ static constexpr int voff(int r, int c) { return r * 2 * D + ((c ^ (vq(r) << 2)) << 4); }
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};   // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, v);
}

// max over the two lanes (j, j + 32) holding one query row
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// 8 E4M3FN codes -> 8 bf16 of the code values themselves (exact: every E4M3FN value is a
// bf16 value; the scaled conversion with scale 1)
__device__ __forceinline__ uint4 codes8(uint32_t lo, uint32_t hi) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return r;
}

struct TileArgs {
  const __bf16 *k, *v;       // live K/V (token-major [tokens][H][D])
  const uint8_t *cache;      // prefix cache arena (denoise) or null
  int H, h, kend, kv_tok, lp;
  int t0;                    // first key tile the workgroup visits (its key chunk)
  int64_t k_off, v_off;
  float k_scale, v_scale;    // fp8 dequantisation scales of this (request, head)
};

// Where a key tile comes from: wholly from the live tensor, wholly from the cache, or
// mixed / partly past kend (per-row choice).
enum { LIVE = 0, CACHED = 1, MIXED = 2 };
template <int SRC>
__device__ __forceinline__ int tile_kind(int kt, const TileArgs &a) {
  const int k0 = kt * BN, k1 = k0 + BN;
  if (k1 > a.kend) return MIXED;
  if (SRC == SRC_ONE || k0 >= a.lp) return LIVE;
  return k1 <= a.lp ? CACHED : MIXED;
}

// ---------------------------------------------------------------------------------------
// Direct global -> LDS tile loads (bf16 rows).  Every load instruction fills 1 KiB of
// LDS, lane l the 16 bytes at offset 16 l, so the layout is set on the global side: each
// lane fetches the key row and chunk that belongs at its LDS slot.
//   K and V: KiB kib of a tile holds rows kib * RPK + l / CH; physical chunk p of row r is
//      logical chunk p ^ ks(r) (K) or p ^ (vq(r) << 2) (V).  vq depends on l only (kib * RPK
//      is a multiple of 4); ks on l and kib % 4 (D=128) or kib % 2 (D=64).
// A group of four wavefronts loads either whole tiles (HALF = false) or one half of the
// rows of each tile (HALF = true, the other group loads the other half); wavefront w of
// the group issues a run of consecutive K and V instructions.  Instruction indices are
// wavefront-uniform, so the LDS destination is a scalar; the per-lane part of every
// global address is a 32-bit offset computed once, added to a scalar base per tile.  Key
// tiles that straddle the cache/live boundary or kend take a slower per-lane path.  Used
// for bf16 rows only: tiles of an E4M3FN cache tensor go through Coded / sync_tile.
template <int D, int SRC, bool HALF>
struct Direct {
  using C = Cfg<D>;
  static constexpr int NI = HALF ? 2 * C::IPW : 4 * C::IPW;        // instructions per tensor
  static constexpr int U = NI / 4;                                 // per wavefront
  static constexpr int KP = D == 128 ? 4 : 2;   // K lane offsets repeat every KP instructions
  int w;                                  // wavefront index in the group (uniform)
  uint32_t k_live[U], k_cache[U];         // K: lane offset from the instruction's first row
  uint32_t v_live, v_cache;               // V: lane offset from the instruction's first row

  __device__ __forceinline__ void init(const TileArgs &a) {
    w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3;
    const int l = threadIdx.x & 63;
    const int vr = l / C::CH;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // instruction U w + u; only its residue mod KP matters (half offsets are multiples)
      const int r = ((U * w + u) % KP) * C::RPK + vr;
      const int kc = (l % C::CH) ^ C::ks(r);
      k_live[u] = (uint32_t)(vr * a.H * D + kc * 8) * 2u;
      k_cache[u] = (uint32_t)(vr * D + kc * 8) * 2u;
    }
    const int vc = (l % C::CH) ^ (C::vq(vr) << 2);
    v_live = (uint32_t)(vr * a.H * D + vc * 8) * 2u;
    v_cache = (uint32_t)(vr * D + vc * 8) * 2u;
  }

  __device__ __forceinline__ static void load(const char *src, __bf16 *tile, int dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(reinterpret_cast<char *>(tile) + dst), 16,
                                     0, 0);
  }

  // key row `key` of this (request, head): cache below lp, else live
  __device__ __forceinline__ static const char *row_ptr(const TileArgs &a, const __bf16 *live,
                                                        int64_t coff, int key) {
    if (SRC != SRC_ONE && key < a.lp)
      return reinterpret_cast<const char *>(a.cache + coff) + (int64_t)(a.h * a.lp + key) * D * 2;
    return reinterpret_cast<const char *>(live + ((int64_t)(a.kv_tok + key - a.lp) * a.H + a.h) * D);
  }

  // loads of tile kt of K (IS_K; live = a.k, coff = a.k_off) or V; HALF: rows of half hf
  template <bool IS_K>
  __device__ __forceinline__ void issue(int kt, const TileArgs &a, const __bf16 *live,
                                        int64_t coff, __bf16 *tile, int hf = 0) const {
    const int k0 = kt * BN + (HALF ? 32 * hf : 0);   // first key of the loaded rows
    const int kd = tile_kind<SRC>(kt, a);
    if (kd == LIVE || (SRC != SRC_ONE && kd == CACHED)) {
      const bool lv = kd == LIVE;
      const char *base = row_ptr(a, live, coff, k0);     // uniform
      const uint32_t rstride = lv ? a.H * D * 2 : D * 2;   // bytes between key rows
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ins = U * w + u;   // instruction within the loaded rows
        const int dst = (HALF ? hf * (NI * 1024) : 0) + ins * 1024;
        const uint32_t lo = IS_K ? (lv ? k_live[u] : k_cache[u]) : (lv ? v_live : v_cache);
        load(base + (uint32_t)(ins * C::RPK) * rstride + lo, tile, dst);
      }
    } else {
      // mixed sources or rows past kend (those load key kend - 1: finite values of this
      // request, masked later)
      const int l = threadIdx.x & 63;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ins = U * w + u;
        const int r = ins * C::RPK + l / C::CH;
        const int ch = (l % C::CH) ^ (IS_K ? C::ks(r) : (C::vq(r) << 2));
        const int dst = (HALF ? hf * (NI * 1024) : 0) + ins * 1024;
        const int key = min(k0 + r, a.kend - 1);
        load(row_ptr(a, live, coff, key) + ch * 16, tile, dst);
      }
    }
  }
};

// ---------------------------------------------------------------------------------------
// E4M3FN cache tiles in the ping-pong kernel.  A key tile lying wholly in an E4M3FN cache
// tensor is loaded as codes (1 byte per element, rows contiguous in the head-major cache)
// straight into a landing buffer, and converted to bf16 code values (exact) in the ring
// slot by the same wavefront in its next VALU phase, after its wait.  Each group lands its
// rows (HALF: its 32-row half of the tile; else the whole tile) in its own landing region
// of BN x D bytes.  A wavefront converts exactly the bytes it loaded, so no barrier is
// needed between landing and conversion.  Tiles that mix cached and live keys, or reach
// past kend, take a synchronous per-lane path instead (sync_tile).
template <int D, bool HALF>
struct Coded {
  static constexpr int ROWS = HALF ? 32 : 64;            // rows one group loads per tile
  static constexpr int NIC = ROWS * D / 1024;            // 1 KiB code loads per group
  static constexpr int PER = (NIC + 3) / 4;              // per wavefront, at most
  static constexpr int REGION = BN * D;                  // landing bytes per group
  int w;   // wavefront index in the group (uniform)

  __device__ __forceinline__ void init() { w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3; }

  // codes of tile kt (the group's rows) from cache tensor `coff` into the group's region
  __device__ __forceinline__ void issue(int kt, const TileArgs &a, int64_t coff, uint8_t *land,
                                        int hf) const {
    const int k0 = kt * BN + (HALF ? 32 * hf : 0);
    const char *base = reinterpret_cast<const char *>(a.cache + coff) + (int64_t)(a.h * a.lp + k0) * D;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int ins = w + 4 * u;
      if (ins < NIC)
        __builtin_amdgcn_global_load_lds(base + ins * 1024 + lane * 16,
                                         (lds_void_t *)(land + hf * REGION + ins * 1024), 16, 0, 0);
    }
  }

  // the codes this wavefront landed for tile rows of half hf -> bf16 code values in `tile`
  template <bool IS_K>
  __device__ __forceinline__ void convert(const uint8_t *land, __bf16 *tile, int hf) const {
    using C = Cfg<D>;
    const int lane = threadIdx.x & 63;
    char *tb = reinterpret_cast<char *>(tile);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int ins = w + 4 * u;
      if (ins < NIC) {
        const int byte = ins * 1024 + lane * 16;   // 16 codes: row byte / D, chunks c0, c0 + 1
        const uint4 cd = *reinterpret_cast<const uint4 *>(land + hf * REGION + byte);
        const int r = (HALF ? 32 * hf : 0) + byte / D, c0 = (byte % D) / 8;
        *reinterpret_cast<uint4 *>(tb + (IS_K ? C::koff(r, c0) : C::voff(r, c0))) = codes8(cd.x, cd.y);
        *reinterpret_cast<uint4 *>(tb + (IS_K ? C::koff(r, c0 + 1) : C::voff(r, c0 + 1))) =
            codes8(cd.z, cd.w);
      }
    }
  }
};

// Synchronous per-lane load of one tile of a coded cache tensor (the rows of half hf, or
// the whole tile), written to the ring slot in the layout the direct loads produce: cached
// rows as code values (tile wholly cached) or code * scale rounded to bf16 (mixed tile),
// live rows as they are, rows past kend as key kend - 1.  Waits for its loads.
template <int D, int SRC, bool HALF, bool IS_K>
__device__ __forceinline__ void sync_tile(int kt, const TileArgs &a, const __bf16 *live,
                                          int64_t coff, __bf16 *tile, int hf) {
  using C = Cfg<D>;
  constexpr int NI = HALF ? 2 * C::IPW : 4 * C::IPW;   // 1 KiB stores per tensor
  constexpr int U = NI / 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3;
  const int l = threadIdx.x & 63;
  const int k0 = kt * BN + (HALF ? 32 * hf : 0);
  const bool whole = tile_kind<SRC>(kt, a) == CACHED;
  const float scale = IS_K ? a.k_scale : a.v_scale;
  char *tb = reinterpret_cast<char *>(tile);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ins = U * w + u;
    const int r = ins * C::RPK + l / C::CH;
    const int ch = (l % C::CH) ^ (IS_K ? C::ks(r) : (C::vq(r) << 2));
    const int key = min(k0 + r, a.kend - 1);
    uint4 val;
    if (key < a.lp) {
      const uint2 raw = *reinterpret_cast<const uint2 *>(a.cache + coff + (int64_t)(a.h * a.lp + key) * D + ch * 8);
      val = whole ? codes8(raw.x, raw.y) : dequant8(raw.x, raw.y, scale);
    } else {
      val = *reinterpret_cast<const uint4 *>(live + ((int64_t)(a.kv_tok + key - a.lp) * a.H + a.h) * D + ch * 8);
    }
    *reinterpret_cast<uint4 *>(tb + (HALF ? hf * (NI * 1024) : 0) + ins * 1024 + l * 16) = val;
  }
}

// Tile loads of the ping-pong kernel for any source: direct loads for bf16 rows, landing
// and conversion for tiles wholly in an E4M3FN cache tensor, the synchronous path for
// mixed coded tiles.  Scales of coded tiles are folded in: K's into the logit scale (ck),
// V's into P (vsc).
// Tile indices m passed to the loader count from the workgroup's first key tile (a.t0).
template <int D, int SRC, bool HALF>
struct Loader {
  static constexpr bool CK = coded(SRC, 0), CV = coded(SRC, 1);
  Direct<D, SRC, HALF> dm;
  Coded<D, HALF> cm;
  uint8_t *lk, *lv;   // landing buffers of the coded tensors

  __device__ __forceinline__ void init(const TileArgs &a, uint8_t *lk_, uint8_t *lv_) {
    dm.init(a);
    cm.init();
    lk = lk_;
    lv = lv_;
  }
  // before the loop: every tile straight into its ring slot
  template <bool IS_K>
  __device__ __forceinline__ void pro(int m, const TileArgs &a, __bf16 *slot, int hf = 0) {
    m += a.t0;
    if constexpr (IS_K ? CK : CV)
      sync_tile<D, SRC, HALF, IS_K>(m, a, IS_K ? a.k : a.v, IS_K ? a.k_off : a.v_off, slot, hf);
    else
      dm.template issue<IS_K>(m, a, IS_K ? a.k : a.v, IS_K ? a.k_off : a.v_off, slot, hf);
  }
  // in the loop: cached coded tiles land and are converted two periods later
  template <bool IS_K>
  __device__ __forceinline__ void issue(int m, const TileArgs &a, __bf16 *slot, int hf = 0) {
    m += a.t0;
    if constexpr (IS_K ? CK : CV) {
      const int kd = tile_kind<SRC>(m, a);
      if (kd == CACHED) {
        cm.issue(m, a, IS_K ? a.k_off : a.v_off, IS_K ? lk : lv, hf);
        return;
      }
      if (kd == MIXED) {
        sync_tile<D, SRC, HALF, IS_K>(m, a, IS_K ? a.k : a.v, IS_K ? a.k_off : a.v_off, slot, hf);
        return;
      }
    }
    dm.template issue<IS_K>(m, a, IS_K ? a.k : a.v, IS_K ? a.k_off : a.v_off, slot, hf);
  }
  // convert tile m if it was landed (the caller knows it was issued two periods ago)
  template <bool IS_K>
  __device__ __forceinline__ void convert(int m, const TileArgs &a, __bf16 *slot, int hf = 0) const {
    m += a.t0;
    if constexpr (IS_K ? CK : CV)
      if (tile_kind<SRC>(m, a) == CACHED) cm.template convert<IS_K>(IS_K ? lk : lv, slot, hf);
  }
  __device__ __forceinline__ float ck(int m, const TileArgs &a, float c) const {
    if constexpr (CK) return tile_kind<SRC>(m + a.t0, a) == CACHED ? c * a.k_scale : c;
    return c;
  }
  __device__ __forceinline__ bool vsc(int m, const TileArgs &a) const {
    if constexpr (CV) return tile_kind<SRC>(m + a.t0, a) == CACHED;
    return false;
  }
};

// Workgroup barrier without the implicit wait for outstanding memory operations that
// __syncthreads() adds: the ping-pong loop waits for its own direct loads explicitly,
// two periods after issuing them.  The memory clobber keeps the compiler from moving
// LDS accesses across it; every LDS read before it has been consumed by an MFMA.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

// Wait for this wavefront's LDS operations only (gfx9 s_waitcnt encoding: lgkmcnt 0,
// vmcnt (bits 3:0, 15:14) and expcnt (6:4) at their maxima).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// Wait until at most N of this wavefront's vector-memory loads are outstanding (loads
// complete in issue order); LDS and scalar-memory counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------------------
// Per-wavefront pieces of one key tile.

template <int D>
__device__ __forceinline__ void qk_tile(const __bf16 *Ks, const bf16x8_t (&qf)[Cfg<D>::QS],
                                        f32x16_t (&s)[2]) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  // row j (+32 kb: same swizzle) of the tile, chunk 2 st + g
  const char *kp = reinterpret_cast<const char *>(Ks) + j * 2 * D;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int st = 0; st < C::QS; ++st) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
          kp + kb * C::KHALF + (((2 * st + g) ^ C::ks(j)) << 4));
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
    }
  }
  // schedule: four operand reads ahead, then one read per MFMA, so LDS latency hides
  // behind the matrix core instead of stalling it
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, QK_AHEAD, 0);
#pragma unroll
  for (int i = 0; i < 2 * C::QS - QK_AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, QK_AHEAD, 0);
}

// Keys at or past kend of the PARTIAL tile kt get score -inf.
__device__ __forceinline__ void mask_tile(f32x16_t (&s)[2], int kt, int kend) {
  const int g = (threadIdx.x & 63) >> 5;
  // score (kb, r) of this lane is key kt BN + 32 kb + 8 (r / 4) + 4 g + r % 4: compare the
  // constant part against one per-lane limit
  const int lim = kend - kt * BN - 4 * g;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
}

// c times the row max of a tile's scores (both lanes of the row agree).  Taken before the
// PARTIAL tile is masked: its key rows past kend hold copies of key kend - 1 (see Direct),
// whose score is already in the row, so they cannot change the max.
__device__ __forceinline__ float tile_max(const f32x16_t (&s)[2], float c) {
  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  return pair_max(mx) * c;
}

// Raise the running max to mc when some row of the wavefront exceeds it by more than TAU,
// rescaling O and l exactly.
template <int D>
__device__ __forceinline__ void raise_max(f32x16_t (&o)[Cfg<D>::DB], float &m_run, float &l_run,
                                          float mc) {
  if (__any(mc > m_run + TAU)) {
    const float mn = fmaxf(m_run, mc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
}

// P = 2^(s c - m) in bf16, in the MFMA B-operand order: step (kb, cc) holds keys
// 32kb + 16cc + {4g..4g+3, 8+4g..8+4g+3}, i.e. this lane's score registers 8cc..8cc+7.
// The row sum accumulates the fp32 values before rounding (plain adds: they overlap the
// other wavefront's MFMAs, which v_dot2 does not).
__device__ __forceinline__ void softmax_exp(const f32x16_t (&s)[2], float m_run, float c,
                                            float &l_run, bf16x8_t (&p)[2][2]) {
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
        l_run += x0 + x1;
      }
      uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
      p[kb][cc] = __builtin_bit_cast(bf16x8_t, u);
    }
}

// The same for a tile whose V rows hold code values that still need a scale vs: P holds
// p * vs (2^(s c - m + log2 vs), so P V_codes = p V), the row sum adds p = (p * vs) / vs.
__device__ __forceinline__ void softmax_exp_vscaled(const f32x16_t (&s)[2], float m_run, float c,
                                                    float log2_vs, float inv_vs, float &l_run,
                                                    bf16x8_t (&p)[2][2]) {
  const float sh = log2_vs - m_run;
  float lt = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * cc + 2 * t], c, sh));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * cc + 2 * t + 1], c, sh));
        w[t] = pack_bf16(x0, x1);
        lt += x0 + x1;
      }
      uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
      p[kb][cc] = __builtin_bit_cast(bf16x8_t, u);
    }
  l_run = __builtin_fmaf(lt, inv_vs, l_run);
}

// The exponential step of a tile: bf16 sources as softmax_exp; E4M3FN caches with the
// folded scales (ck: logit scale of the tile, vs: its V rows are code values).
template <bool FP8>
__device__ __forceinline__ void tile_exp(const f32x16_t (&s)[2], float m_run, float ck, bool vs,
                                         float log2_vs, float inv_vs, float &l_run,
                                         bf16x8_t (&p)[2][2]) {
  if constexpr (FP8)
    softmax_exp_vscaled(s, m_run, ck, vs ? log2_vs : 0.0f, vs ? inv_vs : 1.0f, l_run, p);
  else
    softmax_exp(s, m_run, ck, l_run, p);
}

// O^T += V^T P^T.  V^T fragments by transpose reads: in each 16-lane group (i = lane %
// 16), lane i addresses 4 dims (4 (i % 4) + 16 ((lane / 16) & 1) + 32 db) of key row
// (step base + 4 g + i / 4); the read hands lane i those 4 keys at dim (lane % 32) + 32 db.
// Two reads (rows +0 and +8) give the 8 keys of one 16-key step.
template <int D>
__device__ __forceinline__ void pv_tile(const __bf16 *Vs, const bf16x8_t (&p)[2][2],
                                        f32x16_t (&o)[Cfg<D>::DB]) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int i16 = lane & 15;
  // this lane's first row and its 8 bytes inside the dims of each 32-dim block
  const int r0 = 4 * g + (i16 >> 2);
  const int c2 = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
  const char *vp[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
    vp[db] = reinterpret_cast<const char *>(Vs) + C::voff(r0, 4 * db + c2) + 8 * (i16 & 1);
  // the four output blocks are independent accumulation chains: interleave them so that
  // consecutive MFMAs never wait on each other's results
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        i16x4_t h[2];
#pragma unroll
        for (int r8 = 0; r8 < 2; ++r8) {
          // rows r0 + 32 kb + 16 cc + 8 r8 share the quarter placement of row r0
          const char *src = vp[db] + (32 * kb + 16 * cc + 8 * r8) * 2 * D;
          h[r8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(src));
        }
        const i16x8_t both = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, both),
                                                         p[kb][cc], o[db], 0, 0, 0);
      }
  // schedule: two MFMAs' operands (four transpose reads) ahead, then two reads per MFMA
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * PV_AHEAD, 0);
#pragma unroll
  for (int i = 0; i < 4 * C::DB - PV_AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, PV_AHEAD, 0);
}

// ---------------------------------------------------------------------------------------
// Common prologue / epilogue.

// Q through LDS: the wavefront loads its 32 rows (row0 .. row0 + 31 of the tile) straight
// into `stage` with whole rows per load instruction (chunks placed as in a K tile; rows
// past the tile repeat its last row, finite and never stored), waits, and reads its
// MFMA B fragments back: qf[st] holds dims 16 st + 8 g .. + 7 of row j (lane = j + 32 g).
// `stage` must be wavefront-uniform and touched by no other wavefront meanwhile.
template <int D>
__device__ __forceinline__ void issue_q_lds(const __bf16 *q, const qi_tile &tl, int H, int h,
                                            int row0, __bf16 *stage) {
  using C = Cfg<D>;
  constexpr int RPI = 64 / C::CH;   // rows per 64-lane instruction
  const int lane = threadIdx.x & 63;
  const int c = lane % C::CH;
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / C::CH;
    const int tr = min(row0 + r, tl.nrows - 1);
    const __bf16 *src = q + ((int64_t)(tl.q_tok + tr) * H + h) * D + 8 * (c ^ C::ks(r));
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(reinterpret_cast<char *>(stage) + it * 1024),
                                     16, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void read_q_lds(const __bf16 *stage, bf16x8_t (&qf)[Cfg<D>::QS]) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const char *sb = reinterpret_cast<const char *>(stage);
#pragma unroll
  for (int st = 0; st < C::QS; ++st)
    qf[st] = *reinterpret_cast<const bf16x8_t *>(sb + C::koff(lane & 31, 2 * st + (lane >> 5)));
}

// O through LDS: the wavefront normalises its 32 rows (O / l, rounded to bf16), writes
// them into `stage` (32 rows of 2D bytes, chunks placed as in a K tile, so both the
// 8-byte writes and the 16-byte reads are free of bank conflicts) and reads them back row
// by row, so every global store instruction writes whole rows (64 lanes x 16 bytes)
// rather than 16 bytes in each of 32 rows.  row0: the wavefront's first row in the tile;
// rows past the tile are not stored.  Only this wavefront touches `stage`.
template <int D>
__device__ __forceinline__ void store_o_lds(__bf16 *o, const qi_tile &tl, int H, int h, int row0,
                                            const f32x16_t (&acc)[Cfg<D>::DB], float l_run,
                                            __bf16 *stage) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  const float inv = 1.0f / pair_sum(l_run);
  char *sb = reinterpret_cast<char *>(stage);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      uint2 u;   // dims 32 db + 8 aa + 4 g .. + 3 of row j: half g of chunk 4 db + aa
      u.x = pack_bf16(acc[db][4 * aa] * inv, acc[db][4 * aa + 1] * inv);
      u.y = pack_bf16(acc[db][4 * aa + 2] * inv, acc[db][4 * aa + 3] * inv);
      *reinterpret_cast<uint2 *>(sb + C::koff(j, 4 * db + aa) + 8 * g) = u;
    }
  constexpr int RPI = 64 / C::CH;   // rows per 64-lane instruction
  const int c = lane % C::CH;
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / C::CH;
    const uint4 u = *reinterpret_cast<const uint4 *>(sb + C::koff(r, c));
    if (row0 + r < tl.nrows)
      *reinterpret_cast<uint4 *>(o + ((int64_t)(tl.q_tok + row0 + r) * H + h) * D + 8 * c) = u;
  }
}

// A key chunk's unnormalised state of the wavefront's 32 rows (row0 .. row0 + 31 of the
// tile) into partial slot tl.part + h: O as fp32 [row][D] (lane (j, g) writes 16 bytes
// per 8 dims: dims 32 db + 8 aa + 4 g .. + 3 of row j), then m and l per row.
template <int D>
__device__ __forceinline__ void store_part(float *part, const qi_tile &tl, int h, int row0,
                                           const f32x16_t (&acc)[Cfg<D>::DB], float m_run,
                                           float l_run) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  float *slot = part + (size_t)(tl.part + h) * QI_PART_SLOT_FLOATS(D);
  float *orow = slot + (size_t)(row0 + j) * D + 4 * g;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa)
      *reinterpret_cast<float4 *>(orow + 32 * db + 8 * aa) =
          make_float4(acc[db][4 * aa], acc[db][4 * aa + 1], acc[db][4 * aa + 2], acc[db][4 * aa + 3]);
  const float l = pair_sum(l_run);
  if (g == 0) {
    slot[(size_t)QI_ROWS * D + row0 + j] = m_run;
    slot[(size_t)QI_ROWS * D + QI_ROWS + row0 + j] = l;
  }
}

__device__ __forceinline__ TileArgs make_args(const qi_tile &tl, int H, int h, const __bf16 *k,
                                              const __bf16 *v, const uint8_t *cache, bool fp8) {
  TileArgs a;
  a.k = k;
  a.v = v;
  a.cache = cache;
  a.H = H;
  a.h = h;
  a.kend = tl.kend;
  a.t0 = tl.k0 / BN;
  a.kv_tok = tl.kv_tok;
  a.lp = tl.lp;
  a.k_off = tl.k_off;
  a.v_off = tl.v_off;
  a.k_scale = 1.0f;
  a.v_scale = 1.0f;
  if (fp8) {
    const float *sc = reinterpret_cast<const float *>(cache + tl.s_off);
    a.k_scale = sc[h];
    a.v_scale = sc[H + h];
  }
  return a;
}

// ---------------------------------------------------------------------------------------
// Ping-pong kernel.  Eight wavefronts in two groups of four alternate an
// MFMA phase and a VALU phase between workgroup barriers ("periods").  K and V tiles live
// in a ring of four separate LDS arrays per tensor (slot = tile & 3), so that the compiler
// can tell each direct-load target from every buffer being read and never stalls a read
// on an unrelated load; the loops are unrolled by four so every slot index is constant.
// Loads are issued at the end of a group's VALU phase, after that group waited for the
// loads it issued in its previous VALU phase (and converted the code tiles among them);
// the next barrier publishes them.  A code tile reaches its ring slot two periods after
// its load was issued, as early as a direct load is waited for, so the schedule of first
// reads is the same for both.

template <int P> struct Slot { static constexpr int value = P; };

struct Ring {
  __bf16 *K0, *K1, *K2, *K3, *V0, *V1, *V2, *V3;
  uint8_t *LK, *LV;   // landing buffers of E4M3FN code tiles (null when unused)
};
#define QI_RING(r, arr, i) \
  ((i) == 0 ? (r).arr##0 : (i) == 1 ? (r).arr##1 : (i) == 2 ? (r).arr##2 : (r).arr##3)

// K slot i for a wavefront-uniform run-time i.  Selects of pointer values, not of the
// members' addresses: the ring must stay in registers, since the backend cannot emit a
// memory copy of LDS addresses.
__device__ __forceinline__ __bf16 *pick4(int i, __bf16 *p0, __bf16 *p1, __bf16 *p2, __bf16 *p3) {
  __bf16 *const lo = (i & 1) ? p1 : p0;
  __bf16 *const hi = (i & 1) ? p3 : p2;
  return (i & 2) ? hi : lo;
}
__device__ __forceinline__ __bf16 *ring_k(const Ring &r, int i) {
  return pick4(i, r.K0, r.K1, r.K2, r.K3);
}

// Q staging before the key loop: wavefront w uses half w & 1 of slot K3, V1, V2 or V3
// (w >> 1), the slots the prologue leaves free.
template <int D>
__device__ __forceinline__ __bf16 *q_stage(const Ring &r) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return pick4(w >> 1, r.K3, r.V1, r.V2, r.V3) + (w & 1) * 32 * D;
}

// Row tiles of more than 128 rows: wavefront w owns rows 32w..32w+31 and every key tile
// is read by all eight wavefronts (group 0 = waves 0..3, group 1 = waves 4..7).
//   period 2t:   group 0 MFMA phase t: S = QK^T(K_t) (t < n), O += PV(V_{t-1}) (t >= 1),
//                                     then the row max of S
//                group 1 VALU phase:  raise the max, P = exp of tile t-1; waits; loads its
//                                     halves of K_{t+2} (t >= 1), V_{t+1}
//   period 2t+1: group 1 MFMA phase t; group 0 VALU phase: the same for tile t; waits;
//                                     loads its halves of K_{t+3}, V_{t+2}
// Group g loads half g of each tile's rows.  K_0..K_2 and V_0 are loaded before period 0,
// together with each wavefront's Q rows, staged in the slots still free (K3, V1..V3);
// V_1 follows once every Q stage has been read: group 1 loads its half in period 0, group
// 0 in period 1.  A half tile issued in period p is waited for at the end of p+2 and first
// read in period >= p+3 (>= p+4 in the steady state); the slots it overwrites (K_{m-4},
// V_{m-4}) were last read in p-1.
template <int D, int SRC>
__device__ __forceinline__ void pp_rows256(const Ring &r, const qi_tile &tl, int H, int h,
                                           const TileArgs &a, const __bf16 *q, __bf16 *o,
                                           float *part, float c) {
  using C = Cfg<D>;
  const int wave = threadIdx.x >> 6;
  const int group = wave >> 2;
  const bool active = wave * 32 < tl.nrows;   // the wavefront's rows exist

  const int n = (tl.k1 - tl.k0 + BN - 1) / BN;   // key tiles of the chunk
  constexpr bool FP8 = SRC == SRC_CACHE_FP8 || SRC == SRC_CACHE_FP8V;
  Loader<D, SRC, true> ld;
  ld.init(a, r.LK, r.LV);
  __bf16 *const qst = q_stage<D>(r);
  issue_q_lds<D>(q, tl, H, h, wave * 32, qst);
  ld.template pro<true>(0, a, r.K0, group);
  if (n > 1) ld.template pro<true>(1, a, r.K1, group);
  if (n > 2) ld.template pro<true>(2, a, r.K2, group);
  ld.template pro<false>(0, a, r.V0, group);
  const float log2_vs = FP8 ? __builtin_log2f(a.v_scale) : 0.0f;
  const float inv_vs = FP8 ? 1.0f / a.v_scale : 1.0f;
  f32x16_t acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[db][rr] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  __builtin_amdgcn_s_waitcnt(0);
  bf16x8_t qf[C::QS];
  read_q_lds<D>(qst, qf);
  wait_lds();
  bar();   // every Q stage read: V1 may be loaded (group 1 in period 0, group 0 in period 1)

  f32x16_t s[2];
  bf16x8_t p[2][2];
  float mc = 0.0f;   // c times the row max of the tile in s, taken in the MFMA phase
  auto tile = [&](auto slot, int t) {
    constexpr int T = decltype(slot)::value;   // t & 3
    // MFMA phase: S of tile t, then O += PV of tile t - 1 with the row max of S taken
    // meanwhile; the running max is raised after that PV (and before tile t's exp)
    auto mfma = [&]() {
      __builtin_amdgcn_s_setprio(1);
      if (active) {
        if (t < n) qk_tile<D>(QI_RING(r, K, T), qf, s);
        if (t >= 1) pv_tile<D>(QI_RING(r, V, (T + 3) & 3), p, acc);
        mc = tile_max(s, ld.ck(t, a, c));   // stale when t == n: unused
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // period 2t
    if (group == 0) {
      mfma();
    } else {
      if (active && t >= 1 && t <= n) {
        raise_max<D>(acc, m_run, l_run, mc);
        if ((a.t0 + t) * BN > tl.kend) mask_tile(s, a.t0 + t - 1, tl.kend);   // PARTIAL
        tile_exp<FP8>(s, m_run, ld.ck(t - 1, a, c), ld.vsc(t - 1, a), log2_vs, inv_vs, l_run, p);
      }
      __builtin_amdgcn_s_waitcnt(0);
      // coded tiles this group landed two periods ago: K_{t+1}, V_t
      if (t >= 2 && t + 1 < n) ld.template convert<true>(t + 1, a, QI_RING(r, K, (T + 1) & 3), 1);
      if (t >= 1 && t < n) ld.template convert<false>(t, a, QI_RING(r, V, T), 1);
      if (t >= 1 && t + 2 < n) ld.template issue<true>(t + 2, a, QI_RING(r, K, (T + 2) & 3), 1);
      if (t + 1 < n) ld.template issue<false>(t + 1, a, QI_RING(r, V, (T + 1) & 3), 1);
      if (FP8) wait_lds();   // converted tiles are written before the barrier
    }
    bar();
    // period 2t+1
    if (group == 1) {
      mfma();
    } else {
      if (active && t < n) {
        raise_max<D>(acc, m_run, l_run, mc);
        if ((a.t0 + t + 1) * BN > tl.kend) mask_tile(s, a.t0 + t, tl.kend);   // PARTIAL
        tile_exp<FP8>(s, m_run, ld.ck(t, a, c), ld.vsc(t, a), log2_vs, inv_vs, l_run, p);
      }
      __builtin_amdgcn_s_waitcnt(0);
      // coded tiles this group landed two periods ago: K_{t+2}, V_{t+1}
      if (t >= 1 && t + 2 < n) ld.template convert<true>(t + 2, a, QI_RING(r, K, (T + 2) & 3), 0);
      if (t >= 1 && t + 1 < n) ld.template convert<false>(t + 1, a, QI_RING(r, V, (T + 1) & 3), 0);
      if (t + 3 < n) ld.template issue<true>(t + 3, a, QI_RING(r, K, (T + 3) & 3), 0);
      if (t + 2 < n) ld.template issue<false>(t + 2, a, QI_RING(r, V, (T + 2) & 3), 0);
      // V_1's half 0 shares this period with V_2's, so it skips the landing buffer
      if (T == 0 && t == 0 && n > 1) ld.template pro<false>(1, a, r.V1, 0);
      if (FP8) wait_lds();   // converted tiles are written before the barrier
    }
    bar();
  };
  for (int t0 = 0; t0 <= n; t0 += 4) {
    tile(Slot<0>(), t0);
    if (t0 + 1 <= n) tile(Slot<1>(), t0 + 1);
    if (t0 + 2 <= n) tile(Slot<2>(), t0 + 2);
    if (t0 + 3 <= n) tile(Slot<3>(), t0 + 3);
  }
  // the ring is free: every load was waited for and every read consumed before the last
  // barrier; wavefront w stages its rows in half w & 1 of K slot w >> 1
  if (active) {
    if (tl.part >= 0)
      store_part<D>(part, tl, h, wave * 32, acc, m_run, l_run);
    else
      store_o_lds<D>(o, tl, H, h, wave * 32, acc, l_run,
                     ring_k(r, wave >> 1) + (wave & 1) * 32 * D);
  }
}

// Row tiles of at most 128 rows: wavefronts w and w+4 hold the same 32 rows and the two
// groups split the key tiles (tile t belongs to group t & 1).  Period p = 0 .. n+1:
//   MFMA group (p & 1):       S = QK^T(K_p) if p < n;  O += PV(V_{p-2}, P) if p >= 2;
//                             the row max of S
//   VALU group ((p + 1) & 1): raise the max, P = exp of tile p-1 if 1 <= p <= n; waits for its
//                             loads of two periods ago; loads K_{p+3}, V_{p+1} (its own
//                             MFMA phase reads them in period p+3), overwriting K_{p-1}
//                             and V_{p-3}, last read in period p-1.
// K_0, K_1, K_2 and V_0 are loaded before period 0, with every wavefront's copy of its Q
// rows staged in K3, V1..V3.  Afterwards group 1 stores its (m, l, O) in LDS and group 0
// merges them into its own (fixed order).
template <int D, int SRC>
__device__ __forceinline__ void pp_rows128(const Ring &r, const qi_tile &tl, int H, int h,
                                           const TileArgs &a, const __bf16 *q, __bf16 *o,
                                           float *part, float c) {
  using C = Cfg<D>;
  const int wave = threadIdx.x >> 6;
  const int group = wave >> 2;
  const bool active = (wave & 3) * 32 < tl.nrows;   // the wavefront's rows exist

  const int n = (tl.k1 - tl.k0 + BN - 1) / BN;   // key tiles of the chunk
  constexpr bool FP8 = SRC == SRC_CACHE_FP8 || SRC == SRC_CACHE_FP8V;
  Loader<D, SRC, false> ld;   // whole tiles; coded ones land in the group's region
  ld.init(a, r.LK, r.LV);
  __bf16 *const qst = q_stage<D>(r);   // both groups load their copy of the rows
  issue_q_lds<D>(q, tl, H, h, (wave & 3) * 32, qst);
  if (group == 0) ld.template pro<true>(0, a, r.K0);
  if (group == 1 && n > 1) ld.template pro<true>(1, a, r.K1);
  if (group == 0 && n > 2) ld.template pro<true>(2, a, r.K2);
  if (group == 1) ld.template pro<false>(0, a, r.V0);
  const float log2_vs = FP8 ? __builtin_log2f(a.v_scale) : 0.0f;
  const float inv_vs = FP8 ? 1.0f / a.v_scale : 1.0f;
  f32x16_t acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[db][rr] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  if constexpr (FP8) {
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    // group 0: Q and K_0 (K_2, issued after them, is waited for at the end of its first
    // VALU phase); group 1: Q only (K_1 and V_0 likewise)
    constexpr int U = decltype(ld.dm)::U;
    if (group == 0) {
      if (n > 2) wait_vm<U>();
      else wait_vm<0>();
    } else {
      if (n > 1) wait_vm<2 * U>();
      else wait_vm<U>();
    }
  }
  bf16x8_t qf[C::QS];
  read_q_lds<D>(qst, qf);
  wait_lds();
  bar();   // every Q stage read: its slots may be loaded

  f32x16_t s[2];
  bf16x8_t p[2][2];
  float mc = 0.0f;   // c times the row max of the tile in s, taken in the MFMA phase
  auto period = [&](auto slot, int per) {
    constexpr int P = decltype(slot)::value;   // per & 3
    if ((P & 1) == group) {
      __builtin_amdgcn_s_setprio(1);
      if (active) {
        if (per < n) qk_tile<D>(QI_RING(r, K, P), qf, s);
        if (per >= 2) pv_tile<D>(QI_RING(r, V, (P + 2) & 3), p, acc);
        mc = tile_max(s, ld.ck(per, a, c));   // stale when per >= n: unused
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
      if (active && per >= 1 && per <= n) {
        raise_max<D>(acc, m_run, l_run, mc);
        if ((a.t0 + per) * BN > tl.kend) mask_tile(s, a.t0 + per - 1, tl.kend);   // PARTIAL
        tile_exp<FP8>(s, m_run, ld.ck(per - 1, a, c), ld.vsc(per - 1, a), log2_vs, inv_vs, l_run, p);
      }
      __builtin_amdgcn_s_waitcnt(0);   // this group's loads of two periods ago
      // coded tiles this group landed two periods ago: K_{per+1}, V_{per-1}
      if (per >= 2 && per + 1 < n) ld.template convert<true>(per + 1, a, QI_RING(r, K, (P + 1) & 3), group);
      if (per >= 2 && per - 1 < n) ld.template convert<false>(per - 1, a, QI_RING(r, V, (P + 3) & 3), group);
      if (per + 3 < n) ld.template issue<true>(per + 3, a, QI_RING(r, K, (P + 3) & 3), group);
      if (per + 1 < n) ld.template issue<false>(per + 1, a, QI_RING(r, V, (P + 1) & 3), group);
      if (FP8) wait_lds();   // converted tiles are written before the barrier
    }
    bar();
  };
  for (int p0 = 0; p0 <= n + 1; p0 += 4) {
    period(Slot<0>(), p0);
    if (p0 + 1 <= n + 1) period(Slot<1>(), p0 + 1);
    if (p0 + 2 <= n + 1) period(Slot<2>(), p0 + 2);
    if (p0 + 3 <= n + 1) period(Slot<3>(), p0 + 3);
  }

  // merge the two partial states of each row (group 1 -> LDS -> group 0); the ring is
  // free: every load was waited for and every read consumed
  const int w4 = wave & 3, lane = threadIdx.x & 63;
  float *ost = reinterpret_cast<float *>(ring_k(r, w4)) + lane;
  float *mst = reinterpret_cast<float *>(r.V0) + (w4 * 64 + lane) * 2;
  if (group == 1 && active) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) ost[(16 * db + rr) * 64] = acc[db][rr];
    mst[0] = m_run;
    mst[1] = l_run;
  }
  __syncthreads();
  if (group == 0 && active) {
    const float m1 = mst[0], l1 = mst[1];
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = __builtin_amdgcn_exp2f(m1 - mm);   // 0 when group 1 saw no tile
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) acc[db][rr] = acc[db][rr] * a0 + ost[(16 * db + rr) * 64] * a1;
    l_run = l_run * a0 + l1 * a1;
    if (tl.part >= 0)
      store_part<D>(part, tl, h, w4 * 32, acc, mm, l_run);
    else   // stage in this wavefront's own merge buffer, whose values are now in registers
      store_o_lds<D>(o, tl, H, h, w4 * 32, acc, l_run, ring_k(r, w4));
  }
}

template <int D, int SRC>
__global__ __launch_bounds__(NT, 1) void attn_pp_kernel(
    const int32_t *__restrict__ sched, const qi_tile *__restrict__ tiles, int H,
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ o, const uint8_t *__restrict__ cache, float *__restrict__ part,
    float c) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 K0[C::KTILE], K1[C::KTILE], K2[C::KTILE], K3[C::KTILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V0[C::VTILE], V1[C::VTILE], V2[C::VTILE], V3[C::VTILE];
  // landing buffers of E4M3FN code tiles, one BN x D region per group (coded caches only)
  uint8_t *lk = nullptr, *lv = nullptr;
  if constexpr (coded(SRC, 0)) {
    __shared__ __attribute__((aligned(1024))) uint8_t LK[2 * BN * D];
    lk = LK;
  }
  if constexpr (coded(SRC, 1)) {
    __shared__ __attribute__((aligned(1024))) uint8_t LV[2 * BN * D];
    lv = LV;
  }
  const int item = sched[blockIdx.x];
  if (item < 0) return;   // schedule padding
  const qi_tile tl = tiles[item / H];
  const int h = item % H;
  const TileArgs a = make_args(tl, H, h, k, v, cache, SRC == SRC_CACHE_FP8 || SRC == SRC_CACHE_FP8V);
  const Ring r{K0, K1, K2, K3, V0, V1, V2, V3, lk, lv};
  if (tl.nrows > 128)
    pp_rows256<D, SRC>(r, tl, H, h, a, q, o, part, c);
  else
    pp_rows128<D, SRC>(r, tl, H, h, a, q, o, part, c);
}
#undef QI_RING

// Merge of key chunks: row (tile, head) gets O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M)
// l_s over its chunks s in chunk order (M = max_s m_s), rounded to bf16 -- the same
// combination the online softmax applies between key tiles, done once per chunk.  A
// thread owns 4 dims of one row; a block covers RPB rows of one (tile, head).  The loads
// of up to MB chunks are issued together (entries past the last chunk reload the last one
// and get weight 0, which leaves the sums exact); more chunks are folded MB at a time, the
// running state rescaled by 2^(M_old - M_new) as between key tiles.
template <int D>
__global__ __launch_bounds__(256) void merge_chunks(const qi_merge *__restrict__ mg, int H,
                                                    const float *__restrict__ part,
                                                    __bf16 *__restrict__ o) {
  constexpr int TPR = D / 4, RPB = 256 / TPR, BPT = QI_ROWS / RPB, MB = 8;
  const int b = blockIdx.x;
  const int e = b / (H * BPT), h = (b / BPT) % H, rb = b % BPT;
  const qi_merge m = mg[e];
  const int row = rb * RPB + (int)threadIdx.x / TPR;
  if (row >= m.nrows) return;
  const int d = ((int)threadIdx.x % TPR) * 4;
  const size_t SLOT = QI_PART_SLOT_FLOATS(D), MO = (size_t)QI_ROWS * D;
  float mx = -INFINITY, l = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < m.nchunks; s0 += MB) {
    float ms[MB], ls[MB];
    float4 os[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int sj = min(s0 + j, m.nchunks - 1);
      const float *sl = part + (size_t)(m.part0 + sj * H + h) * SLOT;
      ms[j] = sl[MO + row];
      ls[j] = sl[MO + QI_ROWS + row];
      os[j] = *reinterpret_cast<const float4 *>(sl + (size_t)row * D + d);
    }
    float mn = mx;
#pragma unroll
    for (int j = 0; j < MB; ++j) mn = fmaxf(mn, ms[j]);
    if (s0 > 0) {   // chunks of earlier batches: rescale to the new maximum
      const float a = __builtin_amdgcn_exp2f(mx - mn);
      l *= a;
      acc.x *= a;
      acc.y *= a;
      acc.z *= a;
      acc.w *= a;
    }
    mx = mn;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const float w = s0 + j < m.nchunks ? __builtin_amdgcn_exp2f(ms[j] - mx) : 0.0f;
      l = __builtin_fmaf(w, ls[j], l);
      acc.x = __builtin_fmaf(w, os[j].x, acc.x);
      acc.y = __builtin_fmaf(w, os[j].y, acc.y);
      acc.z = __builtin_fmaf(w, os[j].z, acc.z);
      acc.w = __builtin_fmaf(w, os[j].w, acc.w);
    }
  }
  const float inv = 1.0f / l;
  uint2 u;
  u.x = pack_bf16(acc.x * inv, acc.y * inv);
  u.y = pack_bf16(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2 *>(o + ((int64_t)(m.q_tok + row) * H + h) * D + d) = u;
}

template <int D, int SRC>
qi_status launch(const qi_plan *p, int call, const void *q, const void *k, const void *v,
                 void *o, const void *cache, hipStream_t s) {
  const uint8_t *ws = static_cast<const uint8_t *>(p->d_ws);
  const float c = (float)(1.4426950408889634 / std::sqrt((double)D));   // log2(e)/sqrt(D)
  const auto kern = attn_pp_kernel<D, SRC>;
  const int nt = NT;
  float *part = reinterpret_cast<float *>(const_cast<uint8_t *>(ws) + p->kpart_off);
  hipLaunchKernelGGL(kern, dim3(p->sched_len[call]), dim3(nt), 0, s,
                     reinterpret_cast<const int32_t *>(ws + p->sched_off[call]),
                     reinterpret_cast<const qi_tile *>(ws + p->tiles_off[call]), p->H,
                     static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k),
                     static_cast<const __bf16 *>(v), static_cast<__bf16 *>(o),
                     static_cast<const uint8_t *>(cache), part, c);
  if (hipGetLastError() != hipSuccess) return QI_ERR_HIP;
  if (p->n_merge[call] > 0) {
    constexpr int BPT = QI_ROWS / (256 / (D / 4));   // blocks per (tile, head)
    hipLaunchKernelGGL(merge_chunks<D>, dim3(p->n_merge[call] * p->H * BPT), dim3(256), 0, s,
                       reinterpret_cast<const qi_merge *>(ws + p->merge_off[call]), p->H,
                       static_cast<const float *>(part), static_cast<__bf16 *>(o));
    if (hipGetLastError() != hipSuccess) return QI_ERR_HIP;
  }
  return QI_OK;
}

}  // namespace

qi_status qi_launch_attention(const qi_plan *p, int call, const void *q, const void *k,
                              const void *v, void *o, const void *cache, void *stream) {
  if (p->sched_len[call] == 0) return QI_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int src = call != QI_CALL_DENOISE ? SRC_ONE
                  : p->kv == QI_KV_BF16 ? SRC_CACHE_BF16
                  : p->kv == QI_KV_FP8_E4M3 ? SRC_CACHE_FP8 : SRC_CACHE_FP8V;
  if (p->D == 128) {
    if (src == SRC_ONE) return launch<128, SRC_ONE>(p, call, q, k, v, o, cache, s);
    if (src == SRC_CACHE_BF16) return launch<128, SRC_CACHE_BF16>(p, call, q, k, v, o, cache, s);
    if (src == SRC_CACHE_FP8) return launch<128, SRC_CACHE_FP8>(p, call, q, k, v, o, cache, s);
    return launch<128, SRC_CACHE_FP8V>(p, call, q, k, v, o, cache, s);
  }
  if (src == SRC_ONE) return launch<64, SRC_ONE>(p, call, q, k, v, o, cache, s);
  if (src == SRC_CACHE_BF16) return launch<64, SRC_CACHE_BF16>(p, call, q, k, v, o, cache, s);
  if (src == SRC_CACHE_FP8) return launch<64, SRC_CACHE_FP8>(p, call, q, k, v, o, cache, s);
  return launch<64, SRC_CACHE_FP8V>(p, call, q, k, v, o, cache, s);
}
