// Internal declarations shared by the host plan (plan.cpp), the C-ABI entry points
// (api.hip) and the kernels (attn_fwd.hip, prefix_kv.hip).  Not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "qi.h"   // include/ of the repository, on the include path

// Attention tiles: rows per workgroup x keys per step.  Row tiles of up to 256 rows (8
// wavefronts x 32 rows; tiles of <= 128 rows split their keys over two wave groups), for
// every key source and cache type.
#define QI_ROWS 256
#define QI_KERNEL_BN 64
// Number of XCDs of the MI355X and compute units per XCD; workgroups are dealt to the XCDs
// round-robin in launch order.
#define QI_NUM_XCD 8
#define QI_CUS_PER_XCD 32
// Prefix tokens per workgroup in the cache-write kernels.
#define QI_CACHE_CHUNK 64

// One row tile of one request for one call, or one key chunk of it (device table entry,
// 64 bytes).  The rows see keys [0, kend); the workgroup visits keys [k0, k1) of them:
// [0, kend) unless the plan splits keys, then one chunk whose partial softmax state goes
// to partial slot part + head and is merged afterwards.
struct qi_tile {
  int32_t q_tok;      // packed token index (in the call's Q and O tensors) of the first row
  int32_t nrows;      // 1 .. row tile size of the call
  int32_t kend;       // attended keys are positions [0, kend) of the request
  int32_t kv_tok;     // packed token index (in the call's live K/V) of key position `lp`
  int32_t lp;         // keys below lp come from the prefix cache (denoise); else 0
  int32_t req;        // request index
  int64_t k_off;      // byte offset of the request's cached K  [H][lp][D]   (denoise)
  int64_t v_off;      // byte offset of the request's cached V  [H][lp][D]   (denoise)
  int64_t s_off;      // byte offset of the request's scales [2][H] float32 (fp8 denoise)
  int32_t k0, k1;     // visited keys [k0, k1): k0 a multiple of QI_KERNEL_BN, k1 <= kend
  int32_t part;       // first partial slot of the chunk (slot part + head), or -1: store O
  int32_t pad;
};
static_assert(sizeof(qi_tile) == 64, "qi_tile is a 64-byte device record");

// One row tile whose keys were split into chunks, for the merge kernel (16 bytes): its
// chunk s of head h left its state in partial slot part0 + s * H + h.
struct qi_merge {
  int32_t q_tok;      // packed token index of the first row (in the call's O)
  int32_t nrows;
  int32_t nchunks;
  int32_t part0;
};
static_assert(sizeof(qi_merge) == 16, "qi_merge is a 16-byte device record");

// Partial slot of a key chunk: the unnormalised O of up to QI_ROWS rows ([row][D] fp32),
// then the rows' running max m (log2 units) and sum l: (QI_ROWS * D + 2 * QI_ROWS) floats.
#define QI_PART_SLOT_FLOATS(D) ((size_t)QI_ROWS * (D) + 2 * QI_ROWS)
// Key chunks are used only in a prefix or denoising call with fewer (row tile, head) items
// than compute units; a chunk holds at least this many key tiles.
#define QI_SPLIT_MIN_TILES 8
#define QI_NUM_CUS (QI_NUM_XCD * QI_CUS_PER_XCD)

// Per-request record for the cache-write kernels (device table entry, 48 bytes).
struct qi_req_dev {
  int32_t pre_tok;    // packed token index of the request's first prefix token
  int32_t lp;         // prefix length
  int32_t n_chunks;   // ceil(lp / QI_CACHE_CHUNK)
  int32_t part_idx;   // first float of the request's absmax partials [n_chunks][2][H]
  int64_t k_off, v_off, s_off;
  int64_t pad;
};
static_assert(sizeof(qi_req_dev) == 48, "qi_req_dev is a 48-byte device record");

struct qi_req_host {
  std::vector<int32_t> bl;    // text, ref_1..ref_R, image
  std::vector<int64_t> off;   // block offsets, size bl.size() + 1
  int32_t lp = 0, nimg = 0, n = 0;
  int32_t pre_tok = 0, img_tok = 0, all_tok = 0;
  int64_t k_off = 0, v_off = 0, s_off = -1, end = 0;
};

struct qi_plan {
  int32_t n_req = 0, H = 0, D = 0, kv = 0;
  std::vector<qi_req_host> req;
  int64_t tot_pre = 0, tot_img = 0, tot_all = 0;
  size_t cache_bytes = 0;
  int64_t pairs[3] = {0, 0, 0};

  // device tables, all inside one workspace image (host copy kept for upload)
  std::vector<uint8_t> ws_image;
  size_t ws_bytes = 0;
  size_t tiles_off[3] = {0, 0, 0}, sched_off[3] = {0, 0, 0};
  int32_t n_tiles[3] = {0, 0, 0}, sched_len[3] = {0, 0, 0};
  int32_t bm[3] = {0, 0, 0};   // row tile size per call
  size_t reqs_off = 0, part_off = 0, part_floats = 0;
  int32_t max_chunks = 0;
  // key split: chunk length in key tiles per call (0: none; the full call runs every row
  // in its source call's chunks), merge tables per call, and the partial slots (shared by
  // the calls, which run one after the other on a plan)
  int32_t kchunk_tiles[3] = {0, 0, 0};
  size_t merge_off[3] = {0, 0, 0};
  int32_t n_merge[3] = {0, 0, 0};
  size_t kpart_off = 0;
  int64_t kpart_slots = 0;

  void *d_ws = nullptr;   // caller's workspace once uploaded
  bool built = false;     // a prefix build has been enqueued on this plan
};

// Bytes per cached element of K (which = 0) or V (which = 1) for a cache type.
inline int qi_cache_elem_bytes(int kv, int which) {
  return kv == QI_KV_BF16 ? 2 : kv == QI_KV_FP8_E4M3 ? 1 : (which == 0 ? 2 : 1);
}

// Kernel launchers (defined in the .hip files).  Return QI_OK or QI_ERR_HIP.
qi_status qi_launch_attention(const qi_plan *p, int call, const void *q, const void *k,
                              const void *v, void *o, const void *cache, void *stream);
// partials: device buffer of the fp8 absmax partials (p->part_floats floats), or null for
// the workspace's own region.
qi_status qi_launch_cache_write(const qi_plan *p, const void *k_pre, const void *v_pre,
                                void *cache, float *partials, void *stream);
// Device address of this device's static scratch (QI_NOALLOC_MAX_PARTIALS floats), looked
// up once per device with that device current.  QI_ERR_HIP if the lookup fails.
qi_status qi_scratch_partials(float **out);
