/*
 * qi.h -- C ABI of libqi: prefix-reuse block-causal attention for one MI355X (gfx950).
 *
 * What is computed.  Qwen-Image-2.1's single-stream DiT attends block-causally over a
 * sequence made of a text-instruction block, the reference-image blocks in the order
 * given, and the image-latent block.  Since the prefix (text + references) never attends
 * to the image block, its K/V is the same at every denoising step: it is computed once at
 * the first step, cached, and reused exactly at the later steps, where only the image
 * rows are recomputed; the cache is rebuilt for every generation so nothing leaks from
 * one request to the next.  (ThakiCloud blog "Qwen-Image-2.1 vLLM-Omni day 0", section
 * "Serving architecture: the cross-step prefix KV cache"; vLLM recipe
 * "Qwen/Qwen-Image-2.1", section "Prefix KV cache".)
 *
 * Attention rule (the plain reading of "block-causal"): with blk(p) the block index of
 * position p inside its request, query q may attend key k iff blk(k) <= blk(q); inside a
 * block attention is bidirectional; different requests never see each other.
 *   O[q] = sum_k softmax_k(Q[q].K[k] / sqrt(D)) V[k]    over the allowed keys.
 *
 * Calls.  One plan describes one wave: requests that are at the same denoising phase
 * and run in one launch (the recipe's "Online serving" section batches up to 8 such
 * requests with step execution).  Per DiT layer and request:
 *   step 0      qi_prefix_kv_build   (prefix rows over prefix keys; writes the cache)
 *               qi_denoise_attn_step (image rows; the first denoising step)
 *   steps 1..   qi_denoise_attn_step (image rows over cached prefix + live image KV)
 *   check       qi_attn_full_reference_step (every row over every key, no cache)
 *
 * Tensor layouts (all little-endian, all device memory unless said otherwise):
 *   live Q/K/V/O are token-major packed bf16 [tokens][H][D]; the tokens of each request
 *   are contiguous and requests follow the wave order.  Per call:
 *     prefix build : [sum_r L_p(r)][H][D]   tokens text, ref_1..ref_R of each request
 *     denoise step : [sum_r N_img(r)][H][D] image tokens of each request
 *     full step    : [sum_r N(r)][H][D]     text, ref_1..ref_R, image of each request
 *   prefix cache (one arena per layer and wave): requests in wave order, each region
 *   256-byte aligned and holding, each part again 256-byte aligned,
 *     K [H][L_p][D], then V [H][L_p][D]      bf16, or OCP E4M3FN codes (1 byte): K and V
 *                                            for QI_KV_FP8_E4M3, V only for QI_KV_FP8_V
 *     scales [2][H] float32 (row 0 K, row 1 V) fp8 caches only (QI_KV_FP8_V: K row = 1)
 *   The fp8 caches are the pages' storage options ("fp8": K and V, "fp8_v": V only;
 *   recipe section "Prefix KV cache").  Quantisation: per (request, head, K|V) a = max|x|
 *   over all prefix tokens and channels, scale = a/448, inv = 448/a (float32, correctly
 *   rounded; a == 0 gives 1 and 1), code = nearest E4M3FN value to the float32 product
 *   x*inv, ties to even, saturating at +-448.  Attention uses the code values exactly (they
 *   are bf16 values) with K's scale folded into the logit scale and V's into the
 *   probabilities; on the one key tile of a request that mixes cached and live keys it
 *   uses code*scale rounded to bf16.
 *
 * Ownership and errors.  The caller owns every device buffer (inputs, outputs, the
 * cache arena, the plan workspace) and the stream; the library owns only the host-side
 * plan.  No call allocates device memory or synchronises; work is enqueued on `stream`
 * (a hipStream_t; NULL is the null stream).  Arguments are checked on the host before
 * anything is enqueued: a bad argument returns an error code and enqueues nothing.  A
 * failed launch returns QI_ERR_HIP; faults inside kernels surface at the caller's next
 * synchronisation.  Device pointers must be 16-byte aligned.  Buffer extents are the
 * caller's contract (the library cannot see them), except the cache and workspace whose
 * sizes are passed and checked.  Calls on one plan must not overlap in time; plans are
 * independent of each other.
 */
#ifndef QI_H
#define QI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qi_status {
  QI_OK = 0,
  QI_ERR_INVALID_ARG = 1,      /* null pointer, bad count or length, misaligned pointer   */
  QI_ERR_UNSUPPORTED = 2,      /* head_dim other than 64 or 128                           */
  QI_ERR_STATE = 3,            /* workspace not uploaded, or denoise before any build     */
  QI_ERR_BUFFER_TOO_SMALL = 4, /* cache / workspace / host output smaller than required   */
  QI_ERR_HIP = 5               /* a HIP runtime call or kernel launch failed              */
} qi_status;

/* Prefix cache element type: bf16 K and V; fp8 K and V ("fp8"); bf16 K and fp8 V ("fp8_v").
 * The two fp8 options are the recipe's (vLLM recipe "Qwen/Qwen-Image-2.1", section
 * "Prefix KV cache"). */
typedef enum qi_kv_dtype { QI_KV_BF16 = 0, QI_KV_FP8_E4M3 = 1, QI_KV_FP8_V = 2 } qi_kv_dtype;

typedef enum qi_call { QI_CALL_PREFIX = 0, QI_CALL_DENOISE = 1, QI_CALL_FULL = 2 } qi_call;

/* Largest counts the library accepts. */
#define QI_MAX_REQUESTS 64   /* one wave                                                   */
#define QI_MAX_REFS 10       /* the model takes up to 10 reference images (ThakiCloud blog,
                                section "What is Qwen-Image-2.1", component table)         */
#define QI_MAX_HEADS 128

/* One wave.  block_len holds, request after request, 1 + n_refs[r] + 1 positive lengths:
 * text, ref_1 .. ref_R, image.  All arrays are host memory, read during qi_plan_create
 * only.  Sums per request must stay below 2^24 tokens. */
typedef struct qi_wave_desc {
  int32_t n_requests;        /* 1 .. QI_MAX_REQUESTS                                      */
  const int32_t *n_refs;     /* [n_requests], each 0 .. QI_MAX_REFS                       */
  const int32_t *block_len;  /* [sum_r (n_refs[r] + 2)], each > 0                         */
  int32_t n_heads;           /* 1 .. QI_MAX_HEADS                                         */
  int32_t head_dim;          /* 64 or 128                                                 */
  int32_t kv_dtype;          /* qi_kv_dtype of the prefix cache                           */
} qi_wave_desc;

typedef struct qi_plan qi_plan; /* opaque, host-owned */

/* Validate the wave and build its host-side plan: block offsets, tile lists and launch
 * schedules for the three calls, and the cache layout.  *out receives a new plan (free
 * with qi_plan_destroy) or NULL on error. */
qi_status qi_plan_create(const qi_wave_desc *desc, qi_plan **out);

/* Release a plan (NULL is ignored).  Device buffers stay the caller's. */
void qi_plan_destroy(qi_plan *plan);

/* Bytes the caller must provide: the cache arena of one layer, and the device workspace
 * (launch schedules, fp8 absmax partials, and the partial softmax states of key chunks
 * when the plan splits keys -- see qi_plan_kernel_tile).  Either output pointer may be
 * NULL. */
qi_status qi_plan_sizes(const qi_plan *plan, size_t *cache_bytes, size_t *workspace_bytes);

/* Copy the plan's schedules into the caller's device workspace (enqueued on stream) and
 * remember the workspace for the later calls.  The workspace must stay allocated and
 * untouched by the caller while the plan is in use.  May be called again to move it.
 * The calls of one plan write scratch state into its workspace, so they must run one
 * after the other (one stream, or ordered by events); overlapping calls on one plan race. */
qi_status qi_plan_upload(qi_plan *plan, void *d_workspace, size_t workspace_bytes,
                         void *stream);

/* Step 0, prefix side: write the prefix cache from k_pre/v_pre (bf16 copy, or fp8
 * quantisation as described above) and compute block-causal attention of the prefix rows
 * over the prefix keys into o_pre.  The prompt and reference K/V computed at the first
 * step is what every later step reuses (ThakiCloud blog "Qwen-Image-2.1 vLLM-Omni day 0",
 * section "Serving architecture: the cross-step prefix KV cache"); the prefill runs once,
 * eagerly (vLLM recipe "Qwen/Qwen-Image-2.1", section "CUDA graphs"); FP8 storage is the
 * recipe's "fp8" / "fp8_v" option (section "Prefix KV cache").  q/k/v/o_pre:
 * [sum L_p][H][D] bf16.  Fully overwrites every request's region of d_cache (the cache is
 * rebuilt per generation).  Requests without a prefix cannot occur (the text block is
 * never empty). */
qi_status qi_prefix_kv_build(qi_plan *plan, const void *q_pre, const void *k_pre,
                             const void *v_pre, void *o_pre, void *d_cache,
                             size_t cache_bytes, void *stream);

/* Allocation-free variant of qi_prefix_kv_build, for callers that cannot allocate device
 * memory at the time of the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results bit-identical to
 * qi_prefix_kv_build.  The fp8 quantisation's per-chunk absmax partials, which the
 * ordinary call keeps in the workspace, go to a static device array of the library
 * (QI_NOALLOC_MAX_PARTIALS floats, 1 MiB, held by each GPU the library runs on until the
 * process ends); the workspace must still have been uploaded (QI_ERR_STATE otherwise),
 * since it holds the plan's tables.  Plans whose partials exceed the array
 * (sum over requests of ceil(L_p / 64) * 2 * H floats) get QI_ERR_BUFFER_TOO_SMALL before
 * anything is enqueued.  Calls on one GPU share the array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must not be made. */
#define QI_NOALLOC_MAX_PARTIALS 262144
qi_status qi_prefix_kv_build_noalloc(qi_plan *plan, const void *q_pre, const void *k_pre,
                                     const void *v_pre, void *o_pre, void *d_cache,
                                     size_t cache_bytes, void *stream);

/* Denoising step: attention of the image rows over the cached prefix keys followed by the
 * live image keys of the same request -- the remaining steps reuse the cached prefix K/V
 * exactly and recompute only the image rows (vLLM recipe "Qwen/Qwen-Image-2.1", section
 * "Prefix KV cache"; ThakiCloud blog, section "Serving architecture: the cross-step prefix
 * KV cache"); requests at the same phase share one launch (recipe, "Online serving").
 * q/k/v/o_img: [sum N_img][H][D] bf16.  Reads the cache only.  QI_ERR_STATE if no
 * qi_prefix_kv_build has been enqueued on this plan.  On a bf16 cache the result is
 * bit-identical to the image rows of qi_attn_full_reference_step on the same values (same
 * tiles, same arithmetic). */
qi_status qi_denoise_attn_step(const qi_plan *plan, const void *d_cache, size_t cache_bytes,
                               const void *q_img, const void *k_img, const void *v_img,
                               void *o_img, void *stream);

/* Full recompute without the cache: every row of every request over that request's keys,
 * block-causal, fully masked key tiles skipped -- the no-cache baseline whose work the
 * prefix cache cuts (about a fifth of the sequence is recomputed with four references:
 * vLLM recipe "Qwen/Qwen-Image-2.1", section "Prefix KV cache"), and the check that the
 * cached step is exact (ThakiCloud blog, section "Serving architecture: the cross-step
 * prefix KV cache": block-causal attention is what makes the reuse exact).
 * q/k/v/o_all: [sum N][H][D] bf16.  Used to show that reuse is exact. */
qi_status qi_attn_full_reference_step(const qi_plan *plan, const void *q_all,
                                      const void *k_all, const void *v_all, void *o_all,
                                      void *stream);

/* Tile classification of a call for a tiling of bm rows x bn keys: row tiles never cross
 * a block (each block of the call's rows is cut from its first row), key tiles start at
 * key 0 of the request.  One byte per (request, row tile, key tile), in that nesting
 * order: 0 EMPTY (no allowed pair, skipped), 1 PARTIAL (masked), 2 FULL.  Writes into
 * host_out (host memory) when n is large enough; *n_needed (may be NULL) receives the
 * size.  QI_ERR_BUFFER_TOO_SMALL if host_out is NULL or n is too small. */
qi_status qi_plan_tile_map(const qi_plan *plan, int32_t call, int32_t bm, int32_t bn,
                           uint8_t *host_out, size_t n, size_t *n_needed);

/* Tile shape (rows x keys) the attention kernel of a call uses; the tile map of the call
 * for this shape is the one the kernel follows.  To balance the last wave of workgroups
 * the launch schedule may run a row tile as two halves of at most bm/2 rows each (the
 * halves see the same key tiles, so the map is unchanged).  When the prefix or the
 * denoising call has fewer (row tile, head) items than the GPU has compute units (a head
 * shard, e.g. 3 of 24 heads), the plan instead cuts each of that call's row tiles' keys
 * into chunks of whole key tiles, one workgroup each, and a second kernel merges the
 * chunks' partial softmax states in chunk order; each of the two calls has one chunk
 * length.  Either way the full call runs each row exactly as the prefix or denoising call
 * runs it. */
qi_status qi_plan_kernel_tile(const qi_plan *plan, int32_t call, int32_t *bm, int32_t *bn);

/* The launch schedule of a call: one record of QI_LAUNCH_ITEM_FIELDS int32 per
 * workgroup, in launch order (workgroup i runs on XCD i % 8): request, head, first row,
 * row count, first key, end key.  The first row is a position in the request's sequence
 * (text, references, image; 0-based), so a denoising item starts at L_p or later.  The
 * workgroup visits keys [first key, end key) of the rows' visible keys: all of them, or
 * one key chunk (see qi_plan_kernel_tile).  Padding workgroups, which do no work, read -1
 * in every field.  Row counts above half the kernel's row tile run on the kernel's
 * whole-tile path; the others (half tiles the schedule split off, short block tails) run
 * with the key tiles split over two wavefront groups.  Writes into host_out (host
 * memory) when n >= QI_LAUNCH_ITEM_FIELDS * workgroups; *n_needed (may be NULL)
 * receives that count.  QI_ERR_BUFFER_TOO_SMALL if host_out is NULL or n is too small. */
#define QI_LAUNCH_ITEM_FIELDS 6
qi_status qi_plan_launch_items(const qi_plan *plan, int32_t call, int32_t *host_out, size_t n,
                               size_t *n_needed);

/* Byte offset in the cache arena of element (request, kv = 0 K | 1 V, head, token,
 * channel 0); for kv = 2 the offset of the request's float32 scales [2][H] (fp8 only). */
qi_status qi_plan_cache_offset(const qi_plan *plan, int32_t req, int32_t kv, int32_t head,
                               int32_t tok, size_t *byte_off);

/* Number of allowed (row, key) pairs a call computes over the whole wave (per head).
 * Useful FLOPs of the call = 4 * head_dim * n_heads * pairs. */
qi_status qi_plan_pairs(const qi_plan *plan, int32_t call, int64_t *pairs);

/* Token counts of the wave: sum of prefix, image and total lengths. */
qi_status qi_plan_tokens(const qi_plan *plan, int64_t *prefix_tokens, int64_t *image_tokens,
                         int64_t *total_tokens);

/* Static description of a status code. */
const char *qi_status_string(qi_status status);

#ifdef __cplusplus
}
#endif
#endif /* QI_H */
