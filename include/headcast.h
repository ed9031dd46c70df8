/*
 * headcast.h - C ABI of the head-routed attention library (libheadcast.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (HeadCast, arXiv 2607.20125; described on the pith.science
 * review page "HeadCast: Casting Attention Heads for Efficient
 * Autoregressive Video Generation", sections "Core claim" and "What carries
 * the argument", and in the paper's abstract): every attention head of an
 * autoregressive video diffusion transformer is classified once, when the
 * sliding KV window first fills, as one of four archetypes; from then on the
 * head attends only over its archetype's share of a restructured KV cache:
 *
 *   HC_SINK     the first cached block (the video's first block),
 *   HC_DUMMY    the newest block only (the queries' own block),
 *   HC_SPATIAL  its fixed 10x10 latent-grid cell in every cached frame
 *               (review: ledger entry "deployed spatial grid cell", Fig. 3),
 *   HC_GLOBAL   the whole sliding window.
 *
 * Three calls carry the work: hc_classify (one-shot classifier), then
 * hc_cache_create + hc_cache_append (the restructure, and every later block),
 * and hc_attend (routed attention, every denoising step of every layer).
 *
 * Conventions
 *   - Every function returns hc_status (HC_OK = 0) and never throws.  On a
 *     non-OK status, hc_last_error_message() gives a thread-local detail.
 *   - Arguments are validated before anything is enqueued; an invalid call
 *     enqueues nothing.  A failed kernel launch returns HC_ERR_HIP.
 *   - Device work is enqueued asynchronously on the caller's stream; the
 *     library never synchronises.  Calls that touch one hc_cache must be
 *     ordered (same stream, or caller-side synchronisation).
 *   - The library allocates no device memory: caches live in caller-owned
 *     device buffers, the classifier uses a caller-owned workspace (or, in
 *     hc_classify_static, a static array loaded with the library).
 *   - Stream capture: the enqueuing calls launch kernels only (no
 *     allocation, copy, memset or synchronisation), so they may be recorded
 *     into a HIP graph.  Kernel arguments are fixed when a call is recorded,
 *     from the cache's host-side state, and a replay does not change that
 *     state.  A recorded hc_attend stays valid as long as min(blocks pushed,
 *     W/B) is unchanged, so once the window is full it stays valid for good.
 *     A recorded hc_cache_append writes the block slot that was newest
 *     (HC_REPLACE_NEWEST) or next (HC_PUSH_BLOCK) when it was recorded.  A
 *     recorded HC_REPLACE_NEWEST + hc_attend pair, the per-step work of
 *     denoising one block, is therefore valid until the next
 *     HC_PUSH_BLOCK.
 *   - Tensors (hc_tensor) are per-head row-major matrices: element
 *     (head h, token t, channel c) sits at ptr + h*stride_head +
 *     t*stride_token + c, strides counted in ELEMENTS of the config's dtype.
 *     Channels are contiguous.  ptr must be 16-byte aligned and both strides
 *     must be multiples of 16 bytes.
 *   - Token order inside a block or window is frame-major, then row-major
 *     over the latent grid: t = f*grid_h*grid_w + y*grid_w + x.
 *   - Labels are int8: 0 Sink, 1 Dummy, 2 Spatial, 3 Global.
 */
#ifndef HEADCAST_H
#define HEADCAST_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_MAX_HEADS 128

typedef enum hc_status {
  HC_OK = 0,
  HC_ERR_INVALID_ARG = -1, /* null pointer, bad enum value, bad label */
  HC_ERR_SHAPE = -2,       /* inconsistent or unsupported sizes */
  HC_ERR_DTYPE = -3,       /* dtype not HC_BF16 / HC_FP32, or fp8 K/V with HC_FP32 */
  HC_ERR_ALIGN = -4,       /* pointer or stride not 16-byte aligned */
  HC_ERR_WORKSPACE = -5,   /* caller buffer smaller than required */
  HC_ERR_STATE = -6,       /* call out of order, e.g. attend before any append */
  HC_ERR_HIP = -7,         /* a HIP runtime call or kernel launch failed */
  HC_ERR_UNSUPPORTED = -8  /* valid request the library does not implement */
} hc_status;

enum { HC_SINK = 0, HC_DUMMY = 1, HC_SPATIAL = 2, HC_GLOBAL = 3 };
enum { HC_BF16 = 0, HC_FP32 = 1 };
enum { HC_KV_SAME = 0, HC_KV_FP8_E4M3 = 1 };
enum { HC_PUSH_BLOCK = 0, HC_REPLACE_NEWEST = 1 };

/* Geometry and precision of one attention layer.
 *   num_heads       1 .. HC_MAX_HEADS
 *   head_dim        64 or 128
 *   grid_h, grid_w  latent frame grid; T = grid_h*grid_w tokens per frame
 *   block_frames    B, frames generated per autoregressive block
 *   window_frames   W, frames in the sliding KV window; a multiple of B
 *   cell_h, cell_w  Spatial cell size (the pages use 10 x 10); cells are
 *                   anchored at (0,0) and the last row/column of cells is
 *                   truncated at the frame edge
 *   dtype           HC_BF16 (MFMA path, fp32 accumulation) or HC_FP32
 *   softmax_scale   0 selects 1/sqrt(head_dim)
 *   kv_format       how a cache stores K and V:
 *                   HC_KV_SAME      in dtype;
 *                   HC_KV_FP8_E4M3  as OCP FP8 E4M3 codes (1 byte), the K/V
 *                                   memory of the per-archetype buffers
 *                                   halved again (the review's App. C point:
 *                                   KV bytes are the cost the restructure
 *                                   cuts).  Needs dtype HC_BF16 (else
 *                                   HC_ERR_DTYPE); head_dim 64 or 128.
 *                                   hc_cache_append still takes bf16
 *                                   blocks and stores
 *                                   code(fp32(x * fp32(1/scale))), rounded to
 *                                   nearest even and saturated at +-448
 *                                   (inputs must be finite); hc_attend runs
 *                                   bf16 attention on decode(code) * scale.
 *                                   hc_classify ignores kv_format (it reads
 *                                   the caller's bf16 window).
 *   k_scale, v_scale  fp8 caches: positive finite scales of K and V (0
 *                   selects 1); ignored otherwise
 * Queries are the newest block: Nq = B*T rows per head.  The window holds
 * Nk = W*T keys per head. */
typedef struct hc_config {
  int32_t num_heads, head_dim, grid_h, grid_w, block_frames, window_frames;
  int32_t cell_h, cell_w, dtype;
  float softmax_scale;
  int32_t kv_format;
  float k_scale, v_scale;
} hc_config;

typedef struct hc_tensor {
  const void* ptr;
  int64_t stride_head, stride_token; /* in elements */
} hc_tensor;

typedef struct hc_out_tensor {
  void* ptr;
  int64_t stride_head, stride_token; /* in elements */
} hc_out_tensor;

/* Classifier parameters (review ledger: cosine threshold 0.95, spatial score
 * threshold 0.755, MSE weight 5, proxy radius 2).
 *   rule           0: among the proxies that clear their thresholds pick the
 *                  one with the largest mean cosine (ties Sink<Dummy<Spatial);
 *                  1: the first that clears, in the order Sink, Dummy, Spatial
 *   spatial_proxy  0: the deployed grid cell (the query's 10x10 cell in every
 *                  window frame); 1: the sliding (2r+1)^2 box the review says
 *                  the paper classifies with ([Pith] Referee Report, comment
 *                  2; ledger "Spatial proxy radius r = 2"): keys within
 *                  `radius` rows and columns of the query, in every window
 *                  frame, cut at the frame border
 *   radius         box radius r for spatial_proxy 1, 0..8 (else
 *                  HC_ERR_INVALID_ARG)
 *   percentile     rank of the worst-case Spatial cosine (5 = 5th percentile,
 *                  linear interpolation at rank p/100*(Nq-1)) */
typedef struct hc_classify_params {
  float theta_sink, theta_dummy, theta_spatial, theta_score, gamma, percentile;
  int32_t rule, spatial_proxy, radius;
} hc_classify_params;

typedef struct hc_cache hc_cache; /* opaque host object */

/* Where the per-archetype buffers sit inside the cache's device memory.
 * Offsets are in bytes from the device_mem pointer given to hc_cache_create.
 * Heads of one archetype get slots 0,1,... in ascending head order;
 * head_slot[h] is head h's slot inside its archetype's buffer.
 *   Global  K,V [n_global][W*T][d]: ring of W/B block slots, block b in ring
 *           slot b mod (W/B), rows in token order.
 *   Sink    K,V [n_sink][B*T][d]: the first block ever appended.
 *   Dummy   K,V [n_dummy][B*T][d]: the newest block.
 *   Spatial K,V [n_spatial][W*T][d]: cell-major.  Cell c (row-major over the
 *           cell grid) starts at row W*sum_{c'<c}|c'|; within it frame slot
 *           s = 0..W-1 holds the cell's |c| tokens in row-major (y,x) order;
 *           frame i of block b sits in frame slot (b mod (W/B))*B + i.
 * Rows hold head_dim elements of the dtype, or head_dim bytes (E4M3 codes)
 * in an HC_KV_FP8_E4M3 cache.
 * Rows of a ring slot that no block has reached yet are unspecified. */
typedef struct hc_cache_layout {
  uint64_t total_bytes;
  uint64_t off_global_k, off_global_v, off_sink_k, off_sink_v;
  uint64_t off_dummy_k, off_dummy_v, off_spatial_k, off_spatial_v;
  uint64_t off_scratch, scratch_bytes;
  int32_t n_global, n_sink, n_dummy, n_spatial;
  int32_t blocks_appended;
  /* key-range splits hc_attend uses for the Global, Sink and Dummy heads
   * (chosen from the layer shape so that the work units fill the GPU) */
  int32_t global_splits, sink_splits, dummy_splits;
  int32_t head_slot[HC_MAX_HEADS];
} hc_cache_layout;

/* Fills *p with the defaults above (0.95, 0.95, 0.95, 0.755, 5, 5, rule 0,
 * proxy 0, radius 2). */
void hc_default_classify_params(hc_classify_params* p);

/* Checks a configuration without touching the GPU. */
hc_status hc_validate_config(const hc_config* cfg);

/* Device bytes a cache for (cfg, labels_host[num_heads]) needs.  Host only. */
hc_status hc_cache_bytes(const hc_config* cfg, const int8_t* labels_host, size_t* device_bytes);

/* Creates the host object of a restructured cache over caller-owned device
 * memory (256-byte aligned, at least hc_cache_bytes long; it must outlive the
 * cache).  labels_host[num_heads] is copied.  Host only: nothing is enqueued.
 * The cache starts empty; replay the window's W/B blocks with PUSH_BLOCK to
 * restructure an existing monolithic cache. */
hc_status hc_cache_create(const hc_config* cfg, const int8_t* labels_host, void* device_mem,
                          size_t bytes, hc_cache** out);
hc_status hc_cache_destroy(hc_cache* cache);
hc_status hc_cache_get_layout(const hc_cache* cache, hc_cache_layout* out);

/* Enqueues the copy of one block's keys and values (each [num_heads][B*T][d]
 * as hc_tensor) into the per-archetype buffers.
 *   HC_PUSH_BLOCK      the block becomes the newest; the window slides once
 *                      more than W/B blocks were pushed; the first block ever
 *                      pushed also becomes the Sink block.
 *   HC_REPLACE_NEWEST  overwrites the newest block (the K/V of the block
 *                      being denoised change every step); needs one block.
 * Spatial rows are scattered into cell-major order.  Pure data movement
 * (quantisation to E4M3 codes in an HC_KV_FP8_E4M3 cache): buffers equal the
 * documented layout bit for bit. */
hc_status hc_cache_append(hc_cache* cache, hc_tensor k_block, hc_tensor v_block, int32_t mode,
                          hipStream_t stream);

/* Routed attention for the newest block's queries, q_block
 * [num_heads][B*T][d], into out [num_heads][B*T][d] (same dtype; may not
 * alias q or the cache).  Each head attends, with exact softmax
 * attention (fp32 accumulation), over its archetype's keys:
 *   Global  the last min(n, W/B) blocks; Sink the first block; Dummy the
 *   newest block; Spatial the keys of the query's cell in every cached frame.
 * Uses the cache's scratch region: two hc_attend calls on one cache must
 * not overlap.  Needs at least one appended block (else HC_ERR_STATE). */
hc_status hc_attend(hc_cache* cache, hc_tensor q_block, hc_out_tensor out, hipStream_t stream);

/* Workspace bytes hc_classify needs for cfg. */
hc_status hc_classify_workspace_bytes(const hc_config* cfg, size_t* bytes);

/* One-shot head classifier over a full window (k_window, v_window
 * [num_heads][W*T][d], oldest frame first, the queries' block last) and the
 * newest block's queries q_block [num_heads][B*T][d].  Per head it computes
 * the full-context output and the Sink, Dummy and Spatial proxy outputs,
 * per-query cosines against the full output, the mean cosine per proxy, the
 * worst-case Spatial score S = P_percentile(cos_spatial) - gamma * MSE(full,
 * spatial) and the label by the rule.
 * Writes labels_dev[num_heads] (int8) and diag_dev[num_heads][4] =
 * {C_sink, C_dummy, C_spatial, S} (fp32), both device pointers.
 * The workspace (caller-owned device memory, 256-byte aligned) holds, in
 * this order, each region starting at a 256-byte boundary, and readable
 * after the call:
 *   float O[4][num_heads][Nq][d]   full, sink, dummy, spatial outputs
 *   float C[num_heads][4][Nq]      per-query cos_sink, cos_dummy, cos_spatial,
 *                                  and sum_c (o_full - o_spatial)^2
 *   float S[3][num_heads][Nq][2]   scratch (bf16): per query, the softmax state
 *                                  (running max of the raw scores, sum of
 *                                  weights) over the window's first block, its
 *                                  middle blocks and its last block; the Sink
 *                                  and Dummy proxies' keys are attended once,
 *                                  as part of the full output's, and the three
 *                                  outputs are merged from these states
 * The host copies labels back once (the one synchronisation point) and then
 * builds the cache with hc_cache_create. */
hc_status hc_classify(const hc_config* cfg, const hc_classify_params* params, hc_tensor q_block,
                      hc_tensor k_window, hc_tensor v_window, void* workspace, size_t ws_bytes,
                      int8_t* labels_dev, float* diag_dev, hipStream_t stream);

/* Bytes of the library's static classifier scratch (64 MiB; see
 * hc_classify_static). */
#define HC_STATIC_SCRATCH_BYTES (64u << 20)

/* hc_classify for callers that cannot allocate device memory, or cannot
 * bring a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks, results and
 * kernels as hc_classify, without the workspace: the workspace is a
 * file-scope device array of HC_STATIC_SCRATCH_BYTES inside the library,
 * one per GPU, held from the first call on that GPU until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine);
 * its first call on a GPU looks up the array's device address there.
 * Limit: configurations whose hc_classify_workspace_bytes exceed
 * HC_STATIC_SCRATCH_BYTES are rejected with HC_ERR_WORKSPACE (at d = 128
 * that is num_heads * Nq above about 32,000 query-heads).  The four proxy
 * outputs and cosines stay in the array and are not meant to be read; only
 * labels_dev and diag_dev are results.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, or hosts
 * threads without ordering) race and give undefined results.  The array
 * keeps the last call's contents; nothing in it needs to start at zero. */
hc_status hc_classify_static(const hc_config* cfg, const hc_classify_params* params, hc_tensor q_block,
                             hc_tensor k_window, hc_tensor v_window, int8_t* labels_dev, float* diag_dev,
                             hipStream_t stream);

const char* hc_status_string(hc_status s);
const char* hc_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* HEADCAST_H */
