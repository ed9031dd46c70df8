// Internal declarations shared by the HIP sources of libheadcast.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/headcast.h"

namespace hc {

// ---------------------------------------------------------------------------
// Attention work plan, passed by value as a kernel argument.
//
// The work of one launch is a list of "categories" (at most 4).  Every head of
// a category has the same number of work units and the same key-set shape:
//   RANGED       keys are a contiguous row range [kv_first, kv_first+kv_count)
//                of the head's K/V matrix (Global, Sink, Dummy pathways);
//   CELL_MAJOR   Spatial pathway over a cell-major buffer: cell c's keys are
//                rows [W*off_c, W*off_c + nf*|c|);
//   CELL_GATHER  Spatial pathway over a frame-major window: the keys of cell c
//                in frames 0..nf-1 are gathered row by row.
// Units are numbered category by category (heaviest first).  Ranged units are
// (head, split, q-tile), q-tile fastest, so that work groups running at the
// same time read the same key rows.  Spatial units are (head, cell, q-sub-tile)
// in the fp32 kernel and (q-sub-tile, head, cell) in the bf16 kernel, whose
// cells' full first sub-tiles thus start before the short remainders;
// sub-tiles past a small cell are empty.
// ---------------------------------------------------------------------------
//   BOX_GATHER   classifier's sliding-box Spatial proxy over a frame-major
//                window: a unit is a patch of box_rows x box_cols_q queries of
//                one block frame; its keys are the (box_rows + 2r) x 32 grid
//                positions around the patch (columns px0-r .. px0-r+31) in each
//                of kv_count frames, frame by frame, row by row.  Positions off
//                the grid are loaded clamped and masked; each query keeps only
//                keys within r rows and r columns of itself.
enum : int32_t { KIND_RANGED = 0, KIND_CELL_MAJOR = 1, KIND_CELL_GATHER = 2, KIND_BOX_GATHER = 3 };

constexpr int kBf16QueryBlocks = 1;                  // 32-query blocks per wave, bf16 kernel
constexpr int kBf16Waves = 8;                        // waves per work group, bf16 kernel
constexpr int QTILE_BF16 = 32 * kBf16QueryBlocks * kBf16Waves;          // queries per work group, bf16 kernel
constexpr int QTILE_F32 = 128;                       // queries per work group, fp32 kernel
constexpr int KTILE = 64;                            // keys per inner iteration
constexpr int kMaxSplits = 8;                        // key-range splits per ranged head, at most
constexpr int kMaxBoxRadius = 8;                     // sliding-box proxy radius, at most (patches >= 16 columns)

struct AttnCat {
  int32_t kind;
  int32_t n_heads;
  int32_t units_per_head;
  int32_t unit_begin;
  int32_t kv_first;       // RANGED: first key row
  int32_t kv_count;       // RANGED: number of keys; CELL_*: number of frames present
  int32_t splits;         // RANGED: key-range splits per q tile (>= 1)
  int32_t keys_per_split; // RANGED: keys per split, a multiple of KTILE
  const void* k;          // K base of slot 0
  const void* v;          // V base of slot 0
  int64_t kv_sh, kv_st;   // slot (head) stride and token stride, elements
  void* o;                // output base for this category
  int64_t o_sh, o_st;     // output head / token strides, elements
  float* part;            // split partials: O as [id][split][D/2][q tile] float2, then (m,l) as [id][split][q tile] float2
  int32_t* counters;      // one per (head slot, q tile) when splits > 1
  int32_t out_f32;        // output written as fp32 (else the input dtype)
  int32_t pad_;
  float2* ml_out;         // if set: write the unnormalised O and each query's softmax state (m, l) at
                          // ml_out[head * Nq + token] (raw scores' running max, sum of weights)
};

struct AttnPlan {
  int32_t n_cats;
  int32_t total_units;
  int32_t q_tiles;         // ceil(Nq / queries per work group), for ranged categories
  int32_t cell_subtiles;   // q sub-tiles per spatial cell
  // Q
  const void* q;
  int64_t q_sh, q_st;
  // geometry
  int32_t T, grid_w, grid_h, cell_h, cell_w, cell_cols, B, W, Nq;
  float scale_log2;        // softmax scale * log2(e) (* the K scale of an fp8 cache)
  float v_scale;           // output multiplier: the V scale of an fp8 cache, else 1
  int32_t kv8;             // K/V are fp8 E4M3 codes (bf16 kernel, d = 128, cache kinds)
  // sliding-box proxy (KIND_BOX_GATHER): radius, patch rows and columns,
  // patches per frame down and across
  int32_t box_r, box_rows, box_cols_q, box_bands_y, box_bands_x;
  AttnCat cat[4];
  // bf16 kernel, persistent mode: per-XCD unit counters [8] and finished-work-
  // group counters [8], zero at launch and left zero; grid work groups.
  // nullptr: one work group per unit.
  int32_t* work_ctr;
  int32_t grid;
  int32_t pad2_;
  uint8_t head_of[4][HC_MAX_HEADS];  // category slot -> q/o head index
};

struct CellInfo {
  int base;    // y0*grid_w + x0
  int size;    // |c|
  int width;   // cell width (x extent)
  int off;     // sum of |c'| over cells c' < c
};

// Latent cell c (row-major over the cell grid, cells anchored at (0,0) and cut
// at the frame edge) and where its rows sit in the cell-major Spatial buffer.
__device__ __forceinline__ CellInfo cell_info(const AttnPlan& P, int c) {
  const int cy = c / P.cell_cols, cx = c - cy * P.cell_cols;
  const int y0 = cy * P.cell_h, x0 = cx * P.cell_w;
  const int h = min(P.cell_h, P.grid_h - y0), w = min(P.cell_w, P.grid_w - x0);
  CellInfo ci;
  ci.base = y0 * P.grid_w + x0;
  ci.size = h * w;
  ci.width = w;
  ci.off = cy * P.cell_h * P.grid_w + cx * h * P.cell_w;
  return ci;
}

// Token row of the i-th element of a cell, enumerated frame by frame.
__device__ __forceinline__ int cell_token(const AttnPlan& P, const CellInfo& c, int i) {
  const int f = i / c.size;
  const int r = i - f * c.size;
  const int ry = r / c.width;
  return f * P.T + c.base + ry * P.grid_w + (r - ry * c.width);
}

// Patch of a KIND_BOX_GATHER unit: block frame, first query row and column.
struct BoxInfo {
  int fb, py0, px0;
};
__device__ __forceinline__ BoxInfo box_info(const AttnPlan& P, int j) {
  const int per_frame = P.box_bands_y * P.box_bands_x;
  BoxInfo b;
  b.fb = j / per_frame;
  const int rem = j - b.fb * per_frame;
  const int by = rem / P.box_bands_x;
  b.py0 = by * P.box_rows;
  b.px0 = (rem - by * P.box_bands_x) * P.box_cols_q;
  return b;
}
// Grid row and column of box key k (may lie off the grid).
__device__ __forceinline__ void box_pos(const AttnPlan& P, const BoxInfo& b, int k, int& f, int& ky, int& kx) {
  const int rows = P.box_rows + 2 * P.box_r;
  const int rg = k >> 5;
  f = rg / rows;
  ky = b.py0 - P.box_r + (rg - f * rows);
  kx = b.px0 - P.box_r + (k & 31);
}
// Window token loaded for box key k: its position clamped into the grid.
__device__ __forceinline__ int box_token(const AttnPlan& P, const BoxInfo& b, int k) {
  int f, ky, kx;
  box_pos(P, b, k, f, ky, kx);
  ky = min(max(ky, 0), P.grid_h - 1);
  kx = min(max(kx, 0), P.grid_w - 1);
  return f * P.T + ky * P.grid_w + kx;
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_attn_bf16(const AttnPlan& plan, int head_dim, hipStream_t s);
hipError_t launch_attn_f32(const AttnPlan& plan, int head_dim, hipStream_t s);

// ---------------------------------------------------------------------------
// Cache append.
// ---------------------------------------------------------------------------
struct AppendPlan {
  const uint8_t* k;       // source block K (bytes), head / token strides in bytes
  const uint8_t* v;
  int64_t src_sh, src_st;
  int32_t row_bytes;      // source row: head_dim * element size
  int32_t dst_row_bytes;  // cached row: row_bytes, or head_dim when quantised
  int32_t quant;          // store bf16 rows as E4M3 codes of x * inv_k (inv_v)
  float inv_k, inv_v;
  int32_t rows;           // B*T
  int32_t H;
  int32_t T, grid_w, grid_h, cell_h, cell_w, cell_cols, B, W;
  int32_t ring_slot;      // (block index) mod (W/B)
  int32_t write_sink;     // block index == 0
  uint8_t* dst_k[4];      // per-archetype K buffer base (bytes), by label
  uint8_t* dst_v[4];
  int64_t dst_slot_bytes[4];
  uint8_t label[HC_MAX_HEADS];
  uint8_t slot[HC_MAX_HEADS];
};
hipError_t launch_append(const AppendPlan& plan, hipStream_t s);
hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s);

// ---------------------------------------------------------------------------
// Classifier reductions.
// ---------------------------------------------------------------------------
struct CosPlan {
  const float* o;          // [4][H][Nq][D] fp32
  float* c;                // [H][4][Nq]
  int32_t H, Nq, D;
};
hipError_t launch_cosines(const CosPlan& plan, hipStream_t s);

// Classifier: merge the softmax states of the window's first block, middle
// blocks and last block (written unnormalised into the sink, full and dummy
// output planes) into the full, Sink and Dummy outputs, in place.
struct MergePlan {
  float* o;                // [4][H][Nq][D] fp32: plane 0 full, 1 sink, 2 dummy
  const float2* ml;        // [3][H][Nq]: states of the first block, the middle, the last block
  int32_t H, Nq, D;
  int32_t has_middle;      // the window has more than two blocks
  int32_t one_block;       // the window is one block: first = last, stored as the first
  float scale_log2;
};
hipError_t launch_merge_ranges(const MergePlan& plan, hipStream_t s);

struct ReducePlan {
  const float* c;          // [H][4][Nq]
  int8_t* labels;          // [H]
  float* diag;             // [H][4]
  int32_t H, Nq, D;
  float theta_sink, theta_dummy, theta_spatial, theta_score, gamma, percentile;
  int32_t rule;
};
hipError_t launch_classify_reduce(const ReducePlan& plan, hipStream_t s);

}  // namespace hc
