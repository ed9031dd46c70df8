// Host side of libheadcast.so: argument checking, the restructured cache's
// layout, work plans and kernel launches.  Allocates no device memory (the
// one device array it owns, the static classifier scratch, is part of the
// loaded code object) and never synchronises the device.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <queue>
#include <string>
#include <vector>

#include "hc_internal.h"

using namespace hc;

namespace {

thread_local std::string g_err;

hc_status fail(hc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

hc_status hip_fail(hipError_t e, const char* what) {
  return fail(HC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elt_size(int dtype) { return dtype == HC_BF16 ? 2 : 4; }
bool kv_fp8(const hc_config* c) { return c->kv_format == HC_KV_FP8_E4M3; }
size_t kv_elt_size(const hc_config* c) { return kv_fp8(c) ? 1 : elt_size(c->dtype); }
float scale_or_one(float s) { return s > 0.f ? s : 1.0f; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

hc_status check_config(const hc_config* c) {
  if (!c) return fail(HC_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype != HC_BF16 && c->dtype != HC_FP32) return fail(HC_ERR_DTYPE, "dtype %d is not HC_BF16 or HC_FP32", c->dtype);
  if (c->num_heads < 1 || c->num_heads > HC_MAX_HEADS)
    return fail(HC_ERR_SHAPE, "num_heads %d outside 1..%d", c->num_heads, HC_MAX_HEADS);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(HC_ERR_SHAPE, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->grid_h < 1 || c->grid_w < 1) return fail(HC_ERR_SHAPE, "grid %dx%d is empty", c->grid_h, c->grid_w);
  if (c->block_frames < 1 || c->window_frames < c->block_frames || c->window_frames % c->block_frames)
    return fail(HC_ERR_SHAPE, "window_frames %d must be a positive multiple of block_frames %d", c->window_frames,
                c->block_frames);
  if (c->cell_h < 1 || c->cell_w < 1) return fail(HC_ERR_SHAPE, "cell %dx%d is empty", c->cell_h, c->cell_w);
  const int64_t T = (int64_t)c->grid_h * c->grid_w;
  if (T * c->window_frames * c->head_dim > (int64_t)1 << 31)
    return fail(HC_ERR_SHAPE, "window of %lld tokens x %d channels is too large", (long long)(T * c->window_frames),
                c->head_dim);
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale))
    return fail(HC_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (c->kv_format != HC_KV_SAME && c->kv_format != HC_KV_FP8_E4M3)
    return fail(HC_ERR_INVALID_ARG, "kv_format %d is not HC_KV_SAME or HC_KV_FP8_E4M3", c->kv_format);
  if (kv_fp8(c)) {
    if (c->dtype != HC_BF16) return fail(HC_ERR_DTYPE, "fp8 K/V need dtype HC_BF16");
    for (float sc : {c->k_scale, c->v_scale})
      if (!(sc >= 0.f) || !std::isfinite(sc)) return fail(HC_ERR_INVALID_ARG, "k_scale and v_scale must be finite and >= 0");
  }
  return HC_OK;
}

hc_status check_tensor(const void* ptr, int64_t sh, int64_t st, const hc_config* c, const char* name) {
  const size_t e = elt_size(c->dtype);
  if (!ptr) return fail(HC_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if ((uintptr_t)ptr % 16) return fail(HC_ERR_ALIGN, "%s: pointer not 16-byte aligned", name);
  if (st < c->head_dim) return fail(HC_ERR_SHAPE, "%s: token stride %lld < head_dim", name, (long long)st);
  if (sh < 0) return fail(HC_ERR_SHAPE, "%s: negative head stride", name);
  if ((st * (int64_t)e) % 16 || (sh * (int64_t)e) % 16)
    return fail(HC_ERR_ALIGN, "%s: strides must be multiples of 16 bytes", name);
  return HC_OK;
}

float softmax_scale(const hc_config* c) {
  return c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
}

struct Geom {
  int T, Nq, Nk, nb, q_tiles, n_cells, cell_cols, cell_subtiles;
  std::vector<int> cell_size;
};

int qtile_of(const hc_config* c) { return c->dtype == HC_BF16 ? QTILE_BF16 : QTILE_F32; }

Geom geometry(const hc_config* c) {
  Geom g;
  const int QTILE = qtile_of(c);
  g.T = c->grid_h * c->grid_w;
  g.Nq = c->block_frames * g.T;
  g.Nk = c->window_frames * g.T;
  g.nb = c->window_frames / c->block_frames;
  g.q_tiles = cdiv(g.Nq, QTILE);
  const int rows = cdiv(c->grid_h, c->cell_h);
  g.cell_cols = cdiv(c->grid_w, c->cell_w);
  g.n_cells = rows * g.cell_cols;
  const int max_cell = std::min(c->cell_h, c->grid_h) * std::min(c->cell_w, c->grid_w);
  g.cell_subtiles = cdiv((int64_t)c->block_frames * max_cell, QTILE);
  for (int cy = 0; cy < rows; ++cy)
    for (int cx = 0; cx < g.cell_cols; ++cx) {
      const int h = std::min(c->cell_h, c->grid_h - cy * c->cell_h);
      const int w = std::min(c->cell_w, c->grid_w - cx * c->cell_w);
      g.cell_size.push_back(h * w);
    }
  return g;
}

// How the attention kernel's work spreads over an MI355X.  hc_attend
// launches the bf16 kernel in its persistent mode: one work group per
// compute unit (256), 32 on each of the 8 XCDs, each taking the units of
// its XCD's list one after another as it comes free (list scheduling on 32
// units per XCD).  An XCD's list holds, category by category, its
// contiguous run of each ranged category's units and every eighth Spatial
// unit.
constexpr int kXcds = 8, kUnitsPerXcd = 32, kPersistentGroups = kXcds * kUnitsPerXcd;

// Measured cost of one work unit of the bf16 kernel, in microseconds
// (per-work-group timestamps: s_memrealtime at each unit's start and end): a
// key tile of a full (> 64 queries) unit, a key tile of a small unit (bf16
// K/V: four key phases over eight waves; fp8 K/V: two key halves over four
// waves), and the per-unit set-up and write-back (with split partials and
// merge when a key range is split).
constexpr double kTileUs = 1.65, kSmallTileUs = 0.80, kSmallTileUsFp8 = 1.42;
constexpr double kUnitUs = 8.0, kSplitUnitUs = 24.0, kSmallUnitUs = 6.0;

// Simulated duration of one hc_attend launch of a full window, in
// microseconds, for the given key-range splits.
double simulate(const hc_config* c, const Geom& g, const int count[4], const int splits[4]) {
  const int qt = qtile_of(c);
  const int64_t q_last = g.Nq - (int64_t)(g.q_tiles - 1) * qt;   // queries of a head's last q tile
  const double small_tile = kv_fp8(c) ? kSmallTileUsFp8 : kSmallTileUs;
  auto cost = [&](int64_t queries, int key_tiles, bool split) {
    if (queries <= 64) return key_tiles * small_tile + kSmallUnitUs;
    return key_tiles * kTileUs + (split ? kSplitUnitUs : kUnitUs);
  };
  double makespan = 0.0;
  for (int x = 0; x < kXcds; ++x) {
    double cu[kUnitsPerXcd] = {};
    auto run = [&](double us) {
      int k = 0;
      for (int i = 1; i < kUnitsPerXcd; ++i)
        if (cu[i] < cu[k]) k = i;
      cu[k] += us;
      makespan = std::max(makespan, cu[k]);
    };
    for (int lab : {HC_GLOBAL, HC_SINK, HC_DUMMY}) {   // the kernel's category order
      if (!count[lab]) continue;
      const int s = splits[lab];
      const int per = cdiv(cdiv(lab == HC_GLOBAL ? g.Nk : g.Nq, KTILE), s);
      const int n = count[lab] * s * g.q_tiles;       // units (head, split, q tile), q tile fastest
      const int q8 = n >> 3, r8 = n & 7;
      const int first = x * q8 + std::min(x, r8), len = q8 + (x < r8 ? 1 : 0);
      for (int rel = first; rel < first + len; ++rel) {
        const bool last = rel % g.q_tiles == g.q_tiles - 1;
        run(cost(last ? q_last : qt, per, s > 1));
      }
    }
    if (count[HC_SPATIAL]) {                      // units (q sub-tile, head, cell), every eighth
      const int per_st = count[HC_SPATIAL] * g.n_cells;
      for (int rel = x; rel < g.cell_subtiles * per_st; rel += kXcds) {
        const int st = rel / per_st, cl = rel % g.n_cells;
        const int64_t q_cell = (int64_t)c->block_frames * g.cell_size[cl];
        const int64_t q = std::min<int64_t>(qt, q_cell - (int64_t)st * qt);
        if (q > 0) run(cost(q, cdiv((int64_t)c->window_frames * g.cell_size[cl], KTILE), false));
      }
    }
  }
  return makespan;
}

// Splits for Global heads and one count shared by Sink and Dummy heads (same
// key-set size), searched jointly for the shortest simulated launch; a count
// pair with more splits must be 0.5% faster to be taken.  Each split keeps at
// least 4 key tiles.
void choose_splits(const hc_config* c, const Geom& g, const int count[4], int splits[4]) {
  for (int i = 0; i < 4; ++i) splits[i] = 1;
  if (c->dtype != HC_BF16) return;
  const int gt = cdiv(g.Nk, KTILE), st = cdiv(g.Nq, KTILE);
  const int g_max = count[HC_GLOBAL] ? std::min(kMaxSplits, gt / 4) : 1;
  const int s_max = (count[HC_SINK] + count[HC_DUMMY]) ? std::min(kMaxSplits, st / 4) : 1;
  double best_t = 0.0;
  int best_g = 1, best_s = 1;
  for (int gs = 1; gs <= std::max(1, g_max); ++gs)
    for (int ss = 1; ss <= std::max(1, s_max); ++ss) {
      int trial[4] = {1, 1, 1, 1};
      trial[HC_GLOBAL] = gs;
      trial[HC_SINK] = trial[HC_DUMMY] = ss;
      const double t = simulate(c, g, count, trial);
      const bool first = gs == 1 && ss == 1;
      const bool more = gs + ss > best_g + best_s;
      if (first || t < (more ? 0.995 : 1.0) * best_t) {
        best_t = t;
        best_g = gs;
        best_s = ss;
      }
    }
  splits[HC_GLOBAL] = best_g;
  splits[HC_SINK] = splits[HC_DUMMY] = best_s;
}

struct Layout {
  int count[4] = {0, 0, 0, 0};
  int slot[HC_MAX_HEADS];
  uint8_t head_of[4][HC_MAX_HEADS];
  size_t off_k[4], off_v[4], slot_bytes[4];
  size_t off_part = 0, off_counters = 0, scratch_bytes = 0, total = 0;
  int splits[4] = {1, 1, 1, 1};         // key-range splits per archetype (Spatial: 1)
  size_t part_at[4] = {0, 0, 0, 0};     // byte offset of each archetype's partials
  int64_t counter_at[4] = {0, 0, 0, 0}; // first counter of each archetype
  int64_t work_at = -1;                 // first persistent-kernel counter (bf16 caches)
  int64_t n_counters = 0;
};

hc_status make_layout(const hc_config* c, const int8_t* labels, Layout* L) {
  hc_status st = check_config(c);
  if (st) return st;
  if (!labels) return fail(HC_ERR_INVALID_ARG, "labels is NULL");
  for (int h = 0; h < c->num_heads; ++h) {
    const int lab = labels[h];
    if (lab < HC_SINK || lab > HC_GLOBAL) return fail(HC_ERR_INVALID_ARG, "label of head %d is %d, not 0..3", h, lab);
    L->slot[h] = L->count[lab];
    L->head_of[lab][L->count[lab]++] = (uint8_t)h;
  }
  const Geom g = geometry(c);
  const size_t row = (size_t)c->head_dim * kv_elt_size(c);
  L->slot_bytes[HC_GLOBAL] = L->slot_bytes[HC_SPATIAL] = (size_t)g.Nk * row;
  L->slot_bytes[HC_SINK] = L->slot_bytes[HC_DUMMY] = (size_t)g.Nq * row;
  size_t off = 0;
  for (int lab : {HC_GLOBAL, HC_SINK, HC_DUMMY, HC_SPATIAL}) {
    L->off_k[lab] = off;
    off = align256(off + L->count[lab] * L->slot_bytes[lab]);
    L->off_v[lab] = off;
    off = align256(off + L->count[lab] * L->slot_bytes[lab]);
  }
  choose_splits(c, g, L->count, L->splits);
  // Scratch: fp32 partials of each split archetype, then one int32 counter
  // per (head, q tile) of every split archetype, all counters contiguous.
  L->off_part = off;
  for (int lab : {HC_GLOBAL, HC_SINK, HC_DUMMY}) {
    if (L->splits[lab] == 1) continue;
    const int64_t ids = (int64_t)L->count[lab] * g.q_tiles;
    L->part_at[lab] = off;
    off = align256(off + (size_t)ids * L->splits[lab] * qtile_of(c) * ((size_t)c->head_dim + 2) * sizeof(float));
  }
  L->off_counters = off;
  for (int lab : {HC_GLOBAL, HC_SINK, HC_DUMMY}) {
    if (L->splits[lab] == 1) continue;
    L->counter_at[lab] = L->n_counters;
    L->n_counters += (int64_t)L->count[lab] * g.q_tiles;
  }
  if (c->dtype == HC_BF16) {   // the persistent kernel's per-XCD unit and finish counters
    L->work_at = L->n_counters;
    L->n_counters += 2 * kXcds;
  }
  off = align256(off + (size_t)L->n_counters * sizeof(int32_t));
  L->scratch_bytes = off - L->off_part;
  L->total = off;
  return HC_OK;
}

}  // namespace

struct hc_cache {
  hc_config cfg;
  int8_t labels[HC_MAX_HEADS];
  Layout L;
  uint8_t* dev = nullptr;
  size_t bytes = 0;
  int n_appended = 0;
  bool counters_zeroed = false;
};

extern "C" {

void hc_default_classify_params(hc_classify_params* p) {
  if (!p) return;
  p->theta_sink = 0.95f;
  p->theta_dummy = 0.95f;
  p->theta_spatial = 0.95f;
  p->theta_score = 0.755f;
  p->gamma = 5.0f;
  p->percentile = 5.0f;
  p->rule = 0;
  p->spatial_proxy = 0;
  p->radius = 2;
}

hc_status hc_validate_config(const hc_config* cfg) { return check_config(cfg); }

hc_status hc_cache_bytes(const hc_config* cfg, const int8_t* labels_host, size_t* device_bytes) {
  if (!device_bytes) return fail(HC_ERR_INVALID_ARG, "device_bytes is NULL");
  Layout L;
  hc_status st = make_layout(cfg, labels_host, &L);
  if (st) return st;
  *device_bytes = L.total;
  return HC_OK;
}

hc_status hc_cache_create(const hc_config* cfg, const int8_t* labels_host, void* device_mem, size_t bytes,
                          hc_cache** out) {
  if (!out) return fail(HC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  Layout L;
  hc_status st = make_layout(cfg, labels_host, &L);
  if (st) return st;
  if (!device_mem) return fail(HC_ERR_INVALID_ARG, "device_mem is NULL");
  if ((uintptr_t)device_mem % 256) return fail(HC_ERR_ALIGN, "device_mem must be 256-byte aligned");
  if (bytes < L.total) return fail(HC_ERR_WORKSPACE, "cache needs %zu bytes, got %zu", L.total, bytes);
  hc_cache* c = new (std::nothrow) hc_cache;
  if (!c) return fail(HC_ERR_INVALID_ARG, "out of host memory");
  c->cfg = *cfg;
  std::memcpy(c->labels, labels_host, cfg->num_heads);
  c->L = L;
  c->dev = (uint8_t*)device_mem;
  c->bytes = bytes;
  *out = c;
  return HC_OK;
}

hc_status hc_cache_destroy(hc_cache* cache) {
  if (!cache) return fail(HC_ERR_INVALID_ARG, "cache is NULL");
  delete cache;
  return HC_OK;
}

hc_status hc_cache_get_layout(const hc_cache* c, hc_cache_layout* out) {
  if (!c || !out) return fail(HC_ERR_INVALID_ARG, "NULL argument");
  std::memset(out, 0, sizeof *out);
  out->total_bytes = c->L.total;
  out->off_global_k = c->L.off_k[HC_GLOBAL];
  out->off_global_v = c->L.off_v[HC_GLOBAL];
  out->off_sink_k = c->L.off_k[HC_SINK];
  out->off_sink_v = c->L.off_v[HC_SINK];
  out->off_dummy_k = c->L.off_k[HC_DUMMY];
  out->off_dummy_v = c->L.off_v[HC_DUMMY];
  out->off_spatial_k = c->L.off_k[HC_SPATIAL];
  out->off_spatial_v = c->L.off_v[HC_SPATIAL];
  out->off_scratch = c->L.off_part;
  out->scratch_bytes = c->L.scratch_bytes;
  out->n_global = c->L.count[HC_GLOBAL];
  out->n_sink = c->L.count[HC_SINK];
  out->n_dummy = c->L.count[HC_DUMMY];
  out->n_spatial = c->L.count[HC_SPATIAL];
  out->blocks_appended = c->n_appended;
  out->global_splits = c->L.splits[HC_GLOBAL];
  out->sink_splits = c->L.splits[HC_SINK];
  out->dummy_splits = c->L.splits[HC_DUMMY];
  for (int h = 0; h < c->cfg.num_heads; ++h) out->head_slot[h] = c->L.slot[h];
  return HC_OK;
}

hc_status hc_cache_append(hc_cache* c, hc_tensor k_block, hc_tensor v_block, int32_t mode, hipStream_t stream) {
  if (!c) return fail(HC_ERR_INVALID_ARG, "cache is NULL");
  if (mode != HC_PUSH_BLOCK && mode != HC_REPLACE_NEWEST) return fail(HC_ERR_INVALID_ARG, "mode %d", mode);
  const hc_config* cfg = &c->cfg;
  hc_status st = check_tensor(k_block.ptr, k_block.stride_head, k_block.stride_token, cfg, "k_block");
  if (st) return st;
  st = check_tensor(v_block.ptr, v_block.stride_head, v_block.stride_token, cfg, "v_block");
  if (st) return st;
  if (k_block.stride_head != v_block.stride_head || k_block.stride_token != v_block.stride_token)
    return fail(HC_ERR_SHAPE, "k_block and v_block must share strides");
  if (mode == HC_REPLACE_NEWEST && c->n_appended == 0) return fail(HC_ERR_STATE, "REPLACE_NEWEST before any block");
  const Geom g = geometry(cfg);
  const int b = (mode == HC_PUSH_BLOCK) ? c->n_appended : c->n_appended - 1;
  const size_t e = elt_size(cfg->dtype);

  if (c->L.n_counters > 0 && !c->counters_zeroed) {
    hipError_t err = launch_fill_zero((int32_t*)(c->dev + c->L.off_counters), c->L.n_counters, stream);
    if (err != hipSuccess) return hip_fail(err, "append: zeroing the cache's counters");
    c->counters_zeroed = true;
  }

  AppendPlan P;
  std::memset(&P, 0, sizeof P);
  P.k = (const uint8_t*)k_block.ptr;
  P.v = (const uint8_t*)v_block.ptr;
  P.src_sh = k_block.stride_head * (int64_t)e;
  P.src_st = k_block.stride_token * (int64_t)e;
  P.row_bytes = cfg->head_dim * (int)e;
  P.dst_row_bytes = cfg->head_dim * (int)kv_elt_size(cfg);
  P.quant = kv_fp8(cfg) ? 1 : 0;
  P.inv_k = 1.0f / scale_or_one(cfg->k_scale);
  P.inv_v = 1.0f / scale_or_one(cfg->v_scale);
  P.rows = g.Nq;
  P.H = cfg->num_heads;
  P.T = g.T;
  P.grid_w = cfg->grid_w;
  P.grid_h = cfg->grid_h;
  P.cell_h = cfg->cell_h;
  P.cell_w = cfg->cell_w;
  P.cell_cols = g.cell_cols;
  P.B = cfg->block_frames;
  P.W = cfg->window_frames;
  P.ring_slot = b % g.nb;
  P.write_sink = (b == 0);
  for (int lab = 0; lab < 4; ++lab) {
    P.dst_k[lab] = c->dev + c->L.off_k[lab];
    P.dst_v[lab] = c->dev + c->L.off_v[lab];
    P.dst_slot_bytes[lab] = (int64_t)c->L.slot_bytes[lab];
  }
  for (int h = 0; h < cfg->num_heads; ++h) {
    P.label[h] = (uint8_t)c->labels[h];
    P.slot[h] = (uint8_t)c->L.slot[h];
  }
  hipError_t err = launch_append(P, stream);
  if (err != hipSuccess) return hip_fail(err, "append kernel launch");
  if (mode == HC_PUSH_BLOCK) ++c->n_appended;
  return HC_OK;
}

hc_status hc_attend(hc_cache* c, hc_tensor q, hc_out_tensor out, hipStream_t stream) {
  if (!c) return fail(HC_ERR_INVALID_ARG, "cache is NULL");
  const hc_config* cfg = &c->cfg;
  hc_status st = check_tensor(q.ptr, q.stride_head, q.stride_token, cfg, "q_block");
  if (st) return st;
  st = check_tensor(out.ptr, out.stride_head, out.stride_token, cfg, "out");
  if (st) return st;
  if (out.ptr == q.ptr) return fail(HC_ERR_INVALID_ARG, "out aliases q_block");
  if (c->n_appended < 1) return fail(HC_ERR_STATE, "hc_attend before any block was appended");
  const Geom g = geometry(cfg);
  const int nblk = std::min(c->n_appended, g.nb);
  const bool bf16 = cfg->dtype == HC_BF16;

  AttnPlan P;
  std::memset(&P, 0, sizeof P);
  P.q_tiles = g.q_tiles;
  P.cell_subtiles = g.cell_subtiles;
  P.q = q.ptr;
  P.q_sh = q.stride_head;
  P.q_st = q.stride_token;
  P.T = g.T;
  P.grid_w = cfg->grid_w;
  P.grid_h = cfg->grid_h;
  P.cell_h = cfg->cell_h;
  P.cell_w = cfg->cell_w;
  P.cell_cols = g.cell_cols;
  P.B = cfg->block_frames;
  P.W = cfg->window_frames;
  P.Nq = g.Nq;
  P.scale_log2 = softmax_scale(cfg) * 1.4426950408889634f;
  P.v_scale = 1.0f;
  if (kv_fp8(cfg)) {   // scores and outputs of the decoded codes, times the scales
    P.kv8 = 1;
    P.scale_log2 *= scale_or_one(cfg->k_scale);
    P.v_scale = scale_or_one(cfg->v_scale);
  }
  const size_t ke = kv_elt_size(cfg);
  const int64_t slot_elems[4] = {(int64_t)(c->L.slot_bytes[0] / ke), (int64_t)(c->L.slot_bytes[1] / ke),
                                 (int64_t)(c->L.slot_bytes[2] / ke), (int64_t)(c->L.slot_bytes[3] / ke)};
  int units = 0;
  for (int lab : {HC_GLOBAL, HC_SINK, HC_DUMMY, HC_SPATIAL}) {
    const int n = c->L.count[lab];
    if (!n) continue;
    AttnCat& C = P.cat[P.n_cats];
    C.n_heads = n;
    C.k = c->dev + c->L.off_k[lab];
    C.v = c->dev + c->L.off_v[lab];
    C.kv_sh = slot_elems[lab];
    C.kv_st = cfg->head_dim;
    C.o = out.ptr;
    C.o_sh = out.stride_head;
    C.o_st = out.stride_token;
    C.out_f32 = bf16 ? 0 : 1;
    C.unit_begin = units;
    C.splits = 1;
    if (lab == HC_SPATIAL) {
      C.kind = KIND_CELL_MAJOR;
      C.kv_count = nblk * cfg->block_frames;   // frames present
      C.units_per_head = g.n_cells * g.cell_subtiles;
    } else {
      C.kind = KIND_RANGED;
      C.kv_first = 0;
      C.kv_count = (lab == HC_GLOBAL) ? nblk * g.Nq : g.Nq;
      C.keys_per_split = C.kv_count;
      if (c->L.splits[lab] > 1) {
        const int tiles = cdiv(C.kv_count, KTILE);
        const int kps = cdiv(tiles, c->L.splits[lab]) * KTILE;
        C.keys_per_split = kps;
        C.splits = cdiv(C.kv_count, kps);
        C.part = (float*)(c->dev + c->L.part_at[lab]);
        C.counters = (int32_t*)(c->dev + c->L.off_counters) + c->L.counter_at[lab];
      }
      C.units_per_head = g.q_tiles * C.splits;
    }
    for (int s = 0; s < n; ++s) P.head_of[P.n_cats][s] = c->L.head_of[lab][s];
    units += n * C.units_per_head;
    ++P.n_cats;
  }
  P.total_units = units;
  if (bf16) {   // persistent mode: one work group per compute unit
    P.work_ctr = (int32_t*)(c->dev + c->L.off_counters) + c->L.work_at;
    P.grid = std::min(units, kPersistentGroups);
  }
  hipError_t err = bf16 ? launch_attn_bf16(P, cfg->head_dim, stream) : launch_attn_f32(P, cfg->head_dim, stream);
  if (err != hipSuccess) return hip_fail(err, "attention kernel launch");
  return HC_OK;
}

hc_status hc_classify_workspace_bytes(const hc_config* cfg, size_t* bytes) {
  if (!bytes) return fail(HC_ERR_INVALID_ARG, "bytes is NULL");
  hc_status st = check_config(cfg);
  if (st) return st;
  const Geom g = geometry(cfg);
  const size_t o = align256((size_t)4 * cfg->num_heads * g.Nq * cfg->head_dim * sizeof(float));
  const size_t cs = align256((size_t)cfg->num_heads * 4 * g.Nq * sizeof(float));
  const size_t ml = align256((size_t)3 * cfg->num_heads * g.Nq * 2 * sizeof(float));
  *bytes = o + cs + ml;
  return HC_OK;
}

}  // extern "C"

namespace {

// Every check of hc_classify except those of the workspace, which the two
// entry points bring in differently.
hc_status check_classify(const hc_config* cfg, const hc_classify_params* prm, hc_tensor q, hc_tensor k_window,
                         hc_tensor v_window, int8_t* labels_dev, float* diag_dev) {
  hc_status st = check_config(cfg);
  if (st) return st;
  if (!prm) return fail(HC_ERR_INVALID_ARG, "params is NULL");
  if (prm->rule != 0 && prm->rule != 1) return fail(HC_ERR_INVALID_ARG, "rule %d", prm->rule);
  if (prm->spatial_proxy != 0 && prm->spatial_proxy != 1) return fail(HC_ERR_INVALID_ARG, "spatial_proxy %d", prm->spatial_proxy);
  if (prm->spatial_proxy == 1 && (prm->radius < 0 || prm->radius > kMaxBoxRadius))
    return fail(HC_ERR_INVALID_ARG, "radius %d outside 0..%d", prm->radius, kMaxBoxRadius);
  if (!(prm->percentile >= 0.f && prm->percentile <= 100.f)) return fail(HC_ERR_INVALID_ARG, "percentile outside 0..100");
  if (!std::isfinite(prm->gamma)) return fail(HC_ERR_INVALID_ARG, "gamma is not finite");
  if ((st = check_tensor(q.ptr, q.stride_head, q.stride_token, cfg, "q_block"))) return st;
  if ((st = check_tensor(k_window.ptr, k_window.stride_head, k_window.stride_token, cfg, "k_window"))) return st;
  if ((st = check_tensor(v_window.ptr, v_window.stride_head, v_window.stride_token, cfg, "v_window"))) return st;
  if (k_window.stride_head != v_window.stride_head || k_window.stride_token != v_window.stride_token)
    return fail(HC_ERR_SHAPE, "k_window and v_window must share strides");
  if (!labels_dev || !diag_dev) return fail(HC_ERR_INVALID_ARG, "labels_dev / diag_dev is NULL");
  return HC_OK;
}

// The classifier's launches over a checked configuration and a workspace of
// at least hc_classify_workspace_bytes.
hc_status classify_launch(const hc_config* cfg, const hc_classify_params* prm, hc_tensor q, hc_tensor k_window,
                          hc_tensor v_window, void* workspace, int8_t* labels_dev, float* diag_dev,
                          hipStream_t stream) {
  const Geom g = geometry(cfg);
  const int H = cfg->num_heads, D = cfg->head_dim;
  float* O = (float*)workspace;
  float* Cc = (float*)((uint8_t*)workspace + align256((size_t)4 * H * g.Nq * D * sizeof(float)));
  const int64_t plane = (int64_t)H * g.Nq * D;

  AttnPlan P;
  std::memset(&P, 0, sizeof P);
  P.q_tiles = g.q_tiles;
  P.cell_subtiles = g.cell_subtiles;
  P.q = q.ptr;
  P.q_sh = q.stride_head;
  P.q_st = q.stride_token;
  P.T = g.T;
  P.grid_w = cfg->grid_w;
  P.grid_h = cfg->grid_h;
  P.cell_h = cfg->cell_h;
  P.cell_w = cfg->cell_w;
  P.cell_cols = g.cell_cols;
  P.B = cfg->block_frames;
  P.W = cfg->window_frames;
  P.Nq = g.Nq;
  P.scale_log2 = softmax_scale(cfg) * 1.4426950408889634f;
  P.v_scale = 1.0f;
  // outputs: 0 full, 1 sink, 2 dummy, 3 spatial
  const int first[3] = {0, 0, g.Nk - g.Nq};
  const int count[3] = {g.Nk, g.Nq, g.Nq};
  int units = 0;
  for (int k = 0; k < 4; ++k) {
    AttnCat& C = P.cat[k];
    C.n_heads = H;
    C.k = k_window.ptr;
    C.v = v_window.ptr;
    C.kv_sh = k_window.stride_head;
    C.kv_st = k_window.stride_token;
    C.o = O + k * plane;
    C.o_sh = (int64_t)g.Nq * D;
    C.o_st = D;
    C.out_f32 = 1;
    C.splits = 1;
    C.unit_begin = units;
    if (k < 3) {
      C.kind = KIND_RANGED;
      C.kv_first = first[k];
      C.kv_count = count[k];
      C.keys_per_split = count[k];
      C.units_per_head = g.q_tiles;
    } else if (prm->spatial_proxy == 0) {
      C.kind = KIND_CELL_GATHER;
      C.kv_count = cfg->window_frames;
      C.units_per_head = g.n_cells * g.cell_subtiles;
    } else {
      // sliding (2r+1)^2 box: patches of (queries per work group / 32) rows x
      // (32 - 2r) columns, so each patch's key rows are 32 columns wide
      C.kind = KIND_BOX_GATHER;
      C.kv_count = cfg->window_frames;
      P.box_r = prm->radius;
      P.box_rows = (cfg->dtype == HC_BF16 ? QTILE_BF16 : QTILE_F32) / 32;
      P.box_cols_q = 32 - 2 * prm->radius;
      P.box_bands_y = cdiv(cfg->grid_h, P.box_rows);
      P.box_bands_x = cdiv(cfg->grid_w, P.box_cols_q);
      C.units_per_head = cfg->block_frames * P.box_bands_y * P.box_bands_x;
    }
    for (int h = 0; h < H; ++h) P.head_of[k][h] = (uint8_t)h;
    units += H * C.units_per_head;
  }
  P.n_cats = 4;
  P.total_units = units;
  hipError_t err;
  if (cfg->dtype == HC_BF16) {
    // The Sink and Dummy proxies' keys (the window's first and last block) are
    // part of the full output's keys, so each key is attended once: the first
    // block, the middle blocks and the last block are three contiguous ranges,
    // each written unnormalised with its softmax state, and a merge kernel
    // forms the full output and the two proxies.  The matrix-core kernel is
    // specialised on gathered keys, so the Spatial proxy is a second launch.
    float2* ML = (float2*)((uint8_t*)workspace + align256((size_t)4 * H * g.Nq * D * sizeof(float)) +
                           align256((size_t)H * 4 * g.Nq * sizeof(float)));
    const int64_t rows = (int64_t)H * g.Nq;
    AttnPlan R = P;
    R.n_cats = 0;
    int ru = 0;
    auto add_range = [&](int out_plane, int first, int count, float2* ml) {
      AttnCat C = P.cat[0];
      C.kv_first = first;
      C.kv_count = count;
      C.keys_per_split = count;
      C.o = O + out_plane * plane;
      C.ml_out = ml;
      C.unit_begin = ru;
      R.cat[R.n_cats++] = C;
      ru += H * C.units_per_head;
    };
    if (g.nb >= 3) add_range(0, g.Nq, g.Nk - 2 * g.Nq, ML + rows);   // middle blocks (heaviest first)
    add_range(1, 0, g.Nq, ML);                                       // first block
    if (g.nb >= 2) add_range(2, g.Nk - g.Nq, g.Nq, ML + 2 * rows);   // last block
    R.total_units = ru;
    AttnPlan G = P;
    G.cat[0] = G.cat[3];
    G.cat[0].unit_begin = 0;
    G.n_cats = 1;
    G.total_units = H * G.cat[0].units_per_head;
    err = launch_attn_bf16(R, D, stream);
    if (err == hipSuccess) err = launch_attn_bf16(G, D, stream);
    if (err == hipSuccess) {
      MergePlan mp{O, ML, H, g.Nq, D, g.nb >= 3 ? 1 : 0, g.nb == 1 ? 1 : 0, P.scale_log2};
      err = launch_merge_ranges(mp, stream);
    }
  } else {
    err = launch_attn_f32(P, D, stream);
  }
  if (err != hipSuccess) return hip_fail(err, "classifier attention launch");

  CosPlan cp{O, Cc, H, g.Nq, D};
  err = launch_cosines(cp, stream);
  if (err != hipSuccess) return hip_fail(err, "classifier cosine launch");
  ReducePlan rp;
  rp.c = Cc;
  rp.labels = labels_dev;
  rp.diag = diag_dev;
  rp.H = H;
  rp.Nq = g.Nq;
  rp.D = D;
  rp.theta_sink = prm->theta_sink;
  rp.theta_dummy = prm->theta_dummy;
  rp.theta_spatial = prm->theta_spatial;
  rp.theta_score = prm->theta_score;
  rp.gamma = prm->gamma;
  rp.percentile = prm->percentile;
  rp.rule = prm->rule;
  err = launch_classify_reduce(rp, stream);
  if (err != hipSuccess) return hip_fail(err, "classifier reduce launch");
  return HC_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free classifier: the workspace is this file-scope device array
// instead of caller memory.  Host code must not use the array's name as an
// address (it is a host-side stand-in); its device address is looked up once
// per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[HC_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`.
hc_status scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDevice_t dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(HC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) hipSetDevice(cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || (uintptr_t)p % 256) return fail(HC_ERR_HIP, "scratch array has no usable device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HC_OK;
}

}  // namespace

extern "C" {

hc_status hc_classify(const hc_config* cfg, const hc_classify_params* prm, hc_tensor q, hc_tensor k_window,
                      hc_tensor v_window, void* workspace, size_t ws_bytes, int8_t* labels_dev, float* diag_dev,
                      hipStream_t stream) {
  hc_status st = check_classify(cfg, prm, q, k_window, v_window, labels_dev, diag_dev);
  if (st) return st;
  if (!workspace) return fail(HC_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(HC_ERR_ALIGN, "workspace must be 256-byte aligned");
  size_t need = 0;
  hc_classify_workspace_bytes(cfg, &need);
  if (ws_bytes < need) return fail(HC_ERR_WORKSPACE, "classifier needs %zu workspace bytes, got %zu", need, ws_bytes);
  return classify_launch(cfg, prm, q, k_window, v_window, workspace, labels_dev, diag_dev, stream);
}

hc_status hc_classify_static(const hc_config* cfg, const hc_classify_params* prm, hc_tensor q, hc_tensor k_window,
                             hc_tensor v_window, int8_t* labels_dev, float* diag_dev, hipStream_t stream) {
  hc_status st = check_classify(cfg, prm, q, k_window, v_window, labels_dev, diag_dev);
  if (st) return st;
  size_t need = 0;
  hc_classify_workspace_bytes(cfg, &need);
  if (need > (size_t)HC_STATIC_SCRATCH_BYTES)
    return fail(HC_ERR_WORKSPACE, "hc_classify_static: this layer needs %zu workspace bytes, more than the %zu of "
                "the library's static scratch; use hc_classify with a caller workspace", need,
                (size_t)HC_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(stream, &ws))) return st;
  return classify_launch(cfg, prm, q, k_window, v_window, ws, labels_dev, diag_dev, stream);
}

const char* hc_status_string(hc_status s) {
  switch (s) {
    case HC_OK: return "HC_OK";
    case HC_ERR_INVALID_ARG: return "HC_ERR_INVALID_ARG";
    case HC_ERR_SHAPE: return "HC_ERR_SHAPE";
    case HC_ERR_DTYPE: return "HC_ERR_DTYPE";
    case HC_ERR_ALIGN: return "HC_ERR_ALIGN";
    case HC_ERR_WORKSPACE: return "HC_ERR_WORKSPACE";
    case HC_ERR_STATE: return "HC_ERR_STATE";
    case HC_ERR_HIP: return "HC_ERR_HIP";
    case HC_ERR_UNSUPPORTED: return "HC_ERR_UNSUPPORTED";
  }
  return "HC_ERR_UNKNOWN";
}

const char* hc_last_error_message(void) { return g_err.c_str(); }

}  // extern "C"
