// fp32 head-routed attention on the vector ALUs.  Same work plan and key sets
// as the bf16 matrix-core kernel (every pathway is exact softmax attention
// over the head's key set; HeadCast review page, "What carries the
// argument"), for fp32 layers where results must hold to fp32 accuracy.
// Two lanes share a query (each owns half of the channels); 32-key tiles of K
// and V are staged in LDS; softmax is online, one tile at a time.
#include "hc_internal.h"

namespace hc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int FKT = 32;   // keys per LDS tile

template <int D>
__global__ __launch_bounds__(NT) void attn_f32_kernel(const AttnPlan P) {
  constexpr int H2 = D / 2;
  __shared__ __attribute__((aligned(16))) float Ks[FKT][D];
  __shared__ __attribute__((aligned(16))) float Vs[FKT][D];

  const int u = blockIdx.x;
  if (u >= P.total_units) return;
  int ci = 0;
#pragma unroll
  for (int c = 1; c < 4; ++c)
    if (c < P.n_cats && u >= P.cat[c].unit_begin) ci = c;
  const AttnCat& C = P.cat[ci];
  const int rel = u - C.unit_begin;
  const int slot = rel / C.units_per_head;
  const int j = rel - slot * C.units_per_head;
  const int qh = P.head_of[ci][slot];
  const float* Kb = (const float*)C.k + slot * C.kv_sh;
  const float* Vb = (const float*)C.v + slot * C.kv_sh;
  const float* Qb = (const float*)P.q + qh * P.q_sh;

  int q0, qn, k0, kn;
  CellInfo cell = {0, 0, 1, 0};
  BoxInfo box = {0, 0, 0};
  const bool ranged = C.kind == KIND_RANGED;
  const bool is_box = C.kind == KIND_BOX_GATHER;
  if (ranged) {
    const int split = j / P.q_tiles;
    const int tile = j - split * P.q_tiles;
    q0 = tile * QTILE_F32;
    qn = min(QTILE_F32, P.Nq - q0);
    k0 = C.kv_first;
    kn = C.kv_count;   // this kernel never splits the key range
    (void)split;
  } else if (is_box) {
    box = box_info(P, j);
    q0 = 0;
    qn = QTILE_F32;
    kn = C.kv_count * (P.box_rows + 2 * P.box_r) * 32;
    k0 = 0;
  } else {
    const int c = j / P.cell_subtiles;
    const int st = j - c * P.cell_subtiles;
    cell = cell_info(P, c);
    q0 = st * QTILE_F32;
    const int qall = P.B * cell.size;
    if (q0 >= qall) return;
    qn = min(QTILE_F32, qall - q0);
    kn = C.kv_count * cell.size;
    k0 = (C.kind == KIND_CELL_MAJOR) ? P.W * cell.off : 0;
  }
  const bool gather = C.kind == KIND_CELL_GATHER || is_box;

  const int tid = threadIdx.x;
  const int ql = tid >> 1, half = tid & 1;
  // box proxy: query ql is patch row ql / 32, column ql % 32
  const int qy = box.py0 + (ql >> 5), qx = box.px0 + (ql & 31);
  const bool qvalid = is_box ? ((ql & 31) < P.box_cols_q && qy < P.grid_h && qx < P.grid_w) : ql < qn;
  int qtok = 0;
  if (qvalid) qtok = is_box ? box.fb * P.T + qy * P.grid_w + qx : ranged ? q0 + ql : cell_token(P, cell, q0 + ql);
  float q[H2], o[H2];
#pragma unroll
  for (int c = 0; c < H2; ++c) {
    q[c] = qvalid ? Qb[(int64_t)qtok * P.q_st + half * H2 + c] : 0.f;
    o[c] = 0.f;
  }
  const float c2 = P.scale_log2;
  float m = -INFINITY, l = 0.f;

  constexpr int CPR = D / 4;  // float4 chunks per row
  for (int kb = 0; kb < kn; kb += FKT) {
    __syncthreads();
    for (int idx = tid; idx < FKT * CPR; idx += NT) {
      const int r = idx / CPR, ch = idx - r * CPR;
      const int kk = kb + r;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (kk < kn) {
        const int64_t row = is_box ? (int64_t)box_token(P, box, kk)
                            : gather ? (int64_t)cell_token(P, cell, kk) : (int64_t)(k0 + kk);
        a = *(const f32x4*)(Kb + row * C.kv_st + 4 * ch);
        b = *(const f32x4*)(Vb + row * C.kv_st + 4 * ch);
      }
      *(f32x4*)&Ks[r][4 * ch] = a;
      *(f32x4*)&Vs[r][4 * ch] = b;
    }
    __syncthreads();
    // The tile's scores first, then its weights and weighted values summed
    // within the tile, then one merge into the running state.  Every sum is a
    // chain of at most FKT terms plus one term per tile, so rounding grows
    // with sqrt(FKT) + sqrt(keys / FKT) instead of sqrt(keys).  Rows past the
    // key set were loaded as zeros and are masked here.
    const int nk = min(FKT, kn - kb);
    uint32_t keep = nk == FKT ? ~0u : (1u << nk) - 1u;   // bit r: key kb + r counts
    if (is_box) {   // only keys within r rows and r columns of the query, on the grid
      for (int r = 0; r < nk; ++r) {
        int f, ky, kx;
        box_pos(P, box, kb + r, f, ky, kx);
        const bool ok = ky >= 0 && ky < P.grid_h && kx >= 0 && kx < P.grid_w && abs(ky - qy) <= P.box_r &&
                        abs(kx - qx) <= P.box_r;
        if (!ok) keep &= ~(1u << r);
      }
    }
    float s[FKT];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < FKT; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < H2; ++c) dot = fmaf(q[c], Ks[r][half * H2 + c], dot);
      dot += __shfl_xor(dot, 1, 64);
      s[r] = (keep >> r) & 1u ? dot * c2 : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    if (mt > -INFINITY) {   // the same for both lanes of a query pair
      float lt = 0.f, ot[H2];
#pragma unroll
      for (int c = 0; c < H2; ++c) ot[c] = 0.f;
#pragma unroll
      for (int r = 0; r < FKT; ++r) {
        const float p = exp2f(s[r] - mt);   // 0 for masked keys
        lt += p;
#pragma unroll
        for (int c = 0; c < H2; ++c) ot[c] = fmaf(p, Vs[r][half * H2 + c], ot[c]);
      }
      const float mn = fmaxf(m, mt);
      const float a = exp2f(m - mn), b = exp2f(mt - mn);
      l = fmaf(l, a, lt * b);
#pragma unroll
      for (int c = 0; c < H2; ++c) o[c] = fmaf(o[c], a, ot[c] * b);
      m = mn;
    }
  }
  if (!qvalid) return;
  const float inv = 1.f / l;
  float* out = (float*)C.o + (int64_t)qh * C.o_sh + (int64_t)qtok * C.o_st + half * H2;
#pragma unroll
  for (int c = 0; c < H2; ++c) out[c] = o[c] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const AttnPlan& plan, int head_dim, hipStream_t s) {
  if (plan.total_units <= 0) return hipSuccess;
  dim3 grid(plan.total_units), block(NT);
  if (head_dim == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, plan);
  else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, plan);
  return hipGetLastError();
}

}  // namespace hc
