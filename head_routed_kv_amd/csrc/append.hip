// Cache append: scatter one block's K/V rows into the per-archetype buffers
// of the restructured cache (HeadCast review page, "What carries the
// argument": the monolithic cache is split along the head dimension; Sink and
// Dummy keep one block, Global the sliding window, Spatial the window stored
// cell by cell).  Pure data movement, 16-byte vector copies; every row of the
// block is read once and written once (twice for the very first block of a
// Sink head, which is also its newest).
#include "hc_internal.h"

namespace hc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;

// Row of the archetype buffer that token t of the block goes to.
__device__ __forceinline__ int64_t dest_row(const AppendPlan& P, int lab, int t) {
  if (lab == HC_SPATIAL) {
    const int f = t / P.T;
    const int r = t - f * P.T;
    const int y = r / P.grid_w, x = r - y * P.grid_w;
    const int cy = y / P.cell_h, cx = x / P.cell_w;
    const int y0 = cy * P.cell_h, x0 = cx * P.cell_w;
    const int chh = min(P.cell_h, P.grid_h - y0), cww = min(P.cell_w, P.grid_w - x0);
    const int off = cy * P.cell_h * P.grid_w + cx * chh * P.cell_w;   // sum of earlier cell sizes
    const int size = chh * cww;
    const int fslot = P.ring_slot * P.B + f;
    return (int64_t)P.W * off + (int64_t)fslot * size + (y - y0) * cww + (x - x0);
  }
  if (lab == HC_GLOBAL) return (int64_t)P.ring_slot * P.rows + t;
  return t;
}

__global__ __launch_bounds__(NT) void append_kernel(const AppendPlan P) {
  const int h = blockIdx.y;
  const int lab = P.label[h];
  if (lab == HC_SINK && !P.write_sink) return;
  const int cpr = P.row_bytes >> 4;                 // 16-byte chunks per row
  const int64_t total = (int64_t)P.rows * cpr;
  const uint8_t* sk = P.k + h * P.src_sh;
  const uint8_t* sv = P.v + h * P.src_sh;
  uint8_t* dk = P.dst_k[lab] + P.slot[h] * P.dst_slot_bytes[lab];
  uint8_t* dv = P.dst_v[lab] + P.slot[h] * P.dst_slot_bytes[lab];
  for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * NT) {
    const int t = (int)(idx / cpr);
    const int ch = (int)(idx - (int64_t)t * cpr);
    const int64_t drow = dest_row(P, lab, t);
    const u32x4 a = *(const u32x4*)(sk + t * P.src_st + 16 * ch);
    const u32x4 b = *(const u32x4*)(sv + t * P.src_st + 16 * ch);
    *(u32x4*)(dk + drow * P.dst_row_bytes + 16 * ch) = a;
    *(u32x4*)(dv + drow * P.dst_row_bytes + 16 * ch) = b;
  }
}

// The same scatter into an fp8 cache: each thread turns 16 bf16 values (two
// 16-byte source chunks) into one 16-byte chunk of OCP E4M3 codes, code of
// fp32(x * inv), clamped to +-448 and rounded to nearest even by the
// conversion instruction.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t lo2, uint32_t hi2, float inv) {
  auto f = [&](uint32_t bits) { return fminf(fmaxf(__uint_as_float(bits) * inv, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(f(lo2 << 16), f(lo2 & 0xffff0000u), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(f(hi2 << 16), f(hi2 & 0xffff0000u), w, true);
  return (uint32_t)w;
}

__global__ __launch_bounds__(NT) void append_fp8_kernel(const AppendPlan P) {
  const int h = blockIdx.y;
  const int lab = P.label[h];
  if (lab == HC_SINK && !P.write_sink) return;
  const int cpr = P.dst_row_bytes >> 4;             // 16-byte code chunks per row
  const int64_t total = (int64_t)P.rows * cpr;
  const uint8_t* sk = P.k + h * P.src_sh;
  const uint8_t* sv = P.v + h * P.src_sh;
  uint8_t* dk = P.dst_k[lab] + P.slot[h] * P.dst_slot_bytes[lab];
  uint8_t* dv = P.dst_v[lab] + P.slot[h] * P.dst_slot_bytes[lab];
  for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * NT) {
    const int t = (int)(idx / cpr);
    const int ch = (int)(idx - (int64_t)t * cpr);
    const int64_t drow = dest_row(P, lab, t);
    const u32x4 k0 = *(const u32x4*)(sk + t * P.src_st + 32 * ch);
    const u32x4 k1 = *(const u32x4*)(sk + t * P.src_st + 32 * ch + 16);
    const u32x4 v0 = *(const u32x4*)(sv + t * P.src_st + 32 * ch);
    const u32x4 v1 = *(const u32x4*)(sv + t * P.src_st + 32 * ch + 16);
    const u32x4 kq = {e4m3x4(k0[0], k0[1], P.inv_k), e4m3x4(k0[2], k0[3], P.inv_k),
                      e4m3x4(k1[0], k1[1], P.inv_k), e4m3x4(k1[2], k1[3], P.inv_k)};
    const u32x4 vq = {e4m3x4(v0[0], v0[1], P.inv_v), e4m3x4(v0[2], v0[3], P.inv_v),
                      e4m3x4(v1[0], v1[1], P.inv_v), e4m3x4(v1[2], v1[3], P.inv_v)};
    *(u32x4*)(dk + drow * P.dst_row_bytes + 16 * ch) = kq;
    *(u32x4*)(dv + drow * P.dst_row_bytes + 16 * ch) = vq;
  }
}

__global__ __launch_bounds__(NT) void fill_zero_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] = 0;
}

}  // namespace

hipError_t launch_append(const AppendPlan& plan, hipStream_t s) {
  const int64_t chunks = (int64_t)plan.rows * (plan.dst_row_bytes >> 4);
  int bx = (int)((chunks + NT * 4 - 1) / (NT * 4));
  if (bx < 1) bx = 1;
  if (bx > 4096) bx = 4096;
  if (plan.quant) hipLaunchKernelGGL(append_fp8_kernel, dim3(bx, plan.H), dim3(NT), 0, s, plan);
  else hipLaunchKernelGGL(append_kernel, dim3(bx, plan.H), dim3(NT), 0, s, plan);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int bx = (int)((n + NT - 1) / NT);
  if (bx > 1024) bx = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(bx), dim3(NT), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace hc
