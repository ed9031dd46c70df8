// Classifier reductions (HeadCast review page, "What carries the argument"
// and the free-parameter ledger; the paper's Sec. 4.2 Eq. 2-5 as the review
// describes them).
//   merge_ranges_kernel  the Sink and Dummy proxies attend over the window's
//                   first and last block, which the full output covers too:
//                   the attention kernel computes the first block, the
//                   middle blocks and the last block once each (unnormalised,
//                   with their softmax states), and this kernel forms the
//                   full output (all three merged) and the two proxies from
//                   them.
// Given each head's full-context output and its Sink, Dummy and Spatial proxy
// outputs:
//   cosines_kernel  one wave per (head, query): the three per-query cosines
//                   against the full output, and the squared distance between
//                   the full and Spatial outputs (for the MSE);
//   reduce_kernel   one work group per head: mean cosine per proxy, the exact
//                   p-th percentile of the Spatial cosines (order statistics
//                   by radix selection, linear interpolation at rank
//                   p/100*(Nq-1)), S = P_p - gamma*MSE, and the routing rule.
#include "hc_internal.h"

namespace hc {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void cosines_kernel(const CosPlan P) {
  constexpr int PER = D / 64;
  const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= P.H * P.Nq) return;
  const int h = wave / P.Nq, i = wave - h * P.Nq;
  const int64_t plane = (int64_t)P.H * P.Nq * D;
  const float* f = P.o + ((int64_t)h * P.Nq + i) * D;
  float df_s = 0, df_d = 0, df_p = 0, nf = 0, ns = 0, nd = 0, np = 0, se = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane + 64 * e;
    const float a = f[c], s = f[plane + c], d = f[2 * plane + c], p = f[3 * plane + c];
    df_s = fmaf(a, s, df_s);
    df_d = fmaf(a, d, df_d);
    df_p = fmaf(a, p, df_p);
    nf = fmaf(a, a, nf);
    ns = fmaf(s, s, ns);
    nd = fmaf(d, d, nd);
    np = fmaf(p, p, np);
    se = fmaf(a - p, a - p, se);
  }
  df_s = wave_sum(df_s); df_d = wave_sum(df_d); df_p = wave_sum(df_p);
  nf = wave_sum(nf); ns = wave_sum(ns); nd = wave_sum(nd); np = wave_sum(np); se = wave_sum(se);
  if (lane == 0) {
    float* out = P.c + (int64_t)h * 4 * P.Nq + i;
    const float rf = sqrtf(nf);
    const float den_s = rf * sqrtf(ns), den_d = rf * sqrtf(nd), den_p = rf * sqrtf(np);
    out[0] = den_s > 0.f ? df_s / den_s : 0.f;
    out[P.Nq] = den_d > 0.f ? df_d / den_d : 0.f;
    out[2 * P.Nq] = den_p > 0.f ? df_p / den_p : 0.f;
    out[3 * P.Nq] = se;
  }
}

// One thread per (head, query, 4 channels).  Plane 0 holds the middle
// blocks' unnormalised output, plane 1 the first block's, plane 2 the last
// block's; states ml[r] = (running max of raw scores, sum of weights).
__global__ __launch_bounds__(256) void merge_ranges_kernel(const MergePlan P) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int g4 = P.D / 4;
  const int64_t rows = (int64_t)P.H * P.Nq;
  if (idx >= rows * g4) return;
  const int64_t row = idx / g4;
  const int c = (int)(idx - row * g4) * 4;
  const int64_t plane = rows * P.D;
  float4* o0 = (float4*)(P.o + row * P.D + c);
  float4* o1 = (float4*)(P.o + plane + row * P.D + c);
  float4* o2 = (float4*)(P.o + 2 * plane + row * P.D + c);
  const float2 s0 = P.ml[row];
  const float4 a = *o1;
  if (P.one_block) {   // the window's only block is first, last and all of it
    const float inv = 1.f / s0.y;
    const float4 r = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    *o0 = r;
    *o1 = r;
    *o2 = r;
    return;
  }
  const float2 s2 = P.ml[2 * rows + row];
  const float4 b = *o2;
  float M = fmaxf(s0.x, s2.x);
  float2 s1 = make_float2(-INFINITY, 0.f);
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  if (P.has_middle) {
    s1 = P.ml[rows + row];
    m = *o0;
    M = fmaxf(M, s1.x);
  }
  const float w0 = exp2f((s0.x - M) * P.scale_log2), w2 = exp2f((s2.x - M) * P.scale_log2);
  const float w1 = P.has_middle ? exp2f((s1.x - M) * P.scale_log2) : 0.f;
  const float inv = 1.f / (w0 * s0.y + w1 * s1.y + w2 * s2.y);
  *o0 = make_float4((w0 * a.x + w1 * m.x + w2 * b.x) * inv, (w0 * a.y + w1 * m.y + w2 * b.y) * inv,
                    (w0 * a.z + w1 * m.z + w2 * b.z) * inv, (w0 * a.w + w1 * m.w + w2 * b.w) * inv);
  const float i0 = 1.f / s0.y, i2 = 1.f / s2.y;
  *o1 = make_float4(a.x * i0, a.y * i0, a.z * i0, a.w * i0);
  *o2 = make_float4(b.x * i2, b.y * i2, b.z * i2, b.w * i2);
}

// float <-> order-preserving unsigned key
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int RT = 1024;

// k-th smallest (0-based) of x[0..n): four 8-bit radix passes over the keys.
__device__ float select_kth(const float* x, int n, int k, int* hist, uint32_t* s_prefix, int* s_k) {
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += RT) hist[b] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += RT) {
      const uint32_t key = fkey(x[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0;
      for (int b = 0; b < 256; ++b) {
        if (cum + hist[b] > k) {
          *s_prefix = prefix | ((uint32_t)b << shift);
          *s_k = k - cum;
          break;
        }
        cum += hist[b];
      }
    }
    __syncthreads();
    prefix = *s_prefix;
    k = *s_k;
    mask |= 255u << shift;
    __syncthreads();
  }
  return fkey_inv(prefix);
}

__global__ __launch_bounds__(RT) void reduce_kernel(const ReducePlan P) {
  __shared__ double red[4][RT / 64];
  __shared__ int hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_k;
  const int h = blockIdx.x;
  const float* c = P.c + (int64_t)h * 4 * P.Nq;
  double acc[4] = {0, 0, 0, 0};
  for (int i = threadIdx.x; i < P.Nq; i += RT)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += (double)c[q * P.Nq + i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    double v = acc[q];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[q][wave] = v;
  }
  __syncthreads();

  const double pos = (double)P.percentile / 100.0 * (double)(P.Nq - 1);
  int lo = (int)floor(pos);
  if (lo < 0) lo = 0;
  if (lo > P.Nq - 1) lo = P.Nq - 1;
  const int hi = min(lo + 1, P.Nq - 1);
  const float x_lo = select_kth(c + 2 * P.Nq, P.Nq, lo, hist, &s_prefix, &s_k);
  const float x_hi = select_kth(c + 2 * P.Nq, P.Nq, hi, hist, &s_prefix, &s_k);

  if (threadIdx.x == 0) {
    double sum[4] = {0, 0, 0, 0};
    for (int w = 0; w < RT / 64; ++w)
      for (int q = 0; q < 4; ++q) sum[q] += red[q][w];
    const double C_sink = sum[0] / P.Nq, C_dummy = sum[1] / P.Nq, C_sp = sum[2] / P.Nq;
    const double mse = sum[3] / ((double)P.Nq * P.D);
    const double pct = (double)x_lo + ((double)x_hi - (double)x_lo) * (pos - lo);
    const double score = pct - (double)P.gamma * mse;
    const bool ok_s = C_sink >= (double)P.theta_sink;
    const bool ok_d = C_dummy >= (double)P.theta_dummy;
    const bool ok_p = C_sp >= (double)P.theta_spatial && score >= (double)P.theta_score;
    int label = HC_GLOBAL;
    if (P.rule == 1) {
      label = ok_s ? HC_SINK : ok_d ? HC_DUMMY : ok_p ? HC_SPATIAL : HC_GLOBAL;
    } else {
      double best = -1e300;
      if (ok_s) { label = HC_SINK; best = C_sink; }
      if (ok_d && (label == HC_GLOBAL || C_dummy > best)) { label = HC_DUMMY; best = C_dummy; }
      if (ok_p && (label == HC_GLOBAL || C_sp > best)) { label = HC_SPATIAL; best = C_sp; }
    }
    P.labels[h] = (int8_t)label;
    P.diag[4 * h + 0] = (float)C_sink;
    P.diag[4 * h + 1] = (float)C_dummy;
    P.diag[4 * h + 2] = (float)C_sp;
    P.diag[4 * h + 3] = (float)score;
  }
}

}  // namespace

hipError_t launch_merge_ranges(const MergePlan& plan, hipStream_t s) {
  const int64_t n = (int64_t)plan.H * plan.Nq * (plan.D / 4);
  hipLaunchKernelGGL(merge_ranges_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, plan);
  return hipGetLastError();
}

hipError_t launch_cosines(const CosPlan& plan, hipStream_t s) {
  const int64_t waves = (int64_t)plan.H * plan.Nq;
  const int blocks = (int)((waves + 3) / 4);
  if (plan.D == 128) hipLaunchKernelGGL(cosines_kernel<128>, dim3(blocks), dim3(256), 0, s, plan);
  else hipLaunchKernelGGL(cosines_kernel<64>, dim3(blocks), dim3(256), 0, s, plan);
  return hipGetLastError();
}

hipError_t launch_classify_reduce(const ReducePlan& plan, hipStream_t s) {
  hipLaunchKernelGGL(reduce_kernel, dim3(plan.H), dim3(RT), 0, s, plan);
  return hipGetLastError();
}

}  // namespace hc
