// Flash-style head-routed attention on gfx950 matrix cores (bf16 in, fp32
// accumulate).  One kernel serves every pathway: the Global, Sink and Dummy
// pathways are exact softmax attention over a contiguous key range of the
// head's buffer, the Spatial pathway is exact attention over the keys of the
// query's latent cell in every cached frame (HeadCast review page, "What
// carries the argument" and Fig. 3: per-head pathways, non-overlapping grid
// cells).  Each work group owns 128 queries (4 waves x 32) and streams the
// key set in 64-key tiles through LDS with online softmax.
//
// Per wave and key tile:
//   S^T (64 keys x 32 queries) = K_tile . Q^T      4 x v_mfma_f32_32x32x16_bf16 per 32 keys
//   O^T (D x 32)             += V_tile^T . P^T     D/32 x 4 MFMAs
// Computing S transposed puts one query per lane (32 scores per lane, the
// other 32 of the tile in lane^32), so the row max needs one cross-lane
// exchange and the rescale of O is a per-lane scalar.  V is transposed while
// being staged into LDS, with bits 2 and 3 of the key index swapped so that
// every MFMA operand read is one 16-byte LDS load.
#include "hc_internal.h"

namespace hc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;  // threads per work group

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int RPP = NT / CPR;         // K rows loaded per pass
  static constexpr int KPASS = KTILE / RPP;    // K load passes per thread
  static constexpr int KS = D * 2 + 16;        // LDS bytes per K row (padded)
  static constexpr int VS = KTILE * 2 + 16;    // LDS bytes per V^T row (padded)
  static constexpr int KB = KTILE * KS;
  static constexpr int VB = D * VS;
  static constexpr int BUF = KB + VB;
  static constexpr int VTASKS = (KTILE / 4) * CPR;  // (4 keys x 8 channels) tasks
};

// Position of key k (0..63) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vpos(int k) {
  return (k & ~12) | ((k >> 1) & 4) | ((k << 1) & 8);
}

struct CellInfo {
  int base;    // y0*grid_w + x0
  int size;    // |c|
  int width;   // cell width (x extent)
  int off;     // sum of |c'| over cells c' < c
};

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

// Values of lanes l and l^32 (in either order), via v_permlane32_swap.
struct Pair {
  float a, b;
};
__device__ __forceinline__ Pair halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Pair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Lazy rescaling: the running max is only raised when a tile's max exceeds it
// by more than 2^8 in probability, so exp2 arguments stay <= 8 and the O
// accumulator is rescaled on a few early tiles only.
constexpr float kLazyLog2 = 8.0f;

template <int D, bool OUT_F32, bool GATHER>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(const AttnPlan P) {
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::BUF];
  __shared__ int s_last;

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
  const uint16_t* __restrict__ Kb = (const uint16_t*)C.k + slot * C.kv_sh;
  const uint16_t* __restrict__ Vb = (const uint16_t*)C.v + slot * C.kv_sh;
  const uint16_t* __restrict__ Qb = (const uint16_t*)P.q + qh * P.q_sh;

  // ---- what this unit covers --------------------------------------------
  int q0, qn, k0, kn, split = 0, tile = 0;
  CellInfo cell = {0, 0, 1, 0};
  const bool ranged = (C.kind == KIND_RANGED);
  if (ranged) {
    split = j / P.q_tiles;
    tile = j - split * P.q_tiles;
    q0 = tile * QTILE;
    qn = min(QTILE, P.Nq - q0);
    k0 = C.kv_first + split * C.keys_per_split;
    kn = min(C.keys_per_split, C.kv_count - split * C.keys_per_split);
  } else {
    const int c = j / P.cell_subtiles;
    const int st = j - c * P.cell_subtiles;
    cell = cell_info(P, c);
    q0 = st * QTILE;
    const int qall = P.B * cell.size;
    if (q0 >= qall) return;  // empty sub-tile of a small border cell
    qn = min(QTILE, qall - q0);
    kn = C.kv_count * cell.size;          // frames present x |c|
    k0 = (C.kind == KIND_CELL_MAJOR) ? P.W * cell.off : 0;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- this lane's query row ---------------------------------------------
  const int qlocal = wave * 32 + l32;
  const bool qvalid = qlocal < qn;
  const bool wave_active = wave * 32 < qn;
  int qtok = 0;
  if (qvalid) qtok = ranged ? (q0 + qlocal) : cell_token(P, cell, q0 + qlocal);

  bf16x8 qb[D / 16];
  {
    const uint16_t* qrow = Qb + (int64_t)qtok * P.q_st + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid) w = *(const u32x4*)(qrow + 16 * s);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- staging assignments -------------------------------------------------
  const int kr0 = tid / TL::CPR, kch = tid % TL::CPR;      // K: rows kr0 + RPP*i, chunk kch
  const int vo = tid / 16, va = tid % 16;                   // V: channels 8*vo.., keys 4*va..
  const bool vtask = tid < TL::VTASKS;

  // Contiguous key rows: a uniform (scalar) tile base plus a per-thread
  // 32-bit byte offset; only the ragged last tile checks rows.
  const int64_t rowb = C.kv_st * 2;                       // bytes per key row
  const uint32_t vko = (uint32_t)(kr0 * rowb + 16 * kch);
  const uint32_t vvo = (uint32_t)(4 * va * rowb + 16 * vo);
  const char* __restrict__ Kc = (const char*)Kb;
  const char* __restrict__ Vc = (const char*)Vb;

  u32x4 kreg[TL::KPASS];
  u32x4 vreg[4];
  auto load_tile = [&](int kb) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    if constexpr (!GATHER) {
      const char* kt = Kc + (int64_t)(k0 + kb) * rowb;
      const char* vt = Vc + (int64_t)(k0 + kb) * rowb;
      if (kb + KTILE <= kn) {
#pragma unroll
        for (int i = 0; i < TL::KPASS; ++i) kreg[i] = *(const u32x4*)(kt + i * TL::RPP * rowb + vko);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vreg[r] = (TL::VTASKS == NT || vtask) ? *(const u32x4*)(vt + r * rowb + vvo) : z;
      } else {
#pragma unroll
        for (int i = 0; i < TL::KPASS; ++i)
          kreg[i] = (kb + kr0 + TL::RPP * i < kn) ? *(const u32x4*)(kt + i * TL::RPP * rowb + vko) : z;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vreg[r] = (vtask && kb + 4 * va + r < kn) ? *(const u32x4*)(vt + r * rowb + vvo) : z;
      }
    } else {
#pragma unroll
      for (int i = 0; i < TL::KPASS; ++i) {
        const int kk = kb + kr0 + TL::RPP * i;
        kreg[i] = z;
        if (kk < kn) kreg[i] = *(const u32x4*)(Kb + (int64_t)cell_token(P, cell, kk) * C.kv_st + 8 * kch);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kb + 4 * va + r;
        vreg[r] = z;
        if (vtask && kk < kn) vreg[r] = *(const u32x4*)(Vb + (int64_t)cell_token(P, cell, kk) * C.kv_st + 8 * vo);
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* Ks = smem + buf * TL::BUF;
    uint8_t* Vt = Ks + TL::KB;
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i)
      *(u32x4*)(Ks + (kr0 + TL::RPP * i) * TL::KS + 16 * kch) = kreg[i];
    if (vtask) {
      const int pos = vpos(4 * va) * 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t x0 = vreg[0][w], x1 = vreg[1][w], x2 = vreg[2][w], x3 = vreg[3][w];
        u32x2 pk;
        if (e & 1) {
          pk.x = (x0 >> 16) | (x1 & 0xffff0000u);
          pk.y = (x2 >> 16) | (x3 & 0xffff0000u);
        } else {
          pk.x = (x0 & 0xffffu) | (x1 << 16);
          pk.y = (x2 & 0xffffu) | (x3 << 16);
        }
        *(u32x2*)(Vt + (8 * vo + e) * TL::VS + pos) = pk;
      }
    }
  };

  // ---- main loop -------------------------------------------------------------
  const float c2 = P.scale_log2;
  float m_run = -INFINITY;   // running max of raw scores for this lane's query
  float l_run = 0.f;         // running sum over this lane's half of the keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};

  const int ntiles = (kn + KTILE - 1) / KTILE;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) load_tile((it + 1) * KTILE);

    if (wave_active) {
      const uint8_t* Ks = smem + buf * TL::BUF;
      const uint8_t* Vt = Ks + TL::KB;
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 a0 = *(const bf16x8*)(Ks + l32 * TL::KS + (16 * s + 8 * hi) * 2);
        const bf16x8 a1 = *(const bf16x8*)(Ks + (32 + l32) * TL::KS + (16 * s + 8 * hi) * 2);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[s], s1, 0, 0, 0);
      }
      const int kb = it * KTILE;
      if (kb + KTILE > kn) {   // ragged last tile: keys past the set get -inf
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int key = 8 * (jj >> 2) + 4 * hi + (jj & 3);
          if (kb + key >= kn) s0[jj] = -INFINITY;
          if (kb + 32 + key >= kn) s1[jj] = -INFINITY;
        }
      }
      float mx = s0[0];
#pragma unroll
      for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, s0[jj]);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s1[jj]);
      {
        const Pair pr = halves(mx);
        mx = fmaxf(pr.a, pr.b);
      }
      const bool grow = mx * c2 > fmaf(m_run, c2, kLazyLog2);
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform
        const float m_new = grow ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
        m_run = m_new;
      }
      const float mc = m_run * c2;
      float psum = 0.f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        s0[jj] = __builtin_amdgcn_exp2f(fmaf(s0[jj], c2, -mc));
        s1[jj] = __builtin_amdgcn_exp2f(fmaf(s1[jj], c2, -mc));
        psum += s0[jj] + s1[jj];
      }
      l_run += psum;

      bf16x8 pb[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)s0[e];
        pb[1][e] = (__bf16)s0[8 + e];
        pb[2][e] = (__bf16)s1[e];
        pb[3][e] = (__bf16)s1[8 + e];
      }
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = *(const bf16x8*)(Vt + (32 * t + l32) * TL::VS + (16 * kk + 8 * hi) * 2);
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], oacc[t], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  float l_tot;
  {
    const Pair pr = halves(l_run);
    l_tot = pr.a + pr.b;
  }
  const int splits = ranged ? C.splits : 1;

  if (splits > 1) {
    // Write this split's unnormalised partial; the last split to arrive merges.
    const int id = slot * P.q_tiles + tile;
    const int n_ids = C.n_heads * P.q_tiles;
    float* po = C.part + ((int64_t)id * splits + split) * QTILE * D;
    float* pml = C.part + (int64_t)n_ids * splits * QTILE * D + ((int64_t)id * splits + split) * QTILE * 2;
    if (wave_active) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w4 = {oacc[t][4 * g], oacc[t][4 * g + 1], oacc[t][4 * g + 2], oacc[t][4 * g + 3]};
          *(f32x4*)(po + qlocal * D + 32 * t + 8 * g + 4 * hi) = w4;
        }
      if (hi == 0) {
        pml[2 * qlocal] = m_run;
        pml[2 * qlocal + 1] = l_tot;
      }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int old = atomicAdd(C.counters + id, 1);
      s_last = (old == splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (!qvalid) return;
    // merge all splits for this lane's query (its half of the channels)
    const float* pml0 = C.part + (int64_t)n_ids * splits * QTILE * D + (int64_t)id * splits * QTILE * 2;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, pml0[s * QTILE * 2 + 2 * qlocal]);
    float L = 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
    for (int s = 0; s < splits; ++s) {
      const float ms = pml0[s * QTILE * 2 + 2 * qlocal];
      const float ls = pml0[s * QTILE * 2 + 2 * qlocal + 1];
      const float w = __builtin_amdgcn_exp2f((ms - M) * c2);
      L = fmaf(w, ls, L);
      const float* ps = C.part + ((int64_t)id * splits + s) * QTILE * D + qlocal * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = *(const f32x4*)(ps + 32 * t + 8 * g + 4 * hi);
          oacc[t][4 * g] = fmaf(w, x[0], oacc[t][4 * g]);
          oacc[t][4 * g + 1] = fmaf(w, x[1], oacc[t][4 * g + 1]);
          oacc[t][4 * g + 2] = fmaf(w, x[2], oacc[t][4 * g + 2]);
          oacc[t][4 * g + 3] = fmaf(w, x[3], oacc[t][4 * g + 3]);
        }
    }
    if (tid == 0) C.counters[id] = 0;   // ready for the next call
    const float inv = 1.f / L;
    uint8_t* orow = (uint8_t*)C.o;
    const int64_t obase = (int64_t)qh * C.o_sh + (int64_t)qtok * C.o_st;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * t + 8 * g + 4 * hi;
        if (OUT_F32) {
          f32x4 w4 = {oacc[t][4 * g] * inv, oacc[t][4 * g + 1] * inv, oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv};
          *(f32x4*)((float*)orow + obase + ch) = w4;
        } else {
          bf16x4 b = {(__bf16)(oacc[t][4 * g] * inv), (__bf16)(oacc[t][4 * g + 1] * inv),
                      (__bf16)(oacc[t][4 * g + 2] * inv), (__bf16)(oacc[t][4 * g + 3] * inv)};
          *(u32x2*)((uint16_t*)orow + obase + ch) = __builtin_bit_cast(u32x2, b);
        }
      }
    return;
  }

  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  const int64_t obase = (int64_t)qh * C.o_sh + (int64_t)qtok * C.o_st;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ch = 32 * t + 8 * g + 4 * hi;
      if (OUT_F32) {
        f32x4 w4 = {oacc[t][4 * g] * inv, oacc[t][4 * g + 1] * inv, oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv};
        *(f32x4*)((float*)C.o + obase + ch) = w4;
      } else {
        bf16x4 b = {(__bf16)(oacc[t][4 * g] * inv), (__bf16)(oacc[t][4 * g + 1] * inv),
                    (__bf16)(oacc[t][4 * g + 2] * inv), (__bf16)(oacc[t][4 * g + 3] * inv)};
        *(u32x2*)((uint16_t*)C.o + obase + ch) = __builtin_bit_cast(u32x2, b);
      }
    }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnPlan& plan, int head_dim, hipStream_t s) {
  if (plan.total_units <= 0) return hipSuccess;
  const bool f32 = plan.cat[0].out_f32 != 0;
  const bool gather = plan.cat[0].kind == KIND_CELL_GATHER;
  for (int c = 1; c < plan.n_cats; ++c)
    if ((plan.cat[c].kind == KIND_CELL_GATHER) != gather) return hipErrorInvalidValue;  // one mode per launch
  dim3 grid(plan.total_units), block(NT);
#define HC_LAUNCH(DD, F, G) hipLaunchKernelGGL((attn_bf16_kernel<DD, F, G>), grid, block, 0, s, plan)
  if (head_dim == 128) {
    if (gather) { if (f32) HC_LAUNCH(128, true, true); else HC_LAUNCH(128, false, true); }
    else { if (f32) HC_LAUNCH(128, true, false); else HC_LAUNCH(128, false, false); }
  } else {
    if (gather) { if (f32) HC_LAUNCH(64, true, true); else HC_LAUNCH(64, false, true); }
    else { if (f32) HC_LAUNCH(64, true, false); else HC_LAUNCH(64, false, false); }
  }
#undef HC_LAUNCH
  return hipGetLastError();
}

}  // namespace hc
