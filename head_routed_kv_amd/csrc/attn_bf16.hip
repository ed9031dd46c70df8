// Flash-style head-routed attention on gfx950 matrix cores (bf16 in, fp32
// accumulate).  One kernel serves every pathway: the Global, Sink and Dummy
// pathways are exact softmax attention over a contiguous key range of the
// head's buffer, the Spatial pathway is exact attention over the keys of the
// query's latent cell in every cached frame (HeadCast review page, "What
// carries the argument" and Fig. 3: per-head pathways, non-overlapping grid
// cells).
//
// A work group is NW waves; each wave owns QB blocks of 32 queries, so a work
// group owns 32*QB*NW queries and streams the key set in 64-key tiles through
// a ring of four LDS buffers with online softmax, software-pipelined so that
// the scores of the next tile are computed alongside this tile's softmax.
// Per wave and key tile:
//   S^T (64 keys x 32 queries) = K_tile . Q^T      per query block: 2 x D/16 v_mfma_f32_32x32x16_bf16
//   O^T (D x 32)             += V_tile^T . P^T     per query block: D/32 x 4 MFMAs
// Computing S transposed puts one query per lane (32 scores per lane, the
// other 32 of the tile in lane^32), so the row max needs one
// v_permlane32_swap and rescaling O is a per-lane scalar.
//
// K and V tiles go from global memory straight into LDS (global_load_lds,
// 16 bytes per lane; lane l of a load lands at byte 16*l of its 1 KiB slot),
// so staging costs no registers and no LDS write instructions, and the next
// tile's loads run behind the current tile's math.  Rows keep their natural
// [key][channel] layout; 16-byte chunks are XOR-swizzled per row (chunk c of
// row r sits at slot c ^ sw(r)) so that both read patterns are free of bank
// conflicts.  The K operand of S^T is one 16-byte read per lane.  The V^T
// operand of O^T is two ds_read_b64_tr_b16 per lane: that instruction
// transposes 4x4 blocks of 16-bit values across each group of 16 lanes (lane
// i receives element i&3 of the 8-byte chunks addressed by lanes (i>>2)+4e,
// e = 0..3), so lanes addressing 4 consecutive keys x 16 channels receive 4
// keys of one channel each, which is the MFMA operand layout.
//
// A cache that stores K and V as fp8 (E4M3) codes instantiates KV8: tiles are
// staged as fp8 by the same direct loads and widened once per work group into
// a three-deep bf16 ring, after which the arithmetic is the bf16 path's.
#include "hc_internal.h"

namespace hc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = kBf16Waves;   // waves per work group
constexpr int NT = 64 * NW;      // threads per work group

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int ROWB = D * 2;           // LDS bytes per key row (unpadded)
  static constexpr int RPI = 64 / CPR;         // rows per 1 KiB direct load (64 lanes x 16 B)
  static constexpr int KB = KTILE * ROWB;      // K tile bytes
  static constexpr int BUF = 2 * KB;           // K tile + V tile
  static constexpr int LPW = KB / 1024 / NW;   // direct loads per wave per tile, for K (same for V)
  static_assert(LPW >= 1, "tile too small");
};

typedef uint8_t __attribute__((address_space(3))) lds_u8;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at LDS byte m0 + 16*l (m0 wave-uniform).  Written as one asm statement
// with no output registers (the data goes to LDS), so the compiler's memory
// counter bookkeeping does not see it: the kernel waits for these loads
// itself (s_waitcnt vmcnt before each tile barrier) and otherwise the compiler
// would wait for the newest tile's loads before every LDS read.  `base` is a
// wave-uniform tile address, `voff` this lane's byte offset from it.
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t voff, uint32_t lds_byte) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_byte)
      : "memory", "m0");
}
// The same for a per-lane 64-bit address (gathered rows).
__device__ __forceinline__ void lds_dma16_addr(const char* addr, uint32_t lds_byte) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(addr), "s"(lds_byte)
      : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Chunk swizzles.  K reads: 16 lanes read one chunk of 16 consecutive rows, so
// row r's chunks are XORed with r mod CPR.  V reads (transposing): 32 lanes
// read the 4 aligned chunks {c0..c0+3} of 4 consecutive rows, so the 4 rows
// must map that group onto disjoint slot groups: XOR with 4*(r&3) at 16 chunks
// per row; at 8 chunks per row (two rows per bank sweep) with 4*((r>>1)&1).
template <int D>
__device__ __forceinline__ int swz_k(int r) { return r & (Tile<D>::CPR - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Initial running max: finite, so that a tile whose keys are all masked for a
// query (box proxy) gives exp2(-inf) = 0 instead of exp2(-inf + inf) = NaN.
constexpr float kNoMax = -1e30f;

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

// Device-coherent 8-byte store / load (relaxed, agent scope: sc1), used for
// the split partials that another XCD's work group merges.
__device__ __forceinline__ void store_coherent(uint64_t* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void load_coherent(const uint64_t* p, float& a, float& b) {
  const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  a = __uint_as_float((uint32_t)v);
  b = __uint_as_float((uint32_t)(v >> 32));
}

template <bool OUT_F32>
__device__ __forceinline__ void store_row4(void* base, int64_t off, f32x4 v) {
  if constexpr (OUT_F32) {
    *(f32x4*)((float*)base + off) = v;
  } else {
    bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(u32x2*)((uint16_t*)base + off) = __builtin_bit_cast(u32x2, b);
  }
}

// One work unit: relative unit `rel` of category `ci` (ranged categories:
// after the XCD run mapping).  Every thread of the work group calls it with
// the same arguments and returns from it together.
template <int D, int QB, bool OUT_F32, bool GATHER, bool KV8>
__device__ __forceinline__ void attn_unit(const AttnPlan& P, const int ci, int rel, const int tid) {
  using TL = Tile<D>;
  constexpr int QT = 32 * QB * NW;   // queries per work group
  static_assert(!KV8 || (QB == 1 && !GATHER), "fp8 K/V: ranged and cell-major kinds");
  // The bf16 ring buffers (K tile then V tile each): four, tile j in buffer
  // j mod 4; with fp8 K/V three, tile j in buffer j mod 3, fed from a ring of
  // three fp8 staging buffers.  Separate objects rather than one indexed
  // array, so every LDS address in the unrolled loop is a constant plus a
  // per-lane offset.
  constexpr int KB8 = KTILE * D;   // fp8 K (or V) tile bytes
  __shared__ __attribute__((aligned(16))) uint8_t smem0[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t smem2[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t smem3[KV8 ? 16 : TL::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t stg0[KV8 ? 2 * KB8 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t stg1[KV8 ? 2 * KB8 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t stg2[KV8 ? 2 * KB8 : 16];
  __shared__ int s_last;
  __shared__ float s_ml[NW][2][64];   // small units: each wave's (m, l) for the merge

  const AttnCat& C = P.cat[ci];
  int slot, j;
  if (C.kind == KIND_RANGED || C.kind == KIND_BOX_GATHER) {
    slot = rel / C.units_per_head;
    j = rel - slot * C.units_per_head;
  } else {
    // Spatial units go sub-tile by sub-tile over all heads and cells, so every
    // cell's first (full) query sub-tile starts before any short remainder.
    const int n_cells = C.units_per_head / P.cell_subtiles;
    const int per_st = C.n_heads * n_cells;
    const int st = rel / per_st, rem = rel - st * per_st;
    slot = rem / n_cells;
    j = (rem - slot * n_cells) * P.cell_subtiles + st;
  }
  const int qh = P.head_of[ci][slot];
  constexpr int KVE = KV8 ? 1 : 2;   // bytes per cached K/V element
  const char* __restrict__ Kb = (const char*)C.k + slot * C.kv_sh * KVE;
  const char* __restrict__ Vb = (const char*)C.v + slot * C.kv_sh * KVE;
  const uint16_t* __restrict__ Qb = (const uint16_t*)P.q + qh * P.q_sh;

  // ---- what this unit covers --------------------------------------------
  int q0, qn, k0, kn, split = 0, tile = 0;
  CellInfo cell = {0, 0, 1, 0};
  BoxInfo box = {0, 0, 0};
  const bool ranged = (C.kind == KIND_RANGED);
  const bool is_box = GATHER && C.kind == KIND_BOX_GATHER;
  if (ranged) {
    split = j / P.q_tiles;
    tile = j - split * P.q_tiles;
    q0 = tile * QT;
    qn = min(QT, P.Nq - q0);
    k0 = C.kv_first + split * C.keys_per_split;
    kn = min(C.keys_per_split, C.kv_count - split * C.keys_per_split);
  } else if (is_box) {
    box = box_info(P, j);
    q0 = 0;
    qn = QT;   // query validity is decided per lane from the patch
    kn = C.kv_count * (P.box_rows + 2 * P.box_r) * 32;
    k0 = 0;
  } else {
    const int c = j / P.cell_subtiles;
    const int st = j - c * P.cell_subtiles;
    cell = cell_info(P, c);
    q0 = st * QT;
    const int qall = P.B * cell.size;
    if (q0 >= qall) return;  // empty sub-tile of a small border cell
    qn = min(QT, qall - q0);
    kn = C.kv_count * cell.size;          // frames present x |c|
    k0 = (C.kind == KIND_CELL_MAJOR) ? P.W * cell.off : 0;
  }

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Units with at most 64 queries (the ragged last q tile of a head, the short
  // remainder sub-tile of a cell) would leave six of eight waves idle.  They
  // run their own schedule instead, splitting the key tiles among the waves
  // and merging the parts through LDS: bf16 K/V, all eight waves (query block
  // w & 1, key phase w >> 1, every fourth tile); fp8 K/V, waves 0-3 (query
  // block w & 1, every other tile).
  const bool small = QB == 1 && !is_box && qn <= 64;
  const bool small4 = small && !KV8;

  // ---- this lane's query rows (one per query block) -----------------------
  int qlocal[QB], qtok[QB];
  bool qvalid[QB];
  bf16x8 qb[QB][D / 16];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    qlocal[b] = small ? 32 * (wave & 1) + l32 : wave * 32 * QB + 32 * b + l32;
    qtok[b] = 0;
    if (is_box) {   // patch row wave*QB+b, column l32
      const int y = box.py0 + wave * QB + b, x = box.px0 + l32;
      qvalid[b] = l32 < P.box_cols_q && y < P.grid_h && x < P.grid_w;
      if (qvalid[b]) qtok[b] = box.fb * P.T + y * P.grid_w + x;
    } else {
      qvalid[b] = qlocal[b] < qn && (!small || small4 || wave < 4);
      if (qvalid[b]) qtok[b] = ranged ? (q0 + qlocal[b]) : cell_token(P, cell, q0 + qlocal[b]);
    }
    const uint16_t* qrow = Qb + (int64_t)qtok[b] * P.q_st + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid[b]) w = *(const u32x4*)(qrow + 16 * s);
      qb[b][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  bool wave_active = is_box ? (box.py0 + wave * QB < P.grid_h)
                   : small4 ? (32 * (wave & 1) < qn)
                   : small ? (wave < 4 && 32 * (wave & 1) < qn) : (wave * 32 * QB < qn);
  // Box proxy: bit rx of box_cm says whether this lane's query may see box
  // column rx (within r columns of it, and on the grid), shifted so that bit
  // 8a+e stands for column 8a+4*hi+e, the keys this lane's score registers hold.
  uint32_t box_cm = 0;
  if (is_box) {
    uint32_t m = ((1u << (2 * P.box_r + 1)) - 1u) << l32;
    const int rx_min = P.box_r - box.px0;                  // first on-grid column
    const int rx_max = P.grid_w - 1 - box.px0 + P.box_r;   // last on-grid column (>= r)
    if (rx_min > 0) m &= ~((1u << rx_min) - 1u);
    if (rx_max < 31) m &= (2u << rx_max) - 1u;
    box_cm = m >> (4 * hi);
  }
  // Q has landed (vmcnt(0); expcnt and lgkmcnt untouched).  Said once here, in
  // the form the compiler's wait bookkeeping understands, so the tile loop
  // never waits for Q again.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- staging ---------------------------------------------------------------
  // Tile `it` covers keys [it*KTILE, min((it+1)*KTILE, kn)).  Its rows are
  // loaded from lb(it) = min(it*KTILE, kn - KTILE): the ragged last tile is
  // shifted back so every row it loads exists, and the keys it repeats are
  // masked out of the softmax.  A key set shorter than one tile loads row
  // min(r, kn-1) into slot r; the copies are masked too, and their values are
  // finite, so they add exactly zero.  No load ever leaves the key set.
  const bool short_set = kn < KTILE;
  const int rows_avail = short_set ? kn : KTILE;
  auto tile_base = [&](int it) { return short_set ? 0 : min(it * KTILE, kn - KTILE); };
  const int64_t rowb = C.kv_st * KVE;               // bytes per key row in global memory
  // Direct load i of this wave fills rows [RPI*(NW*i+wave), +RPI) of a tile; this
  // lane writes slot (lane % CPR) of row (RPI*(4*i+wave) + lane / CPR).
  int lrow[TL::LPW];
  uint32_t kofs[TL::LPW], vofs[TL::LPW];
#pragma unroll
  for (int i = 0; i < TL::LPW; ++i) {
    const int r = TL::RPI * (NW * i + wave) + lane / TL::CPR;
    const int slot_c = lane % TL::CPR;
    lrow[i] = min(r, rows_avail - 1);
    kofs[i] = (uint32_t)(lrow[i] * rowb + 16 * (slot_c ^ swz_k<D>(r)));
    vofs[i] = (uint32_t)(lrow[i] * rowb + 16 * (slot_c ^ swz_v<D>(r)));
  }
  const char* __restrict__ Kc = (const char*)Kb;
  const char* __restrict__ Vc = (const char*)Vb;
  auto load_tile = [&](int lb, uint8_t* dst) {
    const uint32_t kdst = lds_addr(dst), vdst = kdst + TL::KB;
    if constexpr (!GATHER) {
      const char* kt = Kc + (int64_t)(k0 + lb) * rowb;   // uniform tile base
      const char* vt = Vc + (int64_t)(k0 + lb) * rowb;
#pragma unroll
      for (int i = 0; i < TL::LPW; ++i) {
        lds_dma16(kt, kofs[i], kdst + 1024 * (NW * i + wave));
        lds_dma16(vt, vofs[i], vdst + 1024 * (NW * i + wave));
      }
    } else {
#pragma unroll
      for (int i = 0; i < TL::LPW; ++i) {
        const int r = TL::RPI * (NW * i + wave) + lane / TL::CPR;
        const int slot_c = lane % TL::CPR;
        const int tok = is_box ? box_token(P, box, lb + lrow[i]) : cell_token(P, cell, lb + lrow[i]);
        const int64_t row = (int64_t)tok * rowb;
        lds_dma16_addr(Kc + row + 16 * (slot_c ^ swz_k<D>(r)), kdst + 1024 * (NW * i + wave));
        lds_dma16_addr(Vc + row + 16 * (slot_c ^ swz_v<D>(r)), vdst + 1024 * (NW * i + wave));
      }
    }
  };
  // LDS address of the V^T operand half q (keys +0..3 or +8..11 of a 16-key
  // step) for d-tile t and k-step kk, relative to the V tile.
  const int vg = lane >> 4, vj = lane & 15;
  auto vt_addr = [&](int t, int kk, int q) {
    const int row = 16 * kk + 8 * q + 4 * (vg >> 1) + (vj >> 2);
    const int col = 32 * t + 16 * (vg & 1) + 4 * (vj & 3);
    return row * TL::ROWB + 16 * ((col >> 3) ^ swz_v<D>(row)) + 2 * (col & 7);
  };
  // fp8 K/V: lane p = 64*wave + lane moves 16-byte piece p of the K tile and
  // of the V tile (row p / (D/16), bytes 16*(p % (D/16)); one piece per
  // thread at d = 128) from global memory into a row-major staging buffer;
  // `widen` later writes the tile to bf16 in the ring buffer, at the swizzled
  // slots the bf16 loads would have used.
  const int p8 = 64 * wave + lane;
  const int r8 = p8 / (D / 16), c8 = p8 % (D / 16);
  const uint32_t ofs8 = (uint32_t)(min(r8, rows_avail - 1) * rowb + 16 * c8);
  // A staged fp8 tile is KB8 / 1 KiB direct loads for K and as many for V:
  // one each for every wave at d = 128, for waves 0-3 at d = 64.
  auto load8 = [&](int lb, uint8_t* stg) {
    if (KB8 >= 1024 * NW || wave < KB8 / 1024) {   // wave-uniform; always true at d = 128
      const char* kt = Kc + (int64_t)(k0 + lb) * rowb;   // uniform tile base
      const char* vt = Vc + (int64_t)(k0 + lb) * rowb;
      const uint32_t kd = lds_addr(stg) + 1024 * wave;
      lds_dma16(kt, ofs8, kd);
      lds_dma16(vt, ofs8, kd + KB8);
    }
  };
  // Widening: thread t writes bf16 chunks g = t and t + NT of the K tile and
  // of the V tile (row g / 16, slot g % 16 at d = 128), converting the eight
  // fp8 codes of the chunk the swizzle puts there.  Each 16 consecutive lanes
  // thus write one whole 256-byte row, and each 8 one contiguous 128 bytes,
  // the pattern LDS writes take without bank conflicts (a per-lane 32-byte
  // piece written as two 16-byte slots is not).  E4M3 values are exact in
  // bf16, so the rest of the kernel is unchanged.
  auto widen = [&](const uint8_t* stg, uint8_t* buf) {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv)
#pragma unroll
      for (int q = 0; q < TL::KB / 16 / NT; ++q) {
        const int g = q * NT + 64 * wave + lane;
        const int row = g / TL::CPR, slot = g % TL::CPR;
        const int chunk = slot ^ (kv == 0 ? swz_k<D>(row) : swz_v<D>(row));
        const u32x2 w = *(const u32x2*)(stg + kv * KB8 + row * D + 8 * chunk);
        bf16x8 h;
#pragma unroll
        for (int i = 0; i < 2; ++i) {   // bytes 4i..4i+3 -> elements 4i..4i+3 of the chunk
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, true);
          h[4 * i + 0] = lo[0];
          h[4 * i + 1] = lo[1];
          h[4 * i + 2] = hi[0];
          h[4 * i + 3] = hi[1];
        }
        *(bf16x8*)(buf + kv * TL::KB + row * TL::ROWB + 16 * slot) = h;
      }
  };

  // ---- main loop -------------------------------------------------------------
  const float c2 = P.scale_log2;
  float m_run[QB], l_run[QB];   // running max (raw scores) and this lane's half of the sum
  f32x16 oacc[QB][D / 32];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m_run[b] = kNoMax;
    l_run[b] = 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[b][t] = f32x16{};
  }

  const int ntiles = (kn + KTILE - 1) / KTILE;
  // Each wave issues 2*LPW loads per tile; waiting until at most that many are
  // in flight means every load but the newest tile's has landed in LDS.
  auto wait_all_but_newest = [&]() {
    if constexpr (2 * TL::LPW == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (2 * TL::LPW == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // Tile barrier.  The LDS buffers are only written by the loads above, and
  // every LDS read of a tile feeds MFMAs issued before the barrier, so a bare
  // s_barrier orders the ring; __syncthreads() would also wait for the newest
  // tile's loads and undo their lead.
  auto tile_barrier = [&]() {
    wait_all_but_newest();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Scores of key slots j < lo or j >= hi_end become -inf.  Score jj of half c
  // is key slot 32c + 8(jj/4) + 4hi + jj%4; compared against lane-relative
  // bounds, every slot offset is a constant.  The bounds are opaque to the
  // compiler, which would otherwise hoist the 32 lane masks of the loop-invariant
  // end bound out of the loop into (spilled) scalar registers.
  auto mask_keys = [&](f32x16 (&s)[2], const int lo, const int hi_end) {
    int lo_l = lo - 4 * hi, he_l = hi_end - 4 * hi;
    asm volatile("" : "+v"(lo_l), "+v"(he_l));   // keep the 32 compares in this branch
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int kc = 32 * c + 8 * (jj >> 2) + (jj & 3);
        if (kc < lo_l || kc >= he_l) s[c][jj] = -INFINITY;
      }
  };
  // S^T of one tile: sc[b][blk] (keys 32*blk.. x 32 queries of block b).
  auto scores = [&](const uint8_t* Ks, f32x16 (&out)[QB][2]) {
#pragma unroll
    for (int b = 0; b < QB; ++b) out[b][0] = out[b][1] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int c = 2 * s + hi;
      const bf16x8 a0 = *(const bf16x8*)(Ks + l32 * TL::ROWB + 16 * (c ^ swz_k<D>(l32)));
      const bf16x8 a1 = *(const bf16x8*)(Ks + (32 + l32) * TL::ROWB + 16 * (c ^ swz_k<D>(32 + l32)));
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        out[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[b][s], out[b][0], 0, 0, 0);
        out[b][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[b][s], out[b][1], 0, 0, 0);
      }
    }
  };

  // Software pipeline over key tiles, 4 LDS buffers (tile j lives in buffer
  // j mod 4).  Step `it` holds V of tile it and K of tile it+1 while tile it+2
  // is landing and tile it+3 is being loaded; it computes S of tile it+1 in
  // the same instruction stream as the softmax of tile it, so neither waits on
  // the other's results (on this chip vector work does not run under the
  // matrix core, so the gain is the removed dependency stall, not
  // concurrency).  Tiles past the end are clamped copies of the last one
  // (finite, unused).
  const bf16x8 ones8 = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                        (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  if (!small) {
  if constexpr (KV8) {
    load8(0, stg0);
    load8(tile_base(min(1, ntiles - 1)), stg1);
    load8(tile_base(min(2, ntiles - 1)), stg2);
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");   // this wave's pieces of tiles 0 and 1
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    widen(stg0, smem0);
    widen(stg1, smem1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // tile 2 staged; widened tiles written
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load8(tile_base(min(3, ntiles - 1)), stg0);   // every wave has read stg0
  } else {
    load_tile(0, smem0);
    load_tile(tile_base(min(1, ntiles - 1)), smem1);
    load_tile(tile_base(min(2, ntiles - 1)), smem2);
    tile_barrier();   // tiles 0 and 1 are in LDS
  }
  f32x16 sc[QB][2];
  scores(smem0, sc);
  // Row max of the tile in sc over both lanes of each query, computed one step
  // ahead (after the PV products, where it fills the vector unit) and redone
  // on the tiles that mask keys.
  auto row_max = [&](const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, s[0][jj]);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[1][jj]);
    const Pair pr = halves(mx);
    return fmaxf(pr.a, pr.b);
  };
  float tmax[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) tmax[b] = row_max(sc[b]);

  // One step: V of tile it and K of tile it+1 are in LDS.  `issue` starts the
  // loads of a later tile: active waves issue them between the PV MFMAs
  // (below), where the issue costs least; idle waves at once.  `after` runs
  // once the PV product is issued (with fp8 K/V: widening a staged tile).
  auto step = [&](const int it, const uint8_t* vbuf, const uint8_t* kbuf, auto issue, auto after)
      __attribute__((always_inline)) {
    if (wave_active) {
      // Keys tile `it` must not count: rows repeated from the previous tile
      // (shifted last tile, lb + j < it*KTILE) or past a short key set.
      const int lo = it * KTILE - tile_base(it);   // slots j < lo are repeats
      const int hi_end = short_set ? kn : KTILE;     // slots j >= hi_end are empty
      if (lo > 0 || hi_end < KTILE) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          mask_keys(sc[b], lo, hi_end);
          tmax[b] = row_max(sc[b]);
        }
      }
      if constexpr (GATHER) {
        if (is_box) {   // box proxy: only keys within r rows and r columns count
          const int rows = P.box_rows + 2 * P.box_r;
          uint32_t cm = box_cm;
          asm volatile("" : "+v"(cm));   // the 16 bit tests stay in this branch
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int ky = box.py0 - P.box_r + (2 * it + c) % rows;   // uniform
#pragma unroll
            for (int b = 0; b < QB; ++b) {
              const int qy = box.py0 + wave * QB + b;
              const bool row_ok = ky >= 0 && ky < P.grid_h && abs(ky - qy) <= P.box_r;
#pragma unroll
              for (int jj = 0; jj < 16; ++jj)
                if (!row_ok || !((cm >> (8 * (jj >> 2) + (jj & 3))) & 1u)) sc[b][c][jj] = -INFINITY;
            }
          }
#pragma unroll
          for (int b = 0; b < QB; ++b) tmax[b] = row_max(sc[b]);
        }
      }
      float mc[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const float mx = tmax[b];
        const bool grow = mx * c2 > fmaf(m_run[b], c2, kLazyLog2);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform
          const float m_new = grow ? mx : m_run[b];
          const float alpha = __builtin_amdgcn_exp2f((m_run[b] - m_new) * c2);
          l_run[b] *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) oacc[b][t] *= alpha;
          m_run[b] = m_new;
        }
        mc[b] = m_run[b] * c2;
      }
      // S of the next tile (matrix core) and P of this tile (vector unit):
      // independent, one basic block, interleaved by the scheduler.
      f32x16 sn[QB][2];
      scores(kbuf, sn);
      bf16x8 pb[QB][4];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          sc[b][0][jj] = __builtin_amdgcn_exp2f(fmaf(sc[b][0][jj], c2, -mc[b]));
          sc[b][1][jj] = __builtin_amdgcn_exp2f(fmaf(sc[b][1][jj], c2, -mc[b]));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[b][0][e] = (__bf16)sc[b][0][e];
          pb[b][1][e] = (__bf16)sc[b][0][8 + e];
          pb[b][2][e] = (__bf16)sc[b][1][e];
          pb[b][3][e] = (__bf16)sc[b][1][8 + e];
        }
        // row sum of the bf16 weights the PV product uses (2 per dot2)
        float psum = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 p2 = {pb[b][kk][2 * e], pb[b][kk][2 * e + 1]};
            const bf16x2 o2 = {ones8[0], ones8[1]};
            psum = __builtin_amdgcn_fdot2_f32_bf16(p2, o2, psum, false);
          }
        l_run[b] += psum;
      }
      // O^T += V^T P^T: k-steps outer, d-tiles inner, so consecutive MFMAs
      // feed different accumulators.
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk == 1) issue();
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3)))*)((lds_u8*)vbuf + TL::KB + vt_addr(t, kk, 0)));
          const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3)))*)((lds_u8*)vbuf + TL::KB + vt_addr(t, kk, 1)));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int b = 0; b < QB; ++b)
            oacc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[b][kk], oacc[b][t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        tmax[b] = row_max(sn[b]);
        sc[b][0] = sn[b][0], sc[b][1] = sn[b][1];
      }
      after();
    } else {
      issue();
      after();
    }
  };
  if constexpr (KV8) {
    // Step it widens tile it+2 (staged in stg[(it+2) mod 3]) into the bf16
    // buffer of tile it-1, whose last reads were in the previous step, and
    // stages tile it+4 into the buffer tile it+1 was widened from.  The
    // barrier waits for this wave's widening writes and for all staged tiles
    // but the newest, so tile it+3 is staged and tile it+2 widened when the
    // next step starts.
    auto step8 = [&](const int it, const uint8_t* vb, const uint8_t* kb, uint8_t* cb, const uint8_t* cs,
                     uint8_t* ls) __attribute__((always_inline)) {
      const int lb4 = tile_base(min(it + 4, ntiles - 1));
      step(it, vb, kb, [&]() { load8(lb4, ls); }, [&]() { widen(cs, cb); });
      asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    for (int it = 0; it < ntiles; it += 3) {
      step8(it, smem0, smem1, smem2, stg2, stg1);
      if (it + 1 < ntiles) step8(it + 1, smem1, smem2, smem0, stg0, stg2);
      if (it + 2 < ntiles) step8(it + 2, smem2, smem0, smem1, stg1, stg0);
    }
  } else {
    // Tile it+3 goes into the buffer tile it-1 left (all its reads were
    // before the last barrier).
    auto step4 = [&](const int it, const uint8_t* vb, const uint8_t* kb, uint8_t* lb)
        __attribute__((always_inline)) {
      const int lb3 = tile_base(min(it + 3, ntiles - 1));
      step(it, vb, kb, [&]() { load_tile(lb3, lb); }, []() {});
      tile_barrier();   // tile it+2 is in LDS (all waves)
    };
    for (int it = 0; it < ntiles; it += 4) {
      step4(it, smem0, smem1, smem3);
      if (it + 1 < ntiles) step4(it + 1, smem1, smem2, smem0);
      if (it + 2 < ntiles) step4(it + 2, smem2, smem3, smem1);
      if (it + 3 < ntiles) step4(it + 3, smem3, smem0, smem2);
    }
  }
  } else if constexpr (QB == 1 && !KV8) {
    // ---- small units: two query blocks x four key phases --------------------
    // Wave w takes query block w & 1 and the key tiles ph, ph + 4, ph + 8, ...
    // (ph = w >> 1).  The two waves of a phase stream their tiles through
    // their own LDS buffer (K then V) and load them themselves, eight of the
    // tile's sixteen 1 KiB pieces each (d = 128): K of round s+1 once both
    // have read K of round s, V of round s+1 once both have read V of round
    // s, so each load runs behind the other half of the round's math.  Three
    // barriers per round keep the pairs in step (every wave meets every
    // barrier; waves whose tile lies past the end skip only the math, and
    // load a clamped copy of the last tile).
    const int ph = wave >> 1, mem = wave & 1;
    uint8_t* const buf = ph == 0 ? smem0 : ph == 1 ? smem1 : ph == 2 ? smem2 : smem3;
    const int nrounds = (ntiles + 3) >> 2;
    constexpr int PPW = TL::KB / 1024 / 2;   // 1 KiB pieces of a K (or V) tile per wave of the pair
    auto wait_newest_part = [&]() {           // all loads but the newest PPW have landed
      if constexpr (PPW == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    };
    auto wait_all = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
    auto barrier = [&]() {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // Pieces j = 2i + mem of the K (kv = 0) or V (kv = 1) tile whose rows start
    // at key lb: piece j holds rows RPI*j .. RPI*j + RPI - 1.
    auto load_part = [&](const int lb, const int kv) {
      const uint32_t dst = lds_addr(buf) + kv * TL::KB;
      const char* base = kv ? Vc : Kc;
      // (gathered rows: not unrolled, which keeps the row arithmetic's
      // registers out of the pressure of the surrounding math)
#pragma unroll(GATHER ? 1 : PPW)
      for (int i = 0; i < PPW; ++i) {
        const int j = 2 * i + mem;
        const int r = TL::RPI * j + lane / TL::CPR;
        const int slot_c = lane % TL::CPR;
        const int lr = min(r, rows_avail - 1);
        const int sw = kv ? swz_v<D>(r) : swz_k<D>(r);
        if constexpr (!GATHER) {
          lds_dma16(base + (int64_t)(k0 + lb) * rowb, (uint32_t)(lr * rowb + 16 * (slot_c ^ sw)), dst + 1024 * j);
        } else {
          const int tok = cell_token(P, cell, lb + lr);
          lds_dma16_addr(base + (int64_t)tok * rowb + 16 * (slot_c ^ sw), dst + 1024 * j);
        }
      }
    };
    auto tb4 = [&](int s) { return tile_base(min(4 * s + ph, ntiles - 1)); };
    load_part(tb4(0), 0);
    load_part(tb4(0), 1);
    wait_newest_part();
    barrier();   // K of round 0 is in LDS
    for (int s = 0; s < nrounds; ++s) {
      const int it = 4 * s + ph;
      const bool act = wave_active && it < ntiles;   // wave-uniform
      const bool more = s + 1 < nrounds;             // uniform
      f32x16 st[2];
      if (act) {
        f32x16 tmp[QB][2];
        scores(buf, tmp);
        st[0] = tmp[0][0];
        st[1] = tmp[0][1];
      }
      barrier();   // both waves of each pair have read K of round s
      if (more) load_part(tb4(s + 1), 0);
      bf16x8 pbs[4];
      if (act) {
        const int lo = it * KTILE - tile_base(it);
        const int hi_end = short_set ? kn : KTILE;
        if (lo > 0 || hi_end < KTILE) mask_keys(st, lo, hi_end);
        float mx = st[0][0];
#pragma unroll
        for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, st[0][jj]);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, st[1][jj]);
        {
          const Pair pr = halves(mx);
          mx = fmaxf(pr.a, pr.b);
        }
        const bool grow = mx * c2 > fmaf(m_run[0], c2, kLazyLog2);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mx : m_run[0];
          const float alpha = __builtin_amdgcn_exp2f((m_run[0] - m_new) * c2);
          l_run[0] *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) oacc[0][t] *= alpha;
          m_run[0] = m_new;
        }
        const float mc = m_run[0] * c2;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          st[0][jj] = __builtin_amdgcn_exp2f(fmaf(st[0][jj], c2, -mc));
          st[1][jj] = __builtin_amdgcn_exp2f(fmaf(st[1][jj], c2, -mc));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pbs[0][e] = (__bf16)st[0][e];
          pbs[1][e] = (__bf16)st[0][8 + e];
          pbs[2][e] = (__bf16)st[1][e];
          pbs[3][e] = (__bf16)st[1][8 + e];
        }
        float psum = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 p2 = {pbs[kk][2 * e], pbs[kk][2 * e + 1]};
            const bf16x2 o2 = {ones8[0], ones8[1]};
            psum = __builtin_amdgcn_fdot2_f32_bf16(p2, o2, psum, false);
          }
        l_run[0] += psum;
      }
      if (more) wait_newest_part();   // V of round s has landed (K of round s+1 may still fly)
      else wait_all();
      barrier();   // ... for both waves of each pair
      if (act) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3)))*)((lds_u8*)buf + TL::KB + vt_addr(t, kk, 0)));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3)))*)((lds_u8*)buf + TL::KB + vt_addr(t, kk, 1)));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pbs[kk], oacc[0][t], 0, 0, 0);
          }
      }
      if (more) wait_all();   // K of round s+1 has landed
      barrier();   // both waves of each pair have read V of round s; K of round s+1 is in LDS
      if (more) load_part(tb4(s + 1), 1);
    }
    // Phases 1-3 hand (O, m, l) to phase 0 of the same query block: O through
    // their own buffer (both waves of a pair: 2 x 64 floats x 64 lanes at
    // d = 128, the buffer's size), m and l through s_ml.
    constexpr int NV = 16 * (D / 32);
    if (ph > 0) {
      float* xo = (float*)buf + mem * NV * 64;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) xo[(16 * t + i) * 64 + lane] = oacc[0][t][i];
      s_ml[wave][0][lane] = m_run[0];
      s_ml[wave][1][lane] = l_run[0];
    }
    __syncthreads();
    if (ph == 0) {
      float mp[4], ap[4];
      mp[0] = m_run[0];
#pragma unroll
      for (int p = 1; p < 4; ++p) mp[p] = s_ml[2 * p + mem][0][lane];
      const float M = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
#pragma unroll
      for (int p = 0; p < 4; ++p) ap[p] = __builtin_amdgcn_exp2f((mp[p] - M) * c2);
      float L = l_run[0] * ap[0];
#pragma unroll
      for (int p = 1; p < 4; ++p) L = fmaf(s_ml[2 * p + mem][1][lane], ap[p], L);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float o = oacc[0][t][i] * ap[0];
          o = fmaf(((const float*)smem1)[mem * NV * 64 + (16 * t + i) * 64 + lane], ap[1], o);
          o = fmaf(((const float*)smem2)[mem * NV * 64 + (16 * t + i) * 64 + lane], ap[2], o);
          o = fmaf(((const float*)smem3)[mem * NV * 64 + (16 * t + i) * 64 + lane], ap[3], o);
          oacc[0][t][i] = o;
        }
      l_run[0] = L;
      m_run[0] = M;
    }
    wave_active = wave_active && wave < 2;
    qvalid[0] = qvalid[0] && wave < 2;
  } else if constexpr (QB == 1) {
    // ---- small units, fp8 K/V: two key halves in parallel -------------------
    // Pair p = tiles 2p (half 0) and 2p+1 (half 1), computed by waves 0-3:
    // query block w & 1, half (w >> 1) & 1.  Pair p is staged as fp8 in two
    // staging buffers, widened by all eight waves into buffers (0,1), and
    // pair p+1 is staged while pair p is computed.  Not pipelined: each wave
    // computes the scores, softmax and PV of its tile in turn.
    const int half = (wave >> 1) & 1;
    const int npairs = (ntiles + 1) >> 1;
    auto tb = [&](int t) { return tile_base(min(t, ntiles - 1)); };
    auto barrier = [&]() {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // This wave's tile it of a pair, from the buffer buf.
    auto tile_compute = [&](const int it, const uint8_t* buf) {
      if (wave_active && it < ntiles) {
        f32x16 st[2];
        {
          f32x16 tmp[QB][2];
          scores(buf, tmp);
          st[0] = tmp[0][0];
          st[1] = tmp[0][1];
        }
        const int lo = it * KTILE - tile_base(it);
        const int hi_end = short_set ? kn : KTILE;
        if (lo > 0 || hi_end < KTILE) mask_keys(st, lo, hi_end);
        float mx = st[0][0];
#pragma unroll
        for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, st[0][jj]);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, st[1][jj]);
        {
          const Pair pr = halves(mx);
          mx = fmaxf(pr.a, pr.b);
        }
        const bool grow = mx * c2 > fmaf(m_run[0], c2, kLazyLog2);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mx : m_run[0];
          const float alpha = __builtin_amdgcn_exp2f((m_run[0] - m_new) * c2);
          l_run[0] *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) oacc[0][t] *= alpha;
          m_run[0] = m_new;
        }
        const float mc = m_run[0] * c2;
        bf16x8 pbs[4];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          st[0][jj] = __builtin_amdgcn_exp2f(fmaf(st[0][jj], c2, -mc));
          st[1][jj] = __builtin_amdgcn_exp2f(fmaf(st[1][jj], c2, -mc));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pbs[0][e] = (__bf16)st[0][e];
          pbs[1][e] = (__bf16)st[0][8 + e];
          pbs[2][e] = (__bf16)st[1][e];
          pbs[3][e] = (__bf16)st[1][8 + e];
        }
        float psum = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 p2 = {pbs[kk][2 * e], pbs[kk][2 * e + 1]};
            const bf16x2 o2 = {ones8[0], ones8[1]};
            psum = __builtin_amdgcn_fdot2_f32_bf16(p2, o2, psum, false);
          }
        l_run[0] += psum;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3)))*)((lds_u8*)buf + TL::KB + vt_addr(t, kk, 0)));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3)))*)((lds_u8*)buf + TL::KB + vt_addr(t, kk, 1)));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pbs[kk], oacc[0][t], 0, 0, 0);
          }
      }
    };
    {
      load8(tb(0), stg0);
      load8(tb(1), stg1);
      for (int p = 0; p < npairs; ++p) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();   // pair p staged by every wave; every read of pair p-1 done
        widen(stg0, smem0);
        widen(stg1, smem1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier();   // pair p widened, and the staging buffers read, by every wave
        if (p + 1 < npairs) {
          load8(tb(2 * p + 2), stg0);
          load8(tb(2 * p + 3), stg1);
        }
        tile_compute(2 * p + half, half ? smem1 : smem0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();   // every LDS read and load done: the buffers are free
    // waves 2, 3 hand their half (O, m, l) to waves 0, 1 of the same block
    constexpr int NV = 16 * (D / 32);
    float* xfer = (float*)((wave & 1) ? smem1 : smem0);
    if (wave == 2 || wave == 3) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) xfer[(16 * t + i) * 64 + lane] = oacc[0][t][i];
      xfer[NV * 64 + lane] = m_run[0];
      xfer[(NV + 1) * 64 + lane] = l_run[0];
    }
    __syncthreads();
    if (wave < 2) {
      const float mb = xfer[NV * 64 + lane], lb = xfer[(NV + 1) * 64 + lane];
      const float M = fmaxf(m_run[0], mb);
      const float aa = __builtin_amdgcn_exp2f((m_run[0] - M) * c2);
      const float ab = __builtin_amdgcn_exp2f((mb - M) * c2);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[0][t][i] = oacc[0][t][i] * aa + xfer[(16 * t + i) * 64 + lane] * ab;
      l_run[0] = l_run[0] * aa + lb * ab;
      m_run[0] = M;
    }
    wave_active = wave_active && wave < 2;
    qvalid[0] = qvalid[0] && wave < 2;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS load may outlive the work group

  // ---- epilogue -------------------------------------------------------------
  float l_tot[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const Pair pr = halves(l_run[b]);
    l_tot[b] = pr.a + pr.b;
  }
  const int splits = ranged ? C.splits : 1;

  if (splits > 1) {
    // Write this split's unnormalised partial, count it, and let the last split
    // to arrive merge.  The partials and the counter are accessed only with
    // device-scope atomic operations (relaxed; sc1 on this chip), which are
    // coherent across the XCDs' separate L2 caches by themselves, so no fence
    // has to write back or invalidate a whole L2 (an agent-scope fence does).
    // Partial layout per (id, split): O as [D/2][QT] float2 (consecutive
    // queries adjacent), then (m, l) as [QT] float2 after all O planes.
    const int id = slot * P.q_tiles + tile;
    const int n_ids = C.n_heads * P.q_tiles;
    uint64_t* po = (uint64_t*)(C.part + ((int64_t)id * splits + split) * QT * D);
    uint64_t* pml = (uint64_t*)(C.part + (int64_t)n_ids * splits * QT * D) + ((int64_t)id * splits + split) * QT;
    if (wave_active) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 2; ++e)
              store_coherent(po + (int64_t)(2 * (8 * t + 2 * g + hi) + e) * QT + qlocal[b],
                             oacc[b][t][4 * g + 2 * e], oacc[b][t][4 * g + 2 * e + 1]);
        if (hi == 0) store_coherent(pml + qlocal[b], m_run[b], l_tot[b]);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this lane's stores have landed
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(C.counters + id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (tid == 0) __hip_atomic_store(C.counters + id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
    // merge all splits for this lane's queries (its half of the channels)
    const uint64_t* pml0 = (const uint64_t*)(C.part + (int64_t)n_ids * splits * QT * D) + (int64_t)id * splits * QT;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      if (!qvalid[b]) continue;
      // (m, l) of every split: all loads issued before any result is used
      // (addresses past the last split repeat its own), then the maximum.
      float ms[kMaxSplits], ls[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        load_coherent(pml0 + (int64_t)min(s, splits - 1) * QT + qlocal[b], ms[s], ls[s]);
      float M = -INFINITY;
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        if (s < splits) M = fmaxf(M, ms[s]);
      float L = 0.f;
      float acc[D / 2];   // this lane's 16 (D=128) or 8 (D=64) column quadruples
#pragma unroll
      for (int i = 0; i < D / 2; ++i) acc[i] = 0.f;
      // Splits in index order whichever merges, so the sum is the same in
      // every run.  With a bf16 output this split's own partial is taken
      // from its registers (acc[16t + j] pairs with oacc[b][t][j]); the fp32
      // output variants read it back, which keeps them within the registers.
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) {
        if (s >= splits) break;   // uniform
        const float w = __builtin_amdgcn_exp2f((ms[s] - M) * c2);
        L = fmaf(w, ls[s], L);
        if (!OUT_F32 && s == split) {   // uniform
#pragma unroll
          for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[16 * t + j] = fmaf(w, oacc[b][t][j], acc[16 * t + j]);
          continue;
        }
        const uint64_t* ps = (const uint64_t*)(C.part + ((int64_t)id * splits + s) * QT * D);
        float x[D / 2];
#pragma unroll
        for (int i = 0; i < D / 4; ++i)   // i = 2*(4t+g)+e
          load_coherent(ps + (int64_t)(2 * (8 * (i >> 3) + 2 * ((i >> 1) & 3) + hi) + (i & 1)) * QT + qlocal[b],
                        x[2 * i], x[2 * i + 1]);
#pragma unroll
        for (int i = 0; i < D / 2; ++i) acc[i] = fmaf(w, x[i], acc[i]);
      }
      const float inv = P.v_scale / L;
      const int64_t obase = (int64_t)qh * C.o_sh + (int64_t)qtok[b] * C.o_st;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i = 4 * (4 * t + g);
          const f32x4 v = {acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
          store_row4<OUT_F32>(C.o, obase + 32 * t + 8 * g + 4 * hi, v);
        }
    }
    return;
  }

  const bool raw = C.ml_out != nullptr;   // unnormalised output plus the softmax state
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    if (!qvalid[b]) continue;
    const float inv = raw ? 1.f : P.v_scale / l_tot[b];
    if (raw && hi == 0) C.ml_out[(int64_t)qh * P.Nq + qtok[b]] = make_float2(m_run[b], l_tot[b]);
    const int64_t obase = (int64_t)qh * C.o_sh + (int64_t)qtok[b] * C.o_st;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {oacc[b][t][4 * g] * inv, oacc[b][t][4 * g + 1] * inv, oacc[b][t][4 * g + 2] * inv,
                         oacc[b][t][4 * g + 3] * inv};
        store_row4<OUT_F32>(C.o, obase + 32 * t + 8 * g + 4 * hi, v);
      }
  }
}

// Units of category ci on XCD x: ranged categories hand each XCD a contiguous
// run of their units (the q tiles of one key range are consecutive, so a
// range is read through one or two XCDs' L2s, not eight); the others every
// eighth unit.  Every XCD gets the same number of units to within one.
__device__ __forceinline__ int xcd_count(const AttnCat& C, int x) {
  const int n = C.n_heads * C.units_per_head;
  return C.kind == KIND_RANGED ? (n >> 3) + (x < (n & 7) ? 1 : 0) : (n > x ? (n - x + 7) >> 3 : 0);
}
__device__ __forceinline__ int xcd_unit(const AttnCat& C, int x, int i) {
  const int n = C.n_heads * C.units_per_head;
  return C.kind == KIND_RANGED ? x * (n >> 3) + min(x, n & 7) + i : x + 8 * i;
}

// Work groups reach the eight XCDs round robin (work group b on XCD b mod 8)
// and each XCD has its own L2.
//   Static mode (P.work_ctr == nullptr): one work group per unit; work group
//   b of a category runs unit i of XCD b mod 8's run, i = its position there.
//   Persistent mode: P.grid work groups; each takes the units of its XCD's
//   list (categories in launch order, heaviest first) one after another,
//   from a per-XCD counter, until the list is exhausted, so each XCD's
//   compute units pick up work as they come free instead of in the fixed
//   queue order of the hardware dispatcher.  The last work group of each XCD
//   to finish resets its counters for the next launch.
template <int D, int QB, bool OUT_F32, bool GATHER, bool KV8 = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2 / QB, 2 / QB)))
void attn_bf16_kernel(const AttnPlan P) {
  __shared__ int s_unit;
  const bool persistent = P.work_ctr != nullptr;
  const int x = blockIdx.x & 7;
  // One copy of the unit body for both modes (static mode: one pass).
  for (int pass = 0;; ++pass) {
    int ci = -1, rel = 0;
    if (!persistent) {
      const int u = blockIdx.x;
      if (pass > 0 || u >= P.total_units) break;
      ci = 0;
#pragma unroll
      for (int c = 1; c < 4; ++c)
        if (c < P.n_cats && u >= P.cat[c].unit_begin) ci = c;
      rel = u - P.cat[ci].unit_begin;
      if (P.cat[ci].kind == KIND_RANGED) rel = xcd_unit(P.cat[ci], rel & 7, rel >> 3);
    } else {
      if (threadIdx.x == 0)
        s_unit = __hip_atomic_fetch_add(P.work_ctr + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      int i = __builtin_amdgcn_readfirstlane(s_unit);
      __syncthreads();   // s_unit is rewritten only after every thread has read it
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < P.n_cats && ci < 0) {
          const int n = xcd_count(P.cat[c], x);
          if (i < n) {
            ci = c;
            rel = xcd_unit(P.cat[c], x, i);
          } else {
            i -= n;
          }
        }
      }
      if (ci < 0) break;   // this XCD's list is exhausted (uniform over the work group)
    }
    // Opaque per pass: nothing the unit derives from the plan or the thread
    // index is hoisted out of this loop and kept live across units (which
    // would not fit the registers of two waves per SIMD).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    attn_unit<D, QB, OUT_F32, GATHER, KV8>(P, ci, rel, tid);
  }
  if (!persistent) return;
  if (threadIdx.x == 0) {
    const int wgs = (P.grid - x + 7) >> 3;   // work groups of this XCD
    if (__hip_atomic_fetch_add(P.work_ctr + 8 + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == wgs - 1) {
      __hip_atomic_store(P.work_ctr + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.work_ctr + 8 + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnPlan& plan, int head_dim, hipStream_t s) {
  if (plan.total_units <= 0) return hipSuccess;
  const bool f32 = plan.cat[0].out_f32 != 0;
  auto gathers = [](int kind) { return kind == KIND_CELL_GATHER || kind == KIND_BOX_GATHER; };
  const bool gather = gathers(plan.cat[0].kind);
  for (int c = 1; c < plan.n_cats; ++c)
    if (gathers(plan.cat[c].kind) != gather) return hipErrorInvalidValue;  // one mode per launch
  dim3 grid(plan.work_ctr ? plan.grid : plan.total_units), block(NT);
#define HC_LAUNCH(DD, F, G) hipLaunchKernelGGL((attn_bf16_kernel<DD, kBf16QueryBlocks, F, G>), grid, block, 0, s, plan)
  if (plan.kv8) {   // fp8 K/V: bf16 output, cache kinds only
    if (gather || f32) return hipErrorInvalidValue;
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_bf16_kernel<128, kBf16QueryBlocks, false, false, true>), grid, block, 0, s, plan);
    else if (head_dim == 64)
      hipLaunchKernelGGL((attn_bf16_kernel<64, kBf16QueryBlocks, false, false, true>), grid, block, 0, s, plan);
    else
      return hipErrorInvalidValue;
  } else if (head_dim == 128) {
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
