// bf16 MFMA GEMM kernels  C = A B^T  (A [M][K], B [N][K], both K-contiguous)
// with the fused epilogues of the block.  Included by gemm.hip only.
//
// Both kernels use v_mfma_f32_32x32x16_bf16 on 64-wide waves: each lane feeds
// one 16-byte LDS read per operand per 16-wide k step.
//
//   gemm_regs_kernel : global -> VGPR -> LDS staging, two LDS buffers of
//                      64-wide K slices (small and odd shapes).
//   gemm_ring_kernel : global -> LDS directly (global_load_lds_dwordx4) into a
//                      ring of K slices, software-pipelined so the MFMA pipe
//                      never waits on a barrier or an LDS read (the large
//                      projections).
//
// LDS bank layout (gfx950: 64 banks x 4 bytes, a 128-bit read serves 16 lanes
// per cycle).  An MFMA operand read puts 16 consecutive rows, same logical
// 16-byte chunk, into one 16-lane group, so the chunk index is XOR-swizzled by
// a function of the row that gives those 16 rows 16 distinct 16-byte slots of
// the 256-byte bank line.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {
namespace gemm {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gmem_void_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));




// Rows of a K slice of width BK hold CPR = BK/8 chunks of 16 bytes; RPL rows
// share a 256-byte bank line.  Chunk c of row r lives at c ^ swz(r).
template <int BK>
struct Layout {
  static constexpr int CPR = BK / 8;
  static constexpr int RPL = 16 / CPR;
  static constexpr int RPB = 64 / CPR;  // rows per 1 KiB (one wave-wide 16-byte access)
  __device__ static __forceinline__ int swz(int row) { return (row / RPL) % CPR; }
};

// One 32x32x16 step of a fragment, computed transposed: the MFMA's A operand
// is the weight fragment and its B operand the activation fragment, so the
// accumulator holds C^T.  Accumulator element r of lane l is then
//   output row = l % 32,  output col = 8 * (r / 4) + 4 * (l / 32) + r % 4,
// i.e. each lane owns one output row and 4 consecutive columns per group of
// 4 registers, which the epilogue stores as one 8- or 16-byte access.
__device__ __forceinline__ floatx16 mma(const bf16x8& x_frag, const bf16x8& w_frag, floatx16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w_frag, x_frag, acc, 0, 0, 0);
}
__device__ __forceinline__ int frag_col(int g4, int lane) { return 8 * g4 + 4 * (lane >> 5); }

// Store half of one fragment row's 32 bf16 values as 16-byte accesses: lo and
// hi are groups 2q and 2q + 1 (columns frag_col(2q, lane) .. +3 and
// frag_col(2q + 1, lane) .. +3 of lane l's row, and lane l ^ 32's).  The two
// lanes first trade groups (v_permlane32_swap moves the upper half's first
// operand and the lower half's second), so lane l holds columns 16q .. 16q+7
// and lane l + 32 columns 16q+8 .. 16q+15; each store then writes 32
// contiguous bytes of the row per lane pair instead of two 8-byte pieces.
// p: the fragment's first column in the row.  Lanes l and l + 32 hold the
// same row, so both are active or neither.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_frag_half(bf16* p, int q, bf16x4 lo, bf16x4 hi, int lane) {
  u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const auto r = __builtin_amdgcn_permlane32_swap(a[d], b[d], false, false);
    a[d] = r[0];
    b[d] = r[1];
  }
  const u32x4_t w = {a[0], a[1], b[0], b[1]};
  *(u32x4_t*)(p + 16 * q + 8 * (lane >> 5)) = w;
}

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 fragments");
};

// Tile order: XCD-contiguous bands of the tile grid (workgroups are dealt to
// the 8 XCDs round-robin), then groups of 3 tile rows, so the tiles running
// at the same time on one XCD share A rows and B rows in that XCD's L2.
// Position `lin` of the grouped order: groups of 3 tile rows, walked column
// by column, so neighbouring positions share A rows or B rows (3 rows of A,
// 4.5 MB at K = 3072, about one XCD's L2; 3 measured faster than 2, 4, 6 or 8
// for the 4608-row in-projection and at the step level).
// GM: tile rows per group (the stream-K output projection passes its own).
__device__ __forceinline__ void grouped_coords(int lin, int tiles_m, int tiles_n, int& tm, int& tn,
                                               int GM = 3) {
  const int group = lin / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = lin - group * GM * tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  grouped_coords(lin, tiles_m, tiles_n, tm, tn);
}

// Tiles of one workgroup of a persistent launch (gridDim.x workgroups, at
// most one per CU, all resident).  Workgroup b runs on XCD b % 8; XCD x owns
// a contiguous band of the grouped order, sized to its workgroup count so
// every workgroup gets floor or ceil of tiles / gridDim.x tiles, and its
// workgroups take the band's tiles round-robin: the tiles one XCD runs at
// the same time are neighbours and share operand rows in its L2.
struct TileWalk {
  int lo, first, step, count;
  __device__ __forceinline__ TileWalk(int total) {
    const int G = gridDim.x, b = blockIdx.x, x = b & 7;
    const int q = total / G, r = total % G;
    lo = 0;
    int cnt = 0;
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      const int c = q * ((G - y + 7) >> 3) + (r > y ? (r - y + 7) >> 3 : 0);
      if (y < x) lo += c;
      if (y == x) cnt = c;
    }
    step = (G - x + 7) >> 3;
    first = b >> 3;
    count = first < cnt ? (cnt - first + step - 1) / step : 0;
  }
  __device__ __forceinline__ void coords(int i, int tiles_m, int tiles_n, int& tm, int& tn) const {
    grouped_coords(lo + first + i * step, tiles_m, tiles_n, tm, tn);
  }
  // Work item i when each tile is split into `splits` K ranges (consecutive
  // items are the ranges of one tile).
  __device__ __forceinline__ void coords(int i, int tiles_m, int tiles_n, int splits, int& tm, int& tn,
                                         int& split) const {
    const int lin = lo + first + i * step;
    split = lin % splits;
    grouped_coords(lin / splits, tiles_m, tiles_n, tm, tn);
  }
};

// Epilogue of one wave's WTM x WTN accumulator tile (rows wrow0.., columns
// wcol0..), for one epilogue kind.  Each lane owns one output row and 4
// consecutive columns per group of 4 accumulator registers.
//
// Register discipline: a spilled register reloaded here would wait for every
// store issued before it (vmcnt counts stores on this architecture).  The
// lane index is recomputed here by an opaque instruction pair, so no per-lane
// address arithmetic is hoisted into the surrounding tile loop to hold a
// register there, and scheduling fences after each fragment keep the
// accumulator reads of one fragment together.
//
// SC (fp8 products): every value is first scaled by its row's and column's
// scale, read from LDS (sc: the wave's 128 row scales, then at sc + 128 its
// 128 column scales); LDS reads wait on lgkmcnt, not on the stores in flight.
//
// MG (stream-K, kGatedResidual): the tile's K range was split into two or
// three parts; acc holds this wave's part, o1 and o2 the other parts' values
// for the same wave tile (o2 null with two parts), in part order, stored by
// sk_store_part.  They are added in part order whoever holds which part:
// (P0 + P1) + P2, with own_last when acc is P2, else acc is P0 or P1 and
// (acc + other) + P2 is the same sum exactly (IEEE addition commutes).
// The q or k columns of a wave tile 128 columns wide (one head: wcol0 is a
// multiple of 128) with the head's RMSNorm and RoPE applied before the store,
// in the arithmetic of qk_norm_rope_kernel: the projection rounded to bf16,
// then x / sqrt(mean_128(x^2) + 1e-6) * scale, then each pair (2p, 2p+1)
// rotated by the row's table entry p, rounded to bf16.  Lane l holds 64 of
// the 128 values of rows wrow0 + 32 i + l % 32 (four consecutive columns per
// register group); lane l ^ 32 holds the other 64.
template <class T>
__device__ __forceinline__ void qk_norm_rope_tile(const GemmArgs& g, floatx16 (&acc)[T::FM][T::FN], int wrow0,
                                                  int wcol0, int lane) {
  static_assert(T::FN * 32 == kHeadDim, "one head per wave tile");
  const int lr = lane & 31;
  const bf16* scale = wcol0 >= kHidden ? g.qk_scale_k : g.qk_scale_q;
  bf16x4 sc[T::FN][4];
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) sc[j][g4] = *(const bf16x4*)(scale + 32 * j + frag_col(g4, lane));
  bf16* C = (bf16*)g.C;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int row = wrow0 + 32 * i + lr;
    // (cos, sin) of this lane's pairs; rows past M-1 read row M-1's
    const float* t = g.rope_table + (size_t)min(row, g.M - 1) * kHeadDim;
    float4 tb[T::FN][4];
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) tb[j][g4] = *(const float4*)(t + 32 * j + frag_col(g4, lane));
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = to_f32(to_bf16(acc[i][j][r]));
        s += v * v;
      }
    s += __shfl_xor(s, 32, 64);
    const float rn = 1.0f / sqrtf(s * (1.0f / kHeadDim) + 1e-6f);
    if (row < g.M) {
      bf16* crow = C + (size_t)row * g.ldc + wcol0;
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          bf16x4 o[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int g4 = 2 * q + u;
            const float4 tt = tb[j][g4];  // (cos, sin) of pairs c/2 and c/2 + 1
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_f32(to_bf16(acc[i][j][4 * g4 + e])) * rn * to_f32(sc[j][g4][e]);
            o[u][0] = to_bf16(v[0] * tt.x - v[1] * tt.y);
            o[u][1] = to_bf16(v[0] * tt.y + v[1] * tt.x);
            o[u][2] = to_bf16(v[2] * tt.z - v[3] * tt.w);
            o[u][3] = to_bf16(v[2] * tt.w + v[3] * tt.z);
          }
          store_frag_half(crow + 32 * j, q, o[0], o[1], lane);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <class T, GemmEpi EPI, bool SC = false, bool MG = false>
__device__ __forceinline__ void epilogue(const GemmArgs& g, floatx16 (&acc)[T::FM][T::FN],
                                         int wrow0, int wcol0, const float* sc = nullptr,
                                         const float* o1 = nullptr, const float* o2 = nullptr,
                                         bool own_last = false) {
  static_assert(!MG || !SC, "stream-K merge: bf16 products");  // MG acts in the gated residual only
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int lr = lane & 31;
  // Fragment (i, j), register group g4, with the fp8 scales applied.
  auto f4 = [&](int i, int j, int g4, float sa) -> float4 {
    float4 v = make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                           acc[i][j][4 * g4 + 3]);
    if constexpr (SC) {
      const float4 w = *(const float4*)(sc + 128 + 32 * j + frag_col(g4, lane));
      v.x *= sa * w.x;
      v.y *= sa * w.y;
      v.z *= sa * w.z;
      v.w *= sa * w.w;
    }
    return v;
  };
  auto row_scale = [&](int i) -> float {
    if constexpr (SC) return sc[32 * i + lr];
    else return 1.f;
  };
  if constexpr (EPI == GemmEpi::kInProj && !SC && T::FN * 32 == kHeadDim) {
    if (g.rope_table != nullptr && wcol0 < 2 * kHidden) {  // wave-uniform
      qk_norm_rope_tile<T>(g, acc, wrow0, wcol0, lane);
      return;
    }
  }
  if constexpr (EPI == GemmEpi::kStoreBf16 || EPI == GemmEpi::kInProj) {
    if (EPI == GemmEpi::kStoreBf16 || wcol0 < 3 * kHidden) {
      bf16* C = (bf16*)g.C;
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int row = wrow0 + 32 * i + lr;
        if (row < g.M) {
          const float sa = row_scale(i);
          bf16* crow = C + (size_t)row * g.ldc + wcol0;
#pragma unroll
          for (int j = 0; j < T::FN; ++j) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              bf16x4 v[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float4 f = f4(i, j, 2 * q + u, sa);
                v[u][0] = to_bf16(f.x);
                v[u][1] = to_bf16(f.y);
                v[u][2] = to_bf16(f.z);
                v[u][3] = to_bf16(f.w);
              }
              store_frag_half(crow + 32 * j, q, v[0], v[1], lane);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
      // SwiGLU: fragment 2p holds a-columns, 2p+1 the matching b-columns.
      static_assert(T::FN % 2 == 0, "SwiGLU needs fragment pairs");
      const int hcol0 = (wcol0 - 3 * kHidden) / 2;
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int row = wrow0 + 32 * i + lr;
        if (row < g.M) {
          const float sa = row_scale(i);
          bf16* hrow = g.H + (size_t)row * g.ldh + hcol0;
#pragma unroll
          for (int p = 0; p < T::FN / 2; ++p) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              bf16x4 v[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float4 a = f4(i, 2 * p, 2 * q + u, sa), b = f4(i, 2 * p + 1, 2 * q + u, sa);
                v[u][0] = to_bf16(silu_f(a.x) * b.x);
                v[u][1] = to_bf16(silu_f(a.y) * b.y);
                v[u][2] = to_bf16(silu_f(a.z) * b.z);
                v[u][3] = to_bf16(silu_f(a.w) * b.w);
              }
              store_frag_half(hrow + 32 * p, q, v[0], v[1], lane);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  } else if constexpr (EPI == GemmEpi::kStoreF32) {
    float* C = (float*)g.C;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int row = wrow0 + 32 * i + lr;
      if (row < g.M) {
        const float sa = row_scale(i);
        float* crow = C + (size_t)row * g.ldc + wcol0;
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *(float4*)(crow + 32 * j + frag_col(g4, lane)) = f4(i, j, g4, sa);
      }
    }
  } else if constexpr (EPI == GemmEpi::kSplitPartial) {
    // fp32 partial product of one K range into the split scratch (rows of a
    // ragged last tile land in padding that is never read).
    float* C = (float*)g.C;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const float sa = row_scale(i);
      float* crow = C + (size_t)(wrow0 + 32 * i + lr) * g.ldc + wcol0;
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(float4*)(crow + 32 * j + frag_col(g4, lane)) = f4(i, j, g4, sa);
    }
  } else {
    static_assert(EPI == GemmEpi::kGatedResidual, "epilogue kind");
    // x and gate are distinct buffers: all loads of one fragment are issued
    // before its stores.
    constexpr int kSC1 = 16;  // buffer cache policy: bypass the non-coherent caches
    constexpr int QB = T::FM * T::FN * 32 * 32 * 4;  // bytes of one wave tile's part
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc((void*)o1, (short)0, QB, 0x00020000);
    const __amdgpu_buffer_rsrc_t r2 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(o2 ? o2 : o1), (short)0, QB, 0x00020000);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int row = wrow0 + 32 * i + lr;
      if (row < g.M) {
        const float sa = row_scale(i);
        const float* __restrict__ gate =
            g.mod + (size_t)seg_of_row(g.seg, row) * g.mod_stride + g.gate_offset + wcol0;
        float* __restrict__ xrow = (float*)g.C + (size_t)row * g.ldc + wcol0;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          float4 gt[4], xv[4];
          [[maybe_unused]] u32x4 p1[4], p2[4];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int c = 32 * j + frag_col(g4, lane);
            gt[g4] = *(const float4*)(gate + c);
            xv[g4] = *(const float4*)(xrow + c);
            if constexpr (MG) {
              const int off = (((i * T::FN + j) * 4 + g4) * 64 + lane) * 16;
              p1[g4] = __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, kSC1);
              p2[g4] = o2 ? __builtin_amdgcn_raw_buffer_load_b128(r2, off, 0, kSC1) : u32x4{0, 0, 0, 0};
            }
          }
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int c = 32 * j + frag_col(g4, lane);
            float4 f = f4(i, j, g4, sa);
            if constexpr (MG) {
              const float4 a = make_float4(__uint_as_float(p1[g4][0]), __uint_as_float(p1[g4][1]),
                                           __uint_as_float(p1[g4][2]), __uint_as_float(p1[g4][3]));
              const float4 b = make_float4(__uint_as_float(p2[g4][0]), __uint_as_float(p2[g4][1]),
                                           __uint_as_float(p2[g4][2]), __uint_as_float(p2[g4][3]));
              if (own_last) {
                f = make_float4((a.x + b.x) + f.x, (a.y + b.y) + f.y, (a.z + b.z) + f.z, (a.w + b.w) + f.w);
              } else {
                f = make_float4((f.x + a.x) + b.x, (f.y + a.y) + b.y, (f.z + a.z) + b.z, (f.w + a.w) + b.w);
              }
            }
            float4 r = xv[g4];
            r.x += gt[g4].x * f.x;
            r.y += gt[g4].y * f.y;
            r.z += gt[g4].z * f.z;
            r.w += gt[g4].w * f.w;
            *(float4*)(xrow + c) = r;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

// Runtime-selected epilogue (small-shape kernel).
template <class T>
__device__ __forceinline__ void epilogue_any(const GemmArgs& g, floatx16 (&acc)[T::FM][T::FN],
                                             int wrow0, int wcol0) {
  switch (g.epi) {
    case GemmEpi::kStoreBf16: epilogue<T, GemmEpi::kStoreBf16>(g, acc, wrow0, wcol0); break;
    case GemmEpi::kStoreF32: epilogue<T, GemmEpi::kStoreF32>(g, acc, wrow0, wcol0); break;
    case GemmEpi::kInProj: epilogue<T, GemmEpi::kInProj>(g, acc, wrow0, wcol0); break;
    case GemmEpi::kGatedResidual: epilogue<T, GemmEpi::kGatedResidual>(g, acc, wrow0, wcol0); break;
  }
}

// ---------------------------------------------------------------------------
// Register-staged kernel (64-wide K slices, two LDS buffers, one barrier per
// slice).
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_regs_kernel(GemmArgs g, int tiles_m,
                                                                int tiles_n) {
  using T = Tile<BM, BN, WM, WN>;
  using Lay = Layout<64>;
  constexpr int ACH = BM * 8 / T::NT;  // 16-byte chunks of A per thread per slice
  constexpr int BCH = BN * 8 / T::NT;
  constexpr int STAGE = (BM + BN) * 8;
  static_assert((BM * 8) % T::NT == 0 && (BN * 8) % T::NT == 0, "slice must split evenly");
  __shared__ bf16x8 lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Global -> register staging addresses (rows of A clamped to M-1).
  const bf16* a_src[ACH];
  int a_lds[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int id = tid + i * T::NT;
    const int row = id >> 3, c = id & 7;
    const int grow = min(m0 + row, g.M - 1);
    a_src[i] = g.A + (size_t)grow * g.lda + c * 8;
    a_lds[i] = row * 8 + (c ^ Lay::swz(row));
  }
  const bf16* b_src[BCH];
  int b_lds[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int id = tid + i * T::NT;
    const int row = id >> 3, c = id & 7;
    b_src[i] = g.B + (size_t)(n0 + row) * g.ldb + c * 8;
    b_lds[i] = BM * 8 + row * 8 + (c ^ Lay::swz(row));
  }

  floatx16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 ra[ACH], rb[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) ra[i] = *(const bf16x8*)a_src[i];
#pragma unroll
  for (int i = 0; i < BCH; ++i) rb[i] = *(const bf16x8*)b_src[i];
#pragma unroll
  for (int i = 0; i < ACH; ++i) lds[a_lds[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < BCH; ++i) lds[b_lds[i]] = rb[i];
  __syncthreads();

  const int lr = lane & 31, lh = lane >> 5;
  int a_off[T::FM], b_off[T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i) a_off[i] = (wm * T::WTM + 32 * i + lr) * 8;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) b_off[j] = BM * 8 + (wn * T::WTN + 32 * j + lr) * 8;
  const int sw = Lay::swz(lr);  // rows read by this lane are 32 k + lr

  const int KT = g.K / 64;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = (kt & 1) * STAGE;
    if (kt + 1 < KT) {
      const int koff = (kt + 1) * 64;
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra[i] = *(const bf16x8*)(a_src[i] + koff);
#pragma unroll
      for (int i = 0; i < BCH; ++i) rb[i] = *(const bf16x8*)(b_src[i] + koff);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = (2 * ks + lh) ^ sw;
      bf16x8 af[T::FM], bfr[T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; ++i) af[i] = lds[cur + a_off[i] + ch];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) bfr[j] = lds[cur + b_off[j] + ch];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = mma(af[i], bfr[j], acc[i][j]);
    }
    // Buffer cur ^ 1 was last read before the previous barrier.
    if (kt + 1 < KT) {
      const int nxt = STAGE - cur;
#pragma unroll
      for (int i = 0; i < ACH; ++i) lds[nxt + a_lds[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) lds[nxt + b_lds[i]] = rb[i];
    }
    __syncthreads();
  }

  epilogue_any<T>(g, acc, m0 + wm * T::WTM, n0 + wn * T::WTN);
}

// ---------------------------------------------------------------------------
// Ring kernel (persistent).
//
// STAGES LDS buffers hold K slices of width BK.  Each global_load_lds_dwordx4
// of a wave fills one KiB of a buffer (RPB rows); lane t lands at chunk t of
// that KiB (row t / CPR, physical chunk t % CPR), so it fetches logical chunk
// (t % CPR) ^ swz(row).
//
// A workgroup walks its tiles (TileWalk) and the K slices of consecutive
// tiles form one stream through the ring: the first slices of the next tile
// are loading while the current tile finishes, and its output stores drain
// behind the next tile's MFMAs.
//
// Per slice (KSTEPS = BK/16 MFMA steps of FM x FN MFMAs per wave):
//   steps 0 .. KSTEPS-2 : read the fragments of the next step, then the MFMAs
//                         of this step (the reads hide behind the MFMAs);
//   before the last step: wait until this wave's copy of the next slice
//                         landed, barrier (next slice visible to all; everyone
//                         has read all of this slice), read the first
//                         fragments of the next slice, then the last MFMAs of
//                         this slice with the refill of its buffer (the slice
//                         STAGES ahead) issued one load per MFMA between them;
//   after the last slice of a tile: the epilogue, then zero accumulators.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

//
// SK (stream-K, kGatedResidual): the work is the product's K slices in tile
// order (grouped order, KTT = K / BK slices per tile), cut into gridDim.x
// equal runs; run v goes to the workgroup at position v of the XCD-major
// order (the runs of one XCD are contiguous, so the parts of a tile mostly
// share an L2).  A workgroup's items are the pieces of tiles its run covers
// (the piece that starts inside a tile last, see `item`);
// a tile covered by one run is finished as usual, a tile cut into parts
// (two or three: runs are at least half a tile long) by the last of its
// parts to arrive (sk_finish), with no workgroup ever waiting for another.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int WAVES_PER_EU, GemmEpi EPI, bool SK = false>
__global__ __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void gemm_ring_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  using T = Tile<BM, BN, WM, WN>;
  using Lay = Layout<BK>;
  constexpr int NW = WM * WN;
  constexpr int CPR = Lay::CPR;
  constexpr int STAGE = (BM + BN) * CPR;     // 16-byte chunks per buffer
  constexpr int A_BLK = BM / Lay::RPB / NW;  // KiB blocks of A per wave per slice
  constexpr int B_BLK = BN / Lay::RPB / NW;
  constexpr int PER = A_BLK + B_BLK;         // loads per wave per slice
  constexpr int KSTEPS = BK / 16;
  constexpr int NMF = T::FM * T::FN;         // MFMAs per step
  static_assert(BM % (Lay::RPB * NW) == 0 && BN % (Lay::RPB * NW) == 0, "rows must split over waves");
  static_assert((STAGES - 1) * PER < 64 && STAGES >= 2 && STAGES <= 5, "ring depth");
  static_assert(KSTEPS >= 2, "BK >= 32");
  __shared__ bf16x8 lds[STAGES * STAGE];

  static_assert(!SK || EPI == GemmEpi::kGatedResidual, "stream-K: gated residual");
  const int splits = EPI == GemmEpi::kSplitPartial ? g.ksplit : 1;
  const TileWalk walk(SK ? 0 : tiles_m * tiles_n * splits);
  const int KTT = g.K / BK;  // K slices per tile
  // Stream-K run [sk_s0, sk_s1) of the S slices; sk_t0 = its first tile.
  const long sk_S = (long)tiles_m * tiles_n * KTT;
  const int sk_v = SK && (gridDim.x & 7) == 0 ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                                              : blockIdx.x;
  const long sk_s0 = (long)sk_v * sk_S / gridDim.x, sk_s1 = (long)(sk_v + 1) * sk_S / gridDim.x;
  const int sk_t0 = (int)(sk_s0 / KTT);
  const int count = SK ? (sk_s1 > sk_s0 ? (int)((sk_s1 - 1) / KTT) - sk_t0 + 1 : 0) : walk.count;
  const int sk_gm = g.group_m > 0 ? g.group_m : 3;  // tile rows per group of the stream-K order
  if constexpr (EPI == GemmEpi::kInProj) {
    // counters the kernels after this one expect at zero
    if (blockIdx.x == 0 && g.zero != nullptr)
      for (int i = threadIdx.x; i < g.nzero; i += NW * 64) g.zero[i] = 0;
  }
  if (count == 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // Load addresses: a uniform base (scalar registers: the tile's origin plus
  // the k offset of the slice) plus a 32-bit per-lane byte offset per KiB
  // block.  A lane's offset inside a block depends only on the block's row
  // (its swizzle) and, for A, on the clamp of rows past M-1 in the last tile
  // row, so the B offsets are fixed and the A offsets change with the tile.
  const int sub_row = lane / CPR;
  unsigned voff_a[A_BLK], voff_b[B_BLK];
#pragma unroll
  for (int q = 0; q < B_BLK; ++q) {
    const int row = (wave * B_BLK + q) * Lay::RPB + sub_row;
    const int chunk = (lane % CPR) ^ Lay::swz(row);
    voff_b[q] = (unsigned)(row * g.ldb * 2 + chunk * 16);
  }
  const char* a_tile;
  const char* b_tile;
  const int KT = g.K / BK / splits;  // K slices per work item without SK, >= 1
  // Stream-K work item i: tile `lin` of the grouped order, its K slices
  // [kb, kb + len).  A run that starts inside a tile takes that piece last:
  // every other item starts at k = 0, so the workgroups running at the same
  // time stay within (tile length - run length) slices of the same k and
  // share the A and B slices they read in L2 (taken in run order, the
  // workgroups' k offsets would differ by multiples of the run length).
  const int sk_rot = SK && count > 1 && sk_s0 % KTT != 0 ? 1 : 0;
  auto item = [&](int i, int& lin, int& kb, int& len) {
    lin = sk_t0 + (i + sk_rot) % count;
    const long t0 = (long)lin * KTT;
    kb = (int)(sk_s0 > t0 ? sk_s0 - t0 : 0);
    len = (int)(sk_s1 - t0 < KTT ? sk_s1 - t0 : KTT) - kb;
  };
  int ld_len = KT;  // slices of the item the load cursor is in
  auto set_src = [&](int i) {
    int tm, tn;
    size_t k0;
    if constexpr (SK) {
      int lin, kb;
      item(i, lin, kb, ld_len);
      grouped_coords(lin, tiles_m, tiles_n, tm, tn, sk_gm);
      k0 = (size_t)kb * BK;
    } else {
      int split;
      walk.coords(i, tiles_m, tiles_n, splits, tm, tn, split);
      k0 = (size_t)split * KT * BK;
    }
    const int m0 = tm * BM;
    a_tile = (const char*)(g.A + (size_t)m0 * g.lda + k0);
    b_tile = (const char*)(g.B + (size_t)tn * BN * g.ldb + k0);
#pragma unroll
    for (int q = 0; q < A_BLK; ++q) {
      const int row = (wave * A_BLK + q) * Lay::RPB + sub_row;
      const int chunk = (lane % CPR) ^ Lay::swz(row);
      voff_a[q] = (unsigned)((min(m0 + row, g.M - 1) - m0) * g.lda * 2 + chunk * 16);
    }
  };
  // One KiB of a slice into LDS from the open refill (sources r_a / r_b,
  // this wave's part of LDS buffer r_dst): each lane lands 16 bytes at
  // m0 + 16 * lane; writing m0 needs one wait state before the load reads
  // it.  Issued as inline assembly: the compiler would otherwise treat the
  // LDS write as possibly aliasing every fragment read that follows it and
  // wait for all loads in flight before each of them.  The ring's explicit
  // vmcnt waits and barriers order these loads against the reads; they have
  // no register results.
  const unsigned lds_base = (unsigned)(size_t)(lds_void_t*)lds;
  const char* r_a = nullptr;
  const char* r_b = nullptr;
  unsigned r_dst = 0;
  auto open_refill = [&](int slot, int koff) {
    r_a = a_tile + koff * 2;
    r_b = b_tile + koff * 2;
    r_dst = lds_base + (unsigned)(slot * STAGE) * 16u;
  };
  auto load_one = [&](int q) __attribute__((always_inline)) {
    const bool is_a = q < A_BLK;
    const int blk = is_a ? wave * A_BLK + q : BM / Lay::RPB + wave * B_BLK + (q - A_BLK);
    const unsigned dst = r_dst + (unsigned)blk * 1024u;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(is_a ? voff_a[q] : voff_b[q - A_BLK]), "s"(is_a ? r_a : r_b), "s"(dst)
                 : "m0");
  };
  // Load cursor: tile ld_i, slice ld_kt.  Past the last slice it stays there:
  // every refill still issues PER loads (the final slice again, into buffers
  // that are no longer read), so the count of loads in flight behind a given
  // slice is constant.
  int ld_i = 0, ld_kt = 0;
  auto advance_load = [&]() {
    const int len = SK ? ld_len : KT;
    if (++ld_kt == len) {
      if (ld_i + 1 < count) {
        ++ld_i;
        ld_kt = 0;
        set_src(ld_i);
      } else {
        ld_kt = len - 1;
      }
    }
  };

  floatx16 acc[T::FM][T::FN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero_acc();

  const int lr = lane & 31, lh = lane >> 5;
  const int sw = Lay::swz(lr);  // rows read by this lane are 32 k + lr
  const int a_base = (wm * T::WTM + lr) * CPR;
  const int b_base = BM * CPR + (wn * T::WTN + lr) * CPR;
  bf16x8 af[2][T::FM], bfr[2][T::FN];
  auto read_frags = [&](int buf, int ks, int p) {
    const int ch = (2 * ks + lh) ^ sw;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) af[p][i] = lds[buf + a_base + i * 32 * CPR + ch];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) bfr[p][j] = lds[buf + b_base + j * 32 * CPR + ch];
  };

  // Refill scheme.  The barrier before the last k step of slice t (every
  // wave has read all of slice t, slice t+1 has landed) opens the refill of
  // slice t's buffer with the slice STAGES ahead.  Its PER loads are spread
  // over the next KSTEPS k steps (the last step of slice t and the first
  // KSTEPS-1 steps of slice t+1), LPS per step, each one issued right after
  // an MFMA: a 64-lane load holds up the wave's instruction issue for a
  // while, and behind a just-issued MFMA that time is mostly hidden (all
  // PER loads in one step cost ~20% of the MFMA rate, spread this way ~9%).
  // So one refill is issued between consecutive barriers, and the slice a
  // barrier waits for had STAGES-2 refills issued after it.
  constexpr int LPS = PER / KSTEPS;
  static_assert(T::FM == 4 && T::FN == 4, "four MFMA segments of four per step");
  static_assert(PER % KSTEPS == 0 && LPS <= 4, "refill loads per step");
  static_assert(STAGES >= 3, "a refill spans a barrier");
  static_assert(KSTEPS % 2 == 0, "the next slice's first fragments land in slot 0");
  // One k step: its 16 MFMAs (fragments P) in four segments.  Each segment
  // also reads two fragments of the next step (into 1-P), then one load of
  // the open refill (the first LPS segments).
  auto step = [&](auto P, int rbuf, int rks, int q0) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int ch = (2 * rks + lh) ^ sw;
#pragma unroll
    for (int seg = 0; seg < 4; ++seg) {
#pragma unroll
      for (int f = 2 * seg; f < 2 * seg + 2; ++f) {
        if (f < T::FM) af[p ^ 1][f] = lds[rbuf + a_base + f * 32 * CPR + ch];
        else bfr[p ^ 1][f - T::FM] = lds[rbuf + b_base + (f - T::FM) * 32 * CPR + ch];
      }
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[seg][j] = mma(af[p][seg], bfr[p][j], acc[seg][j]);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (seg < LPS) load_one(q0 + seg);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  constexpr int pl = (KSTEPS - 1) & 1;  // fragment slot of the last step (1)
  using PL = std::integral_constant<int, pl>;

  // Output origin of this wave in the tile being computed, found before the
  // tile's main loop (scalar registers), so nothing but the epilogue itself
  // runs between the last MFMA and the stores.
  int out_row = 0, out_col = 0, cur_lin = 0, cur_kb = 0, cur_len = KT;
  auto set_out = [&](int i) {
    int tm, tn, split = 0;
    if constexpr (SK) {
      item(i, cur_lin, cur_kb, cur_len);
      grouped_coords(cur_lin, tiles_m, tiles_n, tm, tn, sk_gm);
      cur_len = __builtin_amdgcn_readfirstlane(cur_len);
    } else {
      walk.coords(i, tiles_m, tiles_n, splits, tm, tn, split);
    }
    out_row = __builtin_amdgcn_readfirstlane(split * tiles_m * BM + tm * BM + wm * T::WTM);
    out_col = __builtin_amdgcn_readfirstlane(tn * BN + wn * T::WTN);
  };
  auto store_tile = [&]() { epilogue<T, EPI>(g, acc, out_row, out_col); };
  // Stream-K: the end of a part of a tile cut between runs.  Parts and runs:
  // run v starts at slice floor(v S / G); the part of run v in this tile is
  // that run's first item (slot side 0) or, if the run starts in an earlier
  // tile, its last (side 1).  Each wave handles its own wave tile: unless the
  // counter already shows every other part arrived, it stores its part
  // (write-through stores, so another XCD's L2 cannot hold a stale copy),
  // waits for the stores, and counts its arrival; the wave that completes the
  // count (or found it complete) adds the parts in part order in the
  // epilogue and resets the counter.  No wave ever waits for another.
  auto sk_finish = [&]() {
    const int G = gridDim.x;
    auto run_of = [&](long s) { return (int)(((s + 1) * G + sk_S - 1) / sk_S - 1); };
    auto side_of = [&](int v) { return ((long)v * sk_S / G) / KTT == cur_lin ? 0 : 1; };
    constexpr int QF = T::WTM * T::WTN;
    auto part = [&](int v) { return g.sk_part + (((size_t)v * 2 + side_of(v)) * NW + wave) * QF; };
    const long t0 = (long)cur_lin * KTT;
    const int v_first = run_of(t0);
    const int parts = run_of(t0 + KTT - 1) - v_first + 1;
    const int me = sk_v - v_first;
    int* cnt = g.sk_cnt + (size_t)cur_lin * NW + wave;
    int seen = 0;
    if (lane == 0) seen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    seen = __builtin_amdgcn_readfirstlane(seen);
    bool last = seen == parts - 1;
    if (!last) {
      constexpr int kSC1 = 16;
      const __amdgpu_buffer_rsrc_t mine =
          __builtin_amdgcn_make_buffer_rsrc((void*)part(sk_v), (short)0, QF * 4, 0x00020000);
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const u32x4 d = {__float_as_uint(acc[i][j][4 * g4]), __float_as_uint(acc[i][j][4 * g4 + 1]),
                             __float_as_uint(acc[i][j][4 * g4 + 2]), __float_as_uint(acc[i][j][4 * g4 + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(d, mine, (((i * T::FN + j) * 4 + g4) * 64 + lane) * 16, 0, kSC1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      wait_vmcnt<0>();
      int old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = __builtin_amdgcn_readfirstlane(old) == parts - 1;
    }
    if (last) {
      const float* other[2] = {nullptr, nullptr};
      int k = 0;
      for (int p = 0; p < parts; ++p)
        if (p != me) other[k++] = part(v_first + p);
      epilogue<T, EPI, false, true>(g, acc, out_row, out_col, nullptr, other[0], other[1], me == 2);
      if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // Prologue: slices 0 .. STAGES-2, then the refill of the last buffer is
  // opened as if at a barrier (its first LPS loads now, the rest in the
  // first steps of slice 0), so every k step carries LPS loads.
  set_src(0);
#pragma unroll
  for (int s = 0; s + 1 < STAGES; ++s) {
    open_refill(s, ld_kt * BK);
#pragma unroll
    for (int q = 0; q < PER; ++q) load_one(q);
    advance_load();
  }
  open_refill(STAGES - 1, ld_kt * BK);
#pragma unroll
  for (int q = 0; q < LPS; ++q) load_one(q);
  wait_vmcnt<(STAGES - 2) * PER + LPS>();
  __syncthreads();
  // Nothing but LDS reads may be pending on lgkmcnt inside the loop (a pending
  // scalar load would force full waits), so settle the scalar loads here.
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  read_frags(0, 0, 0);

  int slot = 0;
  for (int ti = 0; ti < count; ++ti) {
    set_out(ti);
    for (int kt = 0; kt < (SK ? cur_len : KT); ++kt) {
      // Steps 0 .. KSTEPS-2.  The fragments of a step were read a whole step
      // earlier; waiting for them before issuing the next reads keeps at most
      // FM + FN reads outstanding (lgkmcnt only counts to 15) and costs
      // nothing.
#pragma unroll
      for (int ks = 0; ks + 1 < KSTEPS; ++ks) {
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
        if (ks & 1) step(P1{}, slot * STAGE, ks + 1, LPS * (ks + 1));
        else step(P0{}, slot * STAGE, ks + 1, LPS * (ks + 1));
      }
      advance_load();  // the open refill is complete
      // The next slice landed for this wave (STAGES-2 refills issued after
      // it), and after the barrier for every wave; everyone has read this
      // slice.
      wait_vmcnt<(STAGES - 2) * PER>();
      __syncthreads();
      const int next = slot + 1 == STAGES ? 0 : slot + 1;
      open_refill(slot, ld_kt * BK);
      // Last step, with the reads of the next slice's first fragments (the
      // ring streams across tiles, so that slice has landed).  At a tile end
      // they are read again after the epilogue, so nothing read here is
      // live across it.
      step(PL{}, next * STAGE, 0, 0);
      slot = next;
    }
    if constexpr (SK) {
      if (cur_kb == 0 && cur_len == KTT) store_tile();
      else sk_finish();
    } else {
      store_tile();
    }
    zero_acc();
    __builtin_amdgcn_sched_barrier(0);
    // First fragments of the next tile (after the last tile: unused).
    read_frags(slot * STAGE, 0, pl ^ 1);
  }
  // No load may still be writing LDS when the workgroup ends.
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
}


// ---------------------------------------------------------------------------
// Skinny products (M <= 128 rows, e.g. the blocks of a 96-token image):
// there is little MFMA work per weight byte, so the kernel is built to stream
// the weight panel once at full memory rate rather than to fill 256x256
// tiles (which would do up to 8x the MFMA work on padding rows).
//
// One workgroup per 128 output columns (a slab) and per K range; its rows are
// all of M, padded to MT fragments of 32.  Four waves: wave (wn, wk) owns
// output columns wn*64 .. wn*64+63 (two fragments, so each SwiGLU a/b pair of
// the packed in-projection stays in one wave) and the k steps of parity wk of
// every slice; the two K halves are added through LDS before the epilogue.
// 64-wide K slices of X (MT*32 rows, rows past M-1 clamped) and W (128 rows)
// go straight to LDS through a ring of four slots, three slices in flight
// (direct-to-LDS loads as inline assembly, as in the ring kernel; the waits
// and barriers below order them against the fragment reads).
// ---------------------------------------------------------------------------
template <int MT>
struct SkinnyTile {
  static constexpr int FM = MT, FN = 2;
};

// Epilogue of a q or k slab of the skinny in-projection with the head's
// RMSNorm and RoPE (the arithmetic of qk_norm_rope_kernel: the projection
// rounded to bf16, then x / sqrt(mean_128(x^2) + 1e-6) * scale, then each
// pair (2p, 2p+1) rotated by the token's table entry p, rounded to bf16).
// Wave (wn, 0) holds head columns 64 wn .. 64 wn + 63 of rows 32 i + lane % 32
// (four consecutive columns per register group, lane halves interleaved by
// four); its row sums of squares go to ss[wn][row] for the other wave.  All
// four waves call this (it holds a barrier); only wk == 0 stores.
template <int MT>
__device__ __forceinline__ void skinny_qk_norm_rope(const GemmArgs& g, floatx16 (&acc)[MT][2], int n0, int wn,
                                                    int wk, int lane, float* ss) {
  const int lr = lane & 31;
  const bool is_k = n0 >= kHidden;
  float part[MT];
  bf16x4 sc[2][4];
  float4 tb[MT][2][4];
  if (wk == 0) {
    // the scales of this lane's columns and the rotations of its rows (rows
    // past M-1 read row M-1's), loaded before the exchange so their latency
    // overlaps it
    const bf16* scale = (is_k ? g.qk_scale_k : g.qk_scale_q) + wn * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) sc[j][g4] = *(const bf16x4*)(scale + 32 * j + frag_col(g4, lane));
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const float* t = g.rope_table + (size_t)min(32 * i + lr, g.M - 1) * 128 + wn * 64;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) tb[i][j][g4] = *(const float4*)(t + 32 * j + frag_col(g4, lane));
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = to_f32(to_bf16(acc[i][j][r]));
          s += v * v;
        }
      part[i] = s + __shfl_xor(s, 32, 64);
      if (lane < 32) ss[wn * 32 * MT + 32 * i + lr] = part[i];
    }
  }
  __syncthreads();
  if (wk != 0) return;
  bf16* C = (bf16*)g.C;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = 32 * i + lr;
    if (row >= g.M) continue;
    const float tot = part[i] + ss[(wn ^ 1) * 32 * MT + 32 * i + lr];
    const float rn = 1.0f / sqrtf(tot * (1.0f / kHeadDim) + 1e-6f);
    bf16* crow = C + (size_t)row * g.ldc + n0 + wn * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = 32 * j + frag_col(g4, lane);  // column within this wave's 64
        const float4 t = tb[i][j][g4];              // (cos, sin) of pairs c/2, c/2 + 1
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_f32(to_bf16(acc[i][j][4 * g4 + e])) * rn * to_f32(sc[j][g4][e]);
        bf16x4 o;
        o[0] = to_bf16(v[0] * t.x - v[1] * t.y);
        o[1] = to_bf16(v[0] * t.y + v[1] * t.x);
        o[2] = to_bf16(v[2] * t.z - v[3] * t.w);
        o[3] = to_bf16(v[2] * t.w + v[3] * t.z);
        *(bf16x4*)(crow + c) = o;
      }
  }
}

template <int MT, GemmEpi EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g, int slabs, int ksplit) {
  using T = SkinnyTile<MT>;
  using Lay = Layout<64>;
  constexpr int CPR = Lay::CPR;            // 8 chunks of 16 bytes per row
  constexpr int MP = 32 * MT;              // X rows in LDS
  constexpr int BN = 128;                  // W rows (output columns) per slab
  constexpr int STAGES = 4;
  constexpr int STAGE = (MP + BN) * CPR;   // 16-byte chunks per slot
  constexpr int X_BLK = MP / Lay::RPB;     // KiB blocks of X per slice
  constexpr int BLK = X_BLK + BN / Lay::RPB;
  static_assert(BLK % 4 == 0, "a slice's blocks split evenly over the 4 waves");
  constexpr int PER = BLK / 4;             // loads per wave per slice
  static_assert((STAGES - 1) * PER < 64, "vmcnt range");
  static_assert(2 * MT * 2 * 16 * 64 * 4 + 2 * MP * 4 <= STAGES * STAGE * 16,
                "K-half reduction and the QK norm's row sums fit the ring");
  __shared__ bf16x8 lds[STAGES * STAGE];

  const int slab = blockIdx.x % slabs, split = blockIdx.x / slabs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wk = wave >> 1;
  const int n0 = slab * BN;
  // K range of this split: slices [kt0, kt0 + kt_per) of 64, the K / 64
  // slices cut as evenly as they go (ranges differ by at most one slice).
  const int kt_all = g.K / 64;
  const int kt0 = split * kt_all / ksplit;
  const int kt_per = (split + 1) * kt_all / ksplit - kt0;
  const size_t k0 = (size_t)kt0 * 64;

  // Block b of a slice: X rows 8b .. 8b+7 (b < X_BLK), else W rows; lane t
  // lands at row t/8, physical chunk t%8 of the block, so it fetches the
  // logical chunk that maps there.  Wave w issues blocks w*PER .. w*PER+PER-1.
  const char* xsrc = (const char*)(g.A + k0);
  const char* wsrc = (const char*)(g.B + (size_t)n0 * g.ldb + k0);
  const int sub_row = lane / CPR;
  unsigned voff[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = wave * PER + q;
    const int row = (b < X_BLK ? b : b - X_BLK) * Lay::RPB + sub_row;
    const int chunk = (lane % CPR) ^ Lay::swz(row);
    voff[q] = b < X_BLK ? (unsigned)((min(row, g.M - 1) * g.lda + chunk * 8) * 2)
                        : (unsigned)((row * g.ldb + chunk * 8) * 2);
  }
  const unsigned lds_base = (unsigned)(size_t)(lds_void_t*)lds;
  // Slice kt into slot `slot`; past the last slice the last one is loaded
  // again (into a slot no longer read), so every iteration has the same
  // number of loads in flight behind the slice it waits for.
  auto issue_slice = [&](int kt, int slot) __attribute__((always_inline)) {
    const int kc = min(kt, kt_per - 1) * 128;  // bytes
    const unsigned dst = lds_base + (unsigned)(slot * STAGE) * 16u;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int b = wave * PER + q;
      const char* src = (b < X_BLK ? xsrc : wsrc) + kc;
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff[q]), "s"(src), "s"(dst + (unsigned)b * 1024u) : "m0");
    }
  };

  floatx16 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int s = 0; s + 1 < STAGES; ++s) issue_slice(s, s);
  const int lr = lane & 31, lh = lane >> 5;
  const int sw = Lay::swz(lr);  // fragment rows are 32 f + lr
  for (int kt = 0; kt < kt_per; ++kt) {
    wait_vmcnt<(STAGES - 2) * PER>();  // slice kt landed
    __syncthreads();                   // ... for every wave; slice kt-1's slot is free
    issue_slice(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const int buf = (kt % STAGES) * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = (2 * (2 * h + wk) + lh) ^ sw;
      bf16x8 xf[MT], wf[2];
#pragma unroll
      for (int i = 0; i < MT; ++i) xf[i] = lds[buf + (32 * i + lr) * CPR + ch];
#pragma unroll
      for (int j = 0; j < 2; ++j) wf[j] = lds[buf + (MP + wn * 64 + 32 * j + lr) * CPR + ch];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma(xf[i], wf[j], acc[i][j]);
    }
  }
  wait_vmcnt<0>();  // the trailing reloads may still be writing the ring
  __syncthreads();

  // Add the odd-k half into the even-k waves, which run the epilogue.
  float* red = (float*)lds + (size_t)wn * (MT * 2 * 16 * 64);
  if (wk == 1) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((i * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
  }
  __syncthreads();
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * 2 + j) * 16 + r) * 64 + lane];
  }
  // A slab of the q or k columns is one head: its two epilogue waves (64
  // columns each) exchange each row's sum of squares through LDS, then store
  // the head normalised and rotated (workgroup-uniform branch).
  if constexpr (EPI == GemmEpi::kInProj) {
    if (g.rope_table != nullptr && n0 < 2 * kHidden) {
      skinny_qk_norm_rope<MT>(g, acc, n0, wn, wk, lane, (float*)lds + 2 * (MT * 2 * 16 * 64));
      return;
    }
  }
  if (wk == 0) {
    const int wrow0 = EPI == GemmEpi::kSplitPartial ? split * MP : 0;
    epilogue<T, EPI>(g, acc, wrow0, n0 + wn * 64);
  }
}

}  // namespace gemm
}  // namespace flux3
