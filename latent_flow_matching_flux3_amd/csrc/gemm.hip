// bf16 MFMA GEMM  C = A B^T  for every projection of the block and stack, with
// fused epilogues:
//   - q|k|v store + SwiGLU (silu(a) * b of the interleaved mlp_in rows), for
//     the block's input projections ("Welcome FLUX.3 Image Klein in
//     Diffusers", §Inside one block: attention and MLP run in parallel on the
//     same modulated input; SwiGLU from "[Feature] FLUX.3 Image Klein support
//     #2142", comment §Structure (from dit.py));
//   - x + gate * (attn_out(o) + mlp_out(h)) as one product over [o | h], for
//     the block's output (same sections: gated residual).
//
// Design (gfx950): v_mfma_f32_32x32x16_bf16 on 64-wide waves.  A and B are
// both K-contiguous, so each lane feeds the MFMA with one 16-byte LDS read per
// operand per 16-wide k step.  K is walked in 64-wide slices through two LDS
// buffers (register-staged global prefetch of the next slice while the MFMAs
// run on the current one, one barrier per slice).  LDS rows are 128 bytes; the
// 16-byte chunk index is XOR-swizzled with (row & 7) so the MFMA operand reads
// and the staging writes are bank-conflict free.  Tiles are assigned so that
// each XCD (own L2) works on a contiguous band of the tile grid, walked in
// groups of 4 tile rows so concurrently running tiles share A and B slices.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int kBK = 64;

// Output coordinates of accumulator element r of a 32x32 fragment, lane l:
//   col = l % 32, row = 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ int frag_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
  static constexpr int ACH = BM * 8 / NT;  // 16-byte chunks of A per thread per slice
  static constexpr int BCH = BN * 8 / NT;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 fragments");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "slice must split evenly");
};

template <class T>
__device__ __forceinline__ void epilogue(const GemmArgs& g, floatx16 (&acc)[T::FM][T::FN],
                                         int wrow0, int wcol0, int lane) {
  const int lc = lane & 31;
  switch (g.epi) {
    case GemmEpi::kStoreBf16:
    case GemmEpi::kInProj: {
      if (g.epi == GemmEpi::kStoreBf16 || wcol0 < 3 * kHidden) {
        bf16* C = (bf16*)g.C;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wrow0 + 32 * i + frag_row(r, lane);
            if (row < g.M) {
#pragma unroll
              for (int j = 0; j < T::FN; ++j)
                C[(size_t)row * g.ldc + wcol0 + 32 * j + lc] = to_bf16(acc[i][j][r]);
            }
          }
      } else {
        // SwiGLU: fragment 2p holds a-columns, 2p+1 the matching b-columns.
        static_assert(T::FN % 2 == 0, "SwiGLU needs fragment pairs");
        const int hcol0 = (wcol0 - 3 * kHidden) / 2;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wrow0 + 32 * i + frag_row(r, lane);
            if (row < g.M) {
#pragma unroll
              for (int p = 0; p < T::FN / 2; ++p) {
                const float a = acc[i][2 * p][r], b = acc[i][2 * p + 1][r];
                g.H[(size_t)row * g.ldh + hcol0 + 32 * p + lc] = to_bf16(silu_f(a) * b);
              }
            }
          }
      }
      break;
    }
    case GemmEpi::kStoreF32: {
      float* C = (float*)g.C;
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wrow0 + 32 * i + frag_row(r, lane);
          if (row < g.M) {
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
              C[(size_t)row * g.ldc + wcol0 + 32 * j + lc] = acc[i][j][r];
          }
        }
      break;
    }
    case GemmEpi::kGatedResidual: {
      float* X = (float*)g.C;
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wrow0 + 32 * i + frag_row(r, lane);
          if (row < g.M) {
            const float* gate = g.mod + (size_t)seg_of_row(g.seg, row) * g.mod_stride + g.gate_offset;
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
              const int col = wcol0 + 32 * j + lc;
              float* px = X + (size_t)row * g.ldc + col;
              *px = *px + gate[col] * acc[i][j][r];
            }
          }
        }
      break;
    }
  }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(GemmArgs g, int tiles_m,
                                                              int tiles_n) {
  using T = Tile<BM, BN, WM, WN>;
  __shared__ bf16x8 lds[2 * (BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Tile order: XCD-contiguous bands, then groups of 4 tile rows.
  const int total = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  constexpr int GM = 4;
  const int group = lin / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = lin - group * GM * tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  // Global -> register staging addresses (rows of A clamped to M-1).
  const bf16* a_src[T::ACH];
  int a_lds[T::ACH];
#pragma unroll
  for (int i = 0; i < T::ACH; ++i) {
    const int id = tid + i * T::NT;
    const int row = id >> 3, c = id & 7;
    const int grow = min(m0 + row, g.M - 1);
    a_src[i] = g.A + (size_t)grow * g.lda + c * 8;
    a_lds[i] = row * 8 + (c ^ (row & 7));
  }
  const bf16* b_src[T::BCH];
  int b_lds[T::BCH];
#pragma unroll
  for (int i = 0; i < T::BCH; ++i) {
    const int id = tid + i * T::NT;
    const int row = id >> 3, c = id & 7;
    b_src[i] = g.B + (size_t)(n0 + row) * g.ldb + c * 8;
    b_lds[i] = BM * 8 + row * 8 + (c ^ (row & 7));
  }

  floatx16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 ra[T::ACH], rb[T::BCH];
#pragma unroll
  for (int i = 0; i < T::ACH; ++i) ra[i] = *(const bf16x8*)a_src[i];
#pragma unroll
  for (int i = 0; i < T::BCH; ++i) rb[i] = *(const bf16x8*)b_src[i];
#pragma unroll
  for (int i = 0; i < T::ACH; ++i) lds[a_lds[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < T::BCH; ++i) lds[b_lds[i]] = rb[i];
  __syncthreads();

  // Operand read offsets (chunk units) inside one buffer.
  const int lr = lane & 31, lh = lane >> 5;
  int a_off[T::FM], b_off[T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i) a_off[i] = (wm * T::WTM + 32 * i + lr) * 8;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) b_off[j] = BM * 8 + (wn * T::WTN + 32 * j + lr) * 8;
  const int sw = lr & 7;  // (row & 7) of every operand row this lane reads

  const int KT = g.K / kBK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = (kt & 1) * (BM + BN) * 8;
    if (kt + 1 < KT) {
      const int koff = (kt + 1) * kBK;
#pragma unroll
      for (int i = 0; i < T::ACH; ++i) ra[i] = *(const bf16x8*)(a_src[i] + koff);
#pragma unroll
      for (int i = 0; i < T::BCH; ++i) rb[i] = *(const bf16x8*)(b_src[i] + koff);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
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
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      const int nxt = ((kt + 1) & 1) * (BM + BN) * 8;
#pragma unroll
      for (int i = 0; i < T::ACH; ++i) lds[nxt + a_lds[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < T::BCH; ++i) lds[nxt + b_lds[i]] = rb[i];
    }
    __syncthreads();
  }

  epilogue<T>(g, acc, m0 + wm * T::WTM, n0 + wn * T::WTN, lane);
}

template <int BM, int BN, int WM, int WN>
void run(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WM, WN>), dim3(tiles_m * tiles_n),
                     dim3(WM * WN * 64), 0, st, g, tiles_m, tiles_n);
}

}  // namespace

// Tile choice: 256x256 (8 waves, 128x64 per wave) when the grid still has at
// least one tile per CU; otherwise 128x128 (4 waves, 64x64 per wave); 64-wide
// outputs use 64x64 tiles.  The host has checked K % 64 == 0 and N % 64 == 0.
void launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0) return;
  const long big_tiles = (long)((g.M + 255) / 256) * (g.N / 256);
  if (g.N % 256 == 0 && big_tiles >= 256) {
    run<256, 256, 2, 4>(g, st);
  } else if (g.N % 128 == 0) {
    run<128, 128, 2, 2>(g, st);
  } else {
    run<64, 64, 2, 1>(g, st);
  }
}

}  // namespace flux3
