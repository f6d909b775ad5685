// bf16 MFMA GEMM  C = A B^T  for every projection of the block and stack, with
// fused epilogues:
//   - q|k|v store + SwiGLU (silu(a) * b of the interleaved mlp_in rows), for
//     the block's input projections ("Welcome FLUX.3 Image Klein in
//     Diffusers", §Inside one block: attention and MLP run in parallel on the
//     same modulated input; SwiGLU from "[Feature] FLUX.3 Image Klein support
//     #2142", comment §Structure (from dit.py));
//   - x + gate * (attn_out(o) + mlp_out(h)) as one product over [o | h], for
//     the block's output (same sections: gated residual).
// The kernels themselves are in gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace flux3 {

namespace {

template <int BM, int BN, int WM, int WN>
void run_regs(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  hipLaunchKernelGGL((gemm::gemm_regs_kernel<BM, BN, WM, WN>), dim3(tiles_m * tiles_n),
                     dim3(WM * WN * 64), 0, st, g, tiles_m, tiles_n);
}

template <int BM, int BN, int WM, int WN, int BK, int ST, int WPE>
void run_ring(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  hipLaunchKernelGGL((gemm::gemm_ring_kernel<BM, BN, WM, WN, BK, ST, WPE>), dim3(tiles_m * tiles_n),
                     dim3(WM * WN * 64), 0, st, g, tiles_m, tiles_n);
}

}  // namespace

// Tile choice: 256x256 (8 waves, 128x64 per wave) when the grid still has at
// least one tile per CU; otherwise 128x128 (4 waves, 64x64 per wave); 64-wide
// outputs use 64x64 tiles.  The host has checked K % 64 == 0 and N % 64 == 0.
void launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0) return;
  const long big_tiles = (long)((g.M + 255) / 256) * (g.N / 256);
  if (g.N % 256 == 0 && big_tiles >= 192) {
    run_ring<256, 256, 2, 2, 64, 2, 1>(g, st);
  } else if (g.N % 128 == 0) {
    run_regs<128, 128, 2, 2>(g, st);
  } else {
    run_regs<64, 64, 2, 1>(g, st);
  }
}

// Variant entry used by the tile-shape sweep: cfg selects one instantiation.
int launch_gemm_variant(const GemmArgs& g, int cfg, hipStream_t st) {
  switch (cfg) {
    case 0: run_regs<256, 256, 2, 4>(g, st); return 0;
    case 1: run_regs<128, 128, 2, 2>(g, st); return 0;
    case 2: run_ring<256, 256, 2, 2, 32, 4, 1>(g, st); return 0;
    case 3: run_ring<256, 256, 2, 2, 32, 3, 1>(g, st); return 0;
    case 4: run_ring<128, 256, 2, 2, 32, 3, 2>(g, st); return 0;
    case 5: run_ring<256, 128, 2, 2, 32, 3, 2>(g, st); return 0;
    case 6: run_ring<128, 128, 2, 2, 32, 4, 2>(g, st); return 0;
    case 7: run_ring<256, 128, 2, 2, 64, 3, 1>(g, st); return 0;
    case 8: run_ring<128, 256, 2, 2, 64, 3, 1>(g, st); return 0;
    case 9: run_ring<256, 256, 2, 2, 64, 2, 1>(g, st); return 0;
    case 10: run_ring<256, 128, 2, 2, 64, 2, 2>(g, st); return 0;
    default: return -1;
  }
}

}  // namespace flux3
