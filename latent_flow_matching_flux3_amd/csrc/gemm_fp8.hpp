// fp8 (OCP E4M3) persistent ring GEMM  C = (A B^T) * a_scale[row] * w_scale[col],
// the rowwise FP8 product of the block's two large projections
// ("Welcome FLUX.3 Image Klein in Diffusers", §Base model and quantized
// variants: the transformer also ships as fp8r, rowwise FP8).
//
// Same structure as the bf16 ring kernel (gemm_kernels.hpp): 256x256 tiles,
// 4 waves with 128x128 fp32 accumulators, one workgroup per CU walking its
// tiles, K slices streamed through an LDS ring by direct-to-LDS loads issued
// as inline assembly.  A K slice is 64 fp8 values = 64 bytes per row, the byte
// geometry of the bf16 kernel's 32-wide slices (same swizzle and loads), and
// it is one MFMA k step: v_mfma_scale_f32_32x32x64_f8f6f4 with unit (E8M0
// 127) block scales, i.e. a plain E4M3 product.  A lane supplies 32 bytes of
// its row: lane half h holds k = 32 h .. 32 h + 31 of the slice, the same
// bytes of A and B (the instruction pairs byte i of an A lane with byte i of
// the B lane of the same half, so any k order shared by both works).
//
// Ring: STAGES slices; the barrier before slice t's k step finds slice t+1
// landed and every wave done reading slice t (its fragments were read during
// the step of slice t-1), so that step refills slice t's buffer with slice
// t+STAGES, one load after every second MFMA.  Fragments alternate between
// two register sets slice by slice, so a work item has an even number of
// slices (K a multiple of 128).
//
// Scales: at a tile's start every wave loads its 128 row scales and 128
// column scales into its own LDS area by three direct-to-LDS loads (the row
// indices clamped to M-1); the ring's waits have retired them long before
// the epilogue, which reads them with LDS loads (a global load there would
// wait for every store in flight).
//
// Two Linears side by side along K (k_part > 0: the block's [o | h] against
// [attn_out | mlp_out], each Linear with its own row and column scales): a
// work item whose K range lies in one Linear takes that Linear's scales; one
// that spans both also loads the ratios of the first Linear's scales to the
// second's, and when its k steps reach k_part it multiplies the accumulators
// (the first Linear's unscaled products so far) by row ratio x column ratio,
// which brings them to the second Linear's scales, applied in the epilogue.
#pragma once

#include "gemm_kernels.hpp"

namespace flux3 {
namespace gemm {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int intx8;

__device__ __forceinline__ floatx16 mma_fp8(const intx8& x_frag, const intx8& w_frag, floatx16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w_frag, x_frag, acc, 0, 0, 0, 127, 0, 127);
}

template <int STAGES, GemmEpi EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_ring_fp8_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 2, BKB = 64;  // BKB: fp8 values (bytes) per slice row
  using T = Tile<BM, BN, WM, WN>;
  using Lay = Layout<32>;                 // 64-byte rows
  constexpr int NW = WM * WN;
  constexpr int CPR = Lay::CPR;           // 4 chunks of 16 bytes per row
  constexpr int STAGE = (BM + BN) * CPR;  // chunks per buffer (32 KiB)
  constexpr int A_BLK = BM / Lay::RPB / NW, B_BLK = BN / Lay::RPB / NW;
  constexpr int PER = A_BLK + B_BLK;      // loads per wave per slice (8)
  // Per-wave scale area (floats): [0, 128) row scales, [128, 384) column
  // scales (+ the copy the 64-lane load writes), [384, 512) row ratios,
  // [512, 768) column ratios (+ copy): 3 KiB.
  constexpr int SC_CHUNKS = 192;
  static_assert(T::FM == 4 && T::FN == 4 && PER == 8, "tile geometry");
  static_assert(STAGES >= 3 && (STAGES - 2) * PER + 6 < 64, "ring depth");
  __shared__ bf16x8 lds[STAGES * STAGE + NW * SC_CHUNKS];

  const int splits = EPI == GemmEpi::kSplitPartial ? g.ksplit : 1;
  const TileWalk walk(tiles_m * tiles_n * splits);
  if (walk.count == 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int sub_row = lane / CPR;

  unsigned voff_a[A_BLK], voff_b[B_BLK];
#pragma unroll
  for (int q = 0; q < B_BLK; ++q) {
    const int row = (wave * B_BLK + q) * Lay::RPB + sub_row;
    voff_b[q] = (unsigned)(row * g.ldb + ((lane % CPR) ^ Lay::swz(row)) * 16);
  }
  const char* a_tile;
  const char* b_tile;
  const int KT = g.K / BKB / splits;  // slices per work item: even, >= STAGES
  auto set_src = [&](int i) {
    int tm, tn, split;
    walk.coords(i, tiles_m, tiles_n, splits, tm, tn, split);
    const int m0 = tm * BM;
    const size_t k0 = (size_t)split * KT * BKB;
    a_tile = (const char*)(g.A8 + (size_t)m0 * g.lda + k0);
    b_tile = (const char*)(g.B8 + (size_t)tn * BN * g.ldb + k0);
#pragma unroll
    for (int q = 0; q < A_BLK; ++q) {
      const int row = (wave * A_BLK + q) * Lay::RPB + sub_row;
      voff_a[q] = (unsigned)((min(m0 + row, g.M - 1) - m0) * g.lda + ((lane % CPR) ^ Lay::swz(row)) * 16);
    }
  };
  const unsigned lds_base = (unsigned)(size_t)(lds_void_t*)lds;
  const char* r_a = nullptr;
  const char* r_b = nullptr;
  unsigned r_dst = 0;
  auto open_refill = [&](int slot, int koff) {
    r_a = a_tile + koff;
    r_b = b_tile + koff;
    r_dst = lds_base + (unsigned)(slot * STAGE) * 16u;
  };
  // One KiB of the open refill into LDS (m0 = destination; one wait state
  // between writing m0 and the load reading it).
  auto load_one = [&](int q) __attribute__((always_inline)) {
    const bool is_a = q < A_BLK;
    const int blk = is_a ? wave * A_BLK + q : BM / Lay::RPB + wave * B_BLK + (q - A_BLK);
    const unsigned dst = r_dst + (unsigned)blk * 1024u;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(is_a ? voff_a[q] : voff_b[q - A_BLK]), "s"(is_a ? r_a : r_b), "s"(dst)
                 : "m0");
  };
  int ld_i = 0, ld_kt = 0;
  auto advance_load = [&]() {
    if (++ld_kt == KT) {
      if (ld_i + 1 < walk.count) {
        ++ld_i;
        ld_kt = 0;
        set_src(ld_i);
      } else {
        ld_kt = KT - 1;
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

  // Fragment reads: row lr of fragment f, chunks 2 lh and 2 lh + 1.
  const int lr = lane & 31, lh = lane >> 5;
  const int sw = Lay::swz(lr);
  const int c0 = (2 * lh) ^ sw, c1 = (2 * lh + 1) ^ sw;
  const int a_base = (wm * T::WTM + lr) * CPR;
  const int b_base = BM * CPR + (wn * T::WTN + lr) * CPR;
  intx8 af[2][T::FM], bfr[2][T::FN];
  auto read_frag = [&](int buf, int f, int p) __attribute__((always_inline)) {
    const int row = f < T::FM ? buf + a_base + f * 32 * CPR : buf + b_base + (f - T::FM) * 32 * CPR;
    const bf16x8 lo = lds[row + c0], hi = lds[row + c1];
    const intx8 v = __builtin_bit_cast(
        intx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
    if (f < T::FM) af[p][f] = v;
    else bfr[p][f - T::FM] = v;
  };
  // The k step of one slice: its 16 MFMAs (fragments P) in four segments of
  // four; each segment reads two fragments of the next slice (buffer rbuf,
  // into 1-P) and issues two loads of the open refill, each after an MFMA.
  auto step = [&](auto P, int rbuf) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int seg = 0; seg < 4; ++seg) {
      read_frag(rbuf, seg, p ^ 1);
      read_frag(rbuf, T::FM + seg, p ^ 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[seg][j] = mma_fp8(af[p][seg], bfr[p][j], acc[seg][j]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_barrier(0);
      load_one(2 * seg);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 2; j < 4; ++j) acc[seg][j] = mma_fp8(af[p][seg], bfr[p][j], acc[seg][j]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_one(2 * seg + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Output origin of the tile being computed, and its scales into this
  // wave's LDS area: rows (clamped to M-1) by two 4-byte loads, columns by
  // one 16-byte load (lanes 32..63 repeat lanes 0..31 into unused bytes).
  // rescale_at: the k step (even) at which the accumulators move from the
  // first Linear's scales to the second's, or -1.
  int out_row = 0, out_col = 0, rescale_at = -1;
  const unsigned sc_lds = lds_base + (unsigned)(STAGES * STAGE + wave * SC_CHUNKS) * 16u;
  auto set_out = [&](int i) {
    int tm, tn, split;
    walk.coords(i, tiles_m, tiles_n, splits, tm, tn, split);
    const int r0 = tm * BM + wm * T::WTM;
    out_row = __builtin_amdgcn_readfirstlane(split * tiles_m * BM + r0);
    out_col = __builtin_amdgcn_readfirstlane(tn * BN + wn * T::WTN);
    const unsigned ra = 4u * (unsigned)min(r0 + lane, g.M - 1);
    const unsigned rb = 4u * (unsigned)min(r0 + 64 + lane, g.M - 1);
    const unsigned cw = 16u * (unsigned)(lane & 31);
    const int k_begin = __builtin_amdgcn_readfirstlane(split * KT * BKB);
    const bool first_only = g.k_part > 0 && k_begin + KT * BKB <= g.k_part;
    const bool spans = g.k_part > k_begin && k_begin + KT * BKB > g.k_part;
    rescale_at = spans ? (g.k_part - k_begin) / BKB : -1;
    const float* as = first_only ? g.a_scale0 : g.a_scale;
    const float* ws = (first_only ? g.w_scale0 : g.w_scale) + out_col;
    asm volatile(
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %0, %4\n\t"
        "s_add_u32 m0, %3, 256\n\ts_nop 0\n\tglobal_load_lds_dword %1, %4\n\t"
        "s_add_u32 m0, %3, 512\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %5"
        :: "v"(ra), "v"(rb), "v"(cw), "s"(sc_lds), "s"(as), "s"(ws)
        : "m0");
    if (spans) {
      const float* wr = g.w_ratio + out_col;
      asm volatile(
          "s_add_u32 m0, %3, 1536\n\ts_nop 0\n\tglobal_load_lds_dword %0, %4\n\t"
          "s_add_u32 m0, %3, 1792\n\ts_nop 0\n\tglobal_load_lds_dword %1, %4\n\t"
          "s_add_u32 m0, %3, 2048\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %5"
          :: "v"(ra), "v"(rb), "v"(cw), "s"(sc_lds), "s"(g.a_ratio), "s"(wr)
          : "m0");
    }
  };
  const float* sc = (const float*)(lds + STAGES * STAGE + wave * SC_CHUNKS);
  auto store_tile = [&]() { epilogue<T, EPI, true>(g, acc, out_row, out_col, sc); };
  // The first Linear's products so far, brought to the second's scales
  // (element r of fragment (i, j): row 32 i + lane % 32, column
  // 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4 of the wave tile).  Each
  // accumulator register is read, scaled and written back in place, so the
  // accumulators never leave their registers.
  auto rescale = [&]() {
    const int lr = lane & 31;
    // the last k step's MFMAs may still be writing these registers: wait
    // out the longest MFMA-write to VALU-read distance before the first read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const float ra = sc[384 + 32 * i + lr];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 wr = *(const float4*)(sc + 512 + 32 * j + frag_col(g4, lane));
          const float f[4] = {ra * wr.x, ra * wr.y, ra * wr.z, ra * wr.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(acc[i][j][4 * g4 + e]), "=&v"(t) : "v"(f[e]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Prologue: slices 0 .. STAGES-1 in flight, wait for slice 0.
  set_src(0);
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    open_refill(s, ld_kt * BKB);
#pragma unroll
    for (int q = 0; q < PER; ++q) load_one(q);
    advance_load();
  }
  wait_vmcnt<(STAGES - 1) * PER>();
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
#pragma unroll
  for (int f = 0; f < T::FM + T::FN; ++f) read_frag(0, f, 0);

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int slot = 0;
  // Slice t: wait until slice t+1 landed (STAGES-2 refills, and any scale
  // loads, issued after it), barrier; refill slice t's buffer with slice
  // t + STAGES during the k step, which also reads slice t+1's fragments.
  auto slice = [&](auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    wait_vmcnt<(STAGES - 2) * PER>();
    __syncthreads();
    // The fragments pass through empty asm after the barrier, so the step's
    // MFMAs stay after it (register-only instructions may otherwise be
    // hoisted across the barrier and the cursor's branch).
#pragma unroll
    for (int f = 0; f < T::FM; ++f) {
      asm volatile("" : "+v"(af[p][f]));
      asm volatile("" : "+v"(bfr[p][f]));
    }
    const int next = slot + 1 == STAGES ? 0 : slot + 1;
    open_refill(slot, ld_kt * BKB);
    step(P, next * STAGE);
    // ... and the accumulators pass through empty asm after it, so they do
    // not sink past the cursor's branch and the next barrier either.
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) asm volatile("" : "+a"(acc[i][j]));
    // Only now: moving to the next tile replaces the A lane offsets the
    // refill's loads use.
    advance_load();
    slot = next;
  };
  for (int ti = 0; ti < walk.count; ++ti) {
    set_out(ti);
    for (int kt = 0; kt < KT; kt += 2) {
      if (kt == rescale_at) rescale();
      slice(P0{});
      slice(P1{});
    }
    store_tile();
    zero_acc();
    __builtin_amdgcn_sched_barrier(0);
    // First fragments of the next tile (read again: those read in the last
    // step are not kept live across the epilogue).
#pragma unroll
    for (int f = 0; f < T::FM + T::FN; ++f) read_frag(slot * STAGE, f, 0);
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

}  // namespace gemm
}  // namespace flux3
