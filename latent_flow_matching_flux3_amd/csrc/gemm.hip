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
#include "gemm_fp8.hpp"

#include <algorithm>

namespace flux3 {

namespace {

template <int BM, int BN, int WM, int WN>
void run_regs(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  hipLaunchKernelGGL((gemm::gemm_regs_kernel<BM, BN, WM, WN>), dim3(tiles_m * tiles_n),
                     dim3(WM * WN * 64), 0, st, g, tiles_m, tiles_n);
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Persistent launch: one workgroup per CU (WPE workgroups per CU when the
// ring leaves room), never more workgroups than tiles; one kernel per
// epilogue kind.
template <int BM, int BN, int WM, int WN, int BK, int ST, int WPE, GemmEpi EPI>
void launch_ring(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  const int total = tiles_m * tiles_n;
  const int items = total * (EPI == GemmEpi::kSplitPartial ? g.ksplit : 1);
  const int grid = std::min(items, cu_count() * WPE);
  hipLaunchKernelGGL((gemm::gemm_ring_kernel<BM, BN, WM, WN, BK, ST, WPE, EPI>), dim3(grid),
                     dim3(WM * WN * 64), 0, st, g, tiles_m, tiles_n);
}

template <int BM, int BN, int WM, int WN, int BK, int ST, int WPE>
void run_ring(const GemmArgs& g, hipStream_t st) {
  switch (g.epi) {
    case GemmEpi::kStoreBf16: launch_ring<BM, BN, WM, WN, BK, ST, WPE, GemmEpi::kStoreBf16>(g, st); break;
    case GemmEpi::kStoreF32: launch_ring<BM, BN, WM, WN, BK, ST, WPE, GemmEpi::kStoreF32>(g, st); break;
    case GemmEpi::kInProj: launch_ring<BM, BN, WM, WN, BK, ST, WPE, GemmEpi::kInProj>(g, st); break;
    case GemmEpi::kGatedResidual: launch_ring<BM, BN, WM, WN, BK, ST, WPE, GemmEpi::kGatedResidual>(g, st); break;
    case GemmEpi::kSplitPartial:
      launch_ring<BM, BN, WM, WN, BK, ST, WPE, GemmEpi::kSplitPartial>(g, st);
      break;
  }
}

// Most K ranges a split product takes (the reduce holds one load per range
// in flight).
constexpr int kMaxReduceSplits = 24;

// K ranges for a split product on 256x256 tiles: the largest
// divisor s of K/32 with s * tiles <= CUs, s <= kMaxReduceSplits and ranges of
// at least 16 slices of 32; 1 when the product already has 128 tiles or more.
int split_count(int m, int n, int k) {
  if (n % 256 != 0 || k % 32 != 0) return 1;
  const long tiles = (long)((m + 255) / 256) * (n / 256);
  if (tiles >= 128) return 1;
  const int kt = k / 32;
  int best = 1;
  for (int s = 2; s <= kt / 16 && s <= kMaxReduceSplits; ++s)
    if (kt % s == 0 && tiles * s <= cu_count()) best = s;
  return best;
}

size_t split_bytes(int m, int n, int s) { return (size_t)s * ((m + 255) / 256) * 256 * n * 4; }

// Stream-K on 256x256 tiles (gated residual): used where the whole tiles
// leave part of the last round of workgroups idle and every run of K slices
// is at least half a tile (so a tile has at most three parts), and the
// longest workgroup's work shrinks by at least 5%: the output projection at
// 4608 rows (216 tiles of 384 slices on 256 CUs: 324 slices per workgroup
// against 384) or 4096 rows (192 tiles: 288 against 384).
constexpr int kSkGroupM = 6;                    // tile rows per group of the tile order
constexpr int kSkWaves = 4;                     // waves per workgroup (2 x 2)
constexpr size_t kSkPartBytes = 128 * 128 * 4;  // one wave tile, fp32

bool sk_plan(int m, int n, int k, long& tiles) {
  if (m <= 0 || n % 256 != 0 || k % 32 != 0) return false;
  tiles = (long)((m + 255) / 256) * (n / 256);
  const long G = cu_count(), kt = k / 32, S = tiles * kt;
  if (tiles % G == 0 || 2 * S < G * kt) return false;
  const long rounds = (tiles + G - 1) / G;
  return rounds * kt * G * 100 >= S * 105;
}

// Skinny products (M <= 128): the weight-streaming kernel, split over K when
// its slabs alone (N / 128 workgroups) leave most CUs idle and the caller lent
// scratch (gated residual and fp32 products).
bool skinny_shape(int m, int n, int k) { return m > 0 && m <= 128 && n % 128 == 0 && k % 64 == 0; }

int skinny_split(int n, int k) {
  // K ranges need not divide K / 64 evenly (the kernel splits it as evenly as
  // it goes), so the split fills the CUs: the output projection at <= 128 rows
  // (24 slabs) takes 10 ranges of 19 or 20 slices instead of 8 of 24.
  const int slabs = n / 128, kt = k / 64;
  return std::max(1, std::min({16, cu_count() / slabs, kt / 4}));
}

size_t skinny_split_bytes(int m, int n, int d) { return (size_t)d * ((m + 31) / 32) * 32 * n * 4; }

// Sum of the K-range partials, four columns per thread: gated (mod != null)
// x[r][c] += gate[seg(r)][c] * sum_s part[s][r][c], else x[r][c] = sum.
__global__ __launch_bounds__(256) void split_reduce_kernel(float* x, int ldx, const float* part,
                                                           size_t stride, int splits, int m, int n,
                                                           const float* mod, int mod_stride,
                                                           int gate_offset, SegTable seg) {
  const int quads = n / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)m * quads) return;
  const int r = (int)(idx / quads), c = (int)(idx % quads) * 4;
  const float* p = part + (size_t)r * n + c;
  // every partial's load in flight at once, then the sum in split order
  float4 t[kMaxReduceSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxReduceSplits; ++sp)
    if (sp < splits) t[sp] = *(const float4*)(p + sp * stride);
  float4 acc = t[0];
#pragma unroll
  for (int sp = 1; sp < kMaxReduceSplits; ++sp)
    if (sp < splits) {
      acc.x += t[sp].x;
      acc.y += t[sp].y;
      acc.z += t[sp].z;
      acc.w += t[sp].w;
    }
  float4* xp = (float4*)(x + (size_t)r * ldx + c);
  if (mod == nullptr) {
    *xp = acc;
    return;
  }
  const float4 gt = *(const float4*)(mod + (size_t)seg_of_row(seg, r) * mod_stride + gate_offset + c);
  float4 xv = *xp;
  xv.x += gt.x * acc.x;
  xv.y += gt.y * acc.y;
  xv.z += gt.z * acc.z;
  xv.w += gt.w * acc.w;
  *xp = xv;
}

// The reduce of a skinny split product (N = 3072) with the next block's
// LayerNorm + modulation: one workgroup per row, thread t owns columns
// 4 (t + 256 i), i < 3.  The sum of the partials and the gated residual are
// those of split_reduce_kernel; the LayerNorm is the exact two-pass form of
// ln_modulate_kernel (mean, then mean((x - mu)^2), eps 1e-6, in fp32), its
// row sums formed per wave and then over the four waves.
__global__ __launch_bounds__(256) void split_reduce_ln_kernel(float* x, int ldx, const float* part,
                                                              size_t stride, int splits,
                                                              const float* mod, int mod_stride,
                                                              int gate_offset, SegTable seg, bf16* xm,
                                                              int ldxm) {
  __shared__ float red[2][4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* shift = mod + (size_t)seg_of_row(seg, row) * mod_stride;
  float v[3][4];
  float s = 0.f;
  // every partial's load in flight at once (splits <= 16 on this path), then
  // the sums in split order
  float4 t[3][16];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int sp = 0; sp < 16; ++sp)
      if (sp < splits) t[i][sp] = *(const float4*)(part + (size_t)row * kHidden + (tid + 256 * i) * 4 + sp * stride);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = (tid + 256 * i) * 4;
    float4 acc = t[i][0];
#pragma unroll
    for (int sp = 1; sp < 16; ++sp)
      if (sp < splits) {
        acc.x += t[i][sp].x;
        acc.y += t[i][sp].y;
        acc.z += t[i][sp].z;
        acc.w += t[i][sp].w;
      }
    const float4 gt = *(const float4*)(shift + gate_offset + c);
    float4* xp = (float4*)(x + (size_t)row * ldx + c);
    float4 xv = *xp;
    xv.x += gt.x * acc.x;
    xv.y += gt.y * acc.y;
    xv.z += gt.z * acc.z;
    xv.w += gt.w * acc.w;
    *xp = xv;
    v[i][0] = xv.x;
    v[i][1] = xv.y;
    v[i][2] = xv.z;
    v[i][3] = xv.w;
    s += (xv.x + xv.y) + (xv.z + xv.w);
  }
  s = wave_sum(s);
  if (lane == 0) red[0][wave] = s;
  __syncthreads();
  const float mu = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) * (1.0f / kHidden);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = v[i][e] - mu;
      q += d * d;
    }
  q = wave_sum(q);
  if (lane == 0) red[1][wave] = q;
  __syncthreads();
  const float var = ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) * (1.0f / kHidden);
  const float rstd = 1.0f / sqrtf(var + 1e-6f);
  const float* scale = shift + kHidden;
  bf16* orow = xm + (size_t)row * ldxm;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = (tid + 256 * i) * 4;
    const float4 sh = *(const float4*)(shift + c), sc = *(const float4*)(scale + c);
    bf16x4 o;
    o[0] = to_bf16((1.0f + sc.x) * ((v[i][0] - mu) * rstd) + sh.x);
    o[1] = to_bf16((1.0f + sc.y) * ((v[i][1] - mu) * rstd) + sh.y);
    o[2] = to_bf16((1.0f + sc.z) * ((v[i][2] - mu) * rstd) + sh.z);
    o[3] = to_bf16((1.0f + sc.w) * ((v[i][3] - mu) * rstd) + sh.w);
    *(bf16x4*)(orow + c) = o;
  }
}

// fp8 products: the persistent ring kernel with 4 slices of 64 fp8 in flight.
constexpr int kFp8Stages = 4;

template <GemmEpi EPI>
void launch_ring_fp8(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (g.M + 255) / 256;
  const int tiles_n = g.N / 256;
  const int items = tiles_m * tiles_n * (EPI == GemmEpi::kSplitPartial ? g.ksplit : 1);
  const int grid = std::min(items, cu_count());
  hipLaunchKernelGGL((gemm::gemm_ring_fp8_kernel<kFp8Stages, EPI>), dim3(grid), dim3(256), 0, st, g,
                     tiles_m, tiles_n);
}

// K ranges of a split fp8 product: the largest divisor s of K/128 with
// s * tiles <= CUs, s <= kMaxReduceSplits and ranges of at least two
// 128-wide units (the ring needs
// an even number of slices, at least as many as its stages); 1 when the
// product already has 128 tiles or more.
int split_count_fp8(int m, int n, int k) {
  const long tiles = (long)((m + 255) / 256) * (n / 256);
  if (tiles >= 128) return 1;
  const int ku = k / 128;
  int best = 1;
  for (int s = 2; s <= ku / 2 && s <= kMaxReduceSplits; ++s)
    if (ku % s == 0 && tiles * s <= cu_count()) best = s;
  return best;
}

}  // namespace

bool gemm_fp8_shape_ok(int m, int n, int k) {
  return m > 0 && n > 0 && n % 256 == 0 && k % 128 == 0 && k / 64 >= kFp8Stages;
}

// C = (A8 B8^T) * a_scale[row] * w_scale[col] with the epilogue g.epi; the
// host has checked gemm_fp8_shape_ok and 16-byte row alignment.
void launch_gemm_fp8(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0) return;
  const bool gated = g.epi == GemmEpi::kGatedResidual;
  if ((gated || g.epi == GemmEpi::kStoreF32) && g.split_ws != nullptr) {
    const int s = split_count_fp8(g.M, g.N, g.K);
    if (s > 1 && split_bytes(g.M, g.N, s) <= g.split_ws_bytes) {
      GemmArgs h = g;
      h.epi = GemmEpi::kSplitPartial;
      h.ksplit = s;
      h.C = g.split_ws;
      h.ldc = g.N;
      launch_ring_fp8<GemmEpi::kSplitPartial>(h, st);
      const size_t stride = (size_t)((g.M + 255) / 256) * 256 * g.N;
      const size_t quads = (size_t)g.M * (g.N / 4);
      hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st,
                         (float*)g.C, g.ldc, (const float*)g.split_ws, stride, s, g.M, g.N,
                         gated ? g.mod : nullptr, g.mod_stride, g.gate_offset, g.seg);
      return;
    }
  }
  switch (g.epi) {
    case GemmEpi::kStoreBf16: launch_ring_fp8<GemmEpi::kStoreBf16>(g, st); break;
    case GemmEpi::kStoreF32: launch_ring_fp8<GemmEpi::kStoreF32>(g, st); break;
    case GemmEpi::kInProj: launch_ring_fp8<GemmEpi::kInProj>(g, st); break;
    case GemmEpi::kGatedResidual: launch_ring_fp8<GemmEpi::kGatedResidual>(g, st); break;
    case GemmEpi::kSplitPartial: break;
  }
}

bool gemm_skinny_used(int m, int n, int k) { return skinny_shape(m, n, k); }

// The kernel launch_gemm picks for a product without split-K or stream-K
// scratch (the in-projection): 256x256 tiles once there are 192 of them.
bool gemm_ring_used(int m, int n, int k) {
  return m > 0 && !skinny_shape(m, n, k) && n % 256 == 0 && (long)((m + 255) / 256) * (n / 256) >= 192;
}

bool gemm_fuses_qk_norm(int m, int n, int k) { return skinny_shape(m, n, k) || gemm_ring_used(m, n, k); }

bool gemm_fuses_next_ln(int m, int n, int k, size_t scratch_bytes) {
  if (!skinny_shape(m, n, k) || n != kHidden) return false;
  const int d = skinny_split(n, k);
  return d > 1 && skinny_split_bytes(m, n, d) <= scratch_bytes;
}

int gemm_sk_counters(int m, int n, int k) {
  long tiles = 0;
  return sk_plan(m, n, k, tiles) ? (int)tiles * kSkWaves : 0;
}

size_t gemm_sk_ws_bytes(int m, int n, int k) {
  const int c = gemm_sk_counters(m, n, k);
  if (c == 0) return 0;
  return ((size_t)c * 4 + 255) / 256 * 256 + (size_t)cu_count() * 2 * kSkWaves * kSkPartBytes;
}

size_t gemm_split_ws_bytes(int m, int n, int k) {
  const int s = split_count(m, n, k);
  const size_t ring = s > 1 ? split_bytes(m, n, s) : 0;
  if (!skinny_shape(m, n, k)) return ring;
  const int d = skinny_split(n, k);
  return std::max(ring, d > 1 ? skinny_split_bytes(m, n, d) : (size_t)0);
}

namespace {

template <int MT, GemmEpi EPI>
void launch_skinny(const GemmArgs& g, int ksplit, hipStream_t st) {
  const int slabs = g.N / 128;
  hipLaunchKernelGGL((gemm::gemm_skinny_kernel<MT, EPI>), dim3(slabs * ksplit), dim3(256), 0, st, g,
                     slabs, ksplit);
}

template <int MT>
void run_skinny_mt(const GemmArgs& g, hipStream_t st) {
  const bool gated = g.epi == GemmEpi::kGatedResidual;
  if ((gated || g.epi == GemmEpi::kStoreF32) && g.split_ws != nullptr) {
    const int d = skinny_split(g.N, g.K);
    if (d > 1 && skinny_split_bytes(g.M, g.N, d) <= g.split_ws_bytes) {
      GemmArgs h = g;
      h.epi = GemmEpi::kSplitPartial;
      h.C = g.split_ws;
      h.ldc = g.N;
      launch_skinny<MT, GemmEpi::kSplitPartial>(h, d, st);
      if (gated && g.ln_out != nullptr && g.N == kHidden) {
        hipLaunchKernelGGL(split_reduce_ln_kernel, dim3(g.M), dim3(256), 0, st, (float*)g.C, g.ldc,
                           (const float*)g.split_ws, (size_t)32 * MT * g.N, d, g.mod, g.mod_stride,
                           g.gate_offset, g.seg, g.ln_out, g.ln_ldo);
        return;
      }
      const size_t quads = (size_t)g.M * (g.N / 4);
      hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st,
                         (float*)g.C, g.ldc, (const float*)g.split_ws, (size_t)32 * MT * g.N, d, g.M,
                         g.N, gated ? g.mod : nullptr, g.mod_stride, g.gate_offset, g.seg);
      return;
    }
  }
  switch (g.epi) {
    case GemmEpi::kStoreBf16: launch_skinny<MT, GemmEpi::kStoreBf16>(g, 1, st); break;
    case GemmEpi::kStoreF32: launch_skinny<MT, GemmEpi::kStoreF32>(g, 1, st); break;
    case GemmEpi::kInProj: launch_skinny<MT, GemmEpi::kInProj>(g, 1, st); break;
    case GemmEpi::kGatedResidual: launch_skinny<MT, GemmEpi::kGatedResidual>(g, 1, st); break;
    case GemmEpi::kSplitPartial: break;
  }
}

void run_skinny(const GemmArgs& g, hipStream_t st) {
  switch ((g.M + 31) / 32) {
    case 1: run_skinny_mt<1>(g, st); break;
    case 2: run_skinny_mt<2>(g, st); break;
    case 3: run_skinny_mt<3>(g, st); break;
    default: run_skinny_mt<4>(g, st); break;
  }
}

}  // namespace

// Tile choice: 256x256 tiles on the persistent ring kernel (4 waves, 128x128
// per wave) when there are at least 192 of them; otherwise the register-staged
// kernel with 128x128 tiles (4 waves, 64x64 per wave), or 64x64 tiles for
// outputs whose width is not a multiple of 128.  The host has checked
// K % 64 == 0 and N % 64 == 0.
void launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0) return;
  if (skinny_shape(g.M, g.N, g.K)) {
    run_skinny(g, st);
    return;
  }
  // Gated residual and fp32 products with too few tiles to fill the chip and
  // a long K (the text stream's and small batches' output projection, the text
  // embedding): split K over the idle CUs when the caller lent scratch for the
  // partial products.
  const bool gated = g.epi == GemmEpi::kGatedResidual;
  if ((gated || g.epi == GemmEpi::kStoreF32) && g.split_ws != nullptr) {
    const int s = split_count(g.M, g.N, g.K);
    if (s > 1 && split_bytes(g.M, g.N, s) <= g.split_ws_bytes) {
      GemmArgs h = g;
      h.epi = GemmEpi::kSplitPartial;
      h.ksplit = s;
      h.C = g.split_ws;
      h.ldc = g.N;
      run_ring<256, 256, 2, 2, 32, 5, 1>(h, st);
      const size_t stride = (size_t)((g.M + 255) / 256) * 256 * g.N;
      const size_t quads = (size_t)g.M * (g.N / 4);
      hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st,
                         (float*)g.C, g.ldc, (const float*)g.split_ws, stride, s, g.M, g.N,
                         gated ? g.mod : nullptr, g.mod_stride, g.gate_offset, g.seg);
      return;
    }
  }
  // Stream-K where whole tiles leave CUs idle in the last round.
  if (gated && g.sk_cnt != nullptr) {
    const size_t need = gemm_sk_ws_bytes(g.M, g.N, g.K);
    if (need > 0 && need <= g.sk_bytes) {
      GemmArgs h = g;
      h.group_m = kSkGroupM;
      hipLaunchKernelGGL((gemm::gemm_ring_kernel<256, 256, 2, 2, 32, 5, 1, GemmEpi::kGatedResidual, true>),
                         dim3(cu_count()), dim3(256), 0, st, h, (g.M + 255) / 256, g.N / 256);
      return;
    }
  }
  if (gemm_ring_used(g.M, g.N, g.K)) {
    run_ring<256, 256, 2, 2, 32, 5, 1>(g, st);
  } else if (g.N % 128 == 0) {
    run_regs<128, 128, 2, 2>(g, st);
  } else {
    run_regs<64, 64, 2, 1>(g, st);
  }
}

}  // namespace flux3
