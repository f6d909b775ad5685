// Memory-bound kernels of the block: LayerNorm + modulation, QK RMSNorm +
// 4-axis RoPE, and the RoPE table.
//
// LayerNorm + modulation: "Welcome FLUX.3 Image Klein in Diffusers",
// §Inside one block (LayerNorm without learned affine, then (1 + scale) * h +
// shift); eps 1e-6 from "[Feature] FLUX.3 Image Klein support #2142",
// comment §Structure (from dit.py).
// RMSNorm + RoPE: same comment §Structure (per-head RMSNorm, eps 1e-6, scale
// over head_dim 128, then RoPE with 4 axes of 32 dims, theta 10000).
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

// ---------------------------------------------------------------------------
// K1: one wave per row of the fp32 residual stream.  A row of 3072 floats is
// 768 chunks of 16 bytes; lane l owns chunks l, l+64, ..., l+704 (coalesced
// 1 KiB per wave instruction) and keeps its 48 values in registers, so the
// row is read once and the variance is the exact two-pass form
// mean((x - mu)^2) in fp32.  Output bf16 (the GEMM operand).
// ---------------------------------------------------------------------------
constexpr int kLnRowsPerBlock = 4;

__global__ __launch_bounds__(256) void ln_modulate_kernel(const float* __restrict__ x, int ldx,
                                                          bf16* __restrict__ out, int ldo, int n,
                                                          SegTable seg,
                                                          const float* __restrict__ mod,
                                                          int mod_stride) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kLnRowsPerBlock + (threadIdx.x >> 6);
  if (row >= n) return;
  const float* xr = x + (size_t)row * ldx;
  // The row's shift and scale are loaded with x (they do not depend on it).
  const float* shift = mod + (size_t)seg_of_row(seg, row) * mod_stride;
  const float* scale = shift + kHidden;
  float4 shv[12], scv[12];
  float v[12][4];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    shv[i] = *(const float4*)(shift + (lane + 64 * i) * 4);
    scv[i] = *(const float4*)(scale + (lane + 64 * i) * 4);
  }
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const float4 c = *(const float4*)(xr + (lane + 64 * i) * 4);
    v[i][0] = c.x;
    v[i][1] = c.y;
    v[i][2] = c.z;
    v[i][3] = c.w;
    s += (c.x + c.y) + (c.z + c.w);
  }
  const float mu = wave_sum(s) * (1.0f / kHidden);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 12; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = v[i][e] - mu;
      q += d * d;
    }
  const float var = wave_sum(q) * (1.0f / kHidden);
  const float rstd = 1.0f / sqrtf(var + 1e-6f);
  bf16* orow = out + (size_t)row * ldo;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const int c0 = (lane + 64 * i) * 4;
    const float4 sh = shv[i], sc = scv[i];
    bf16x4 o;
    o[0] = to_bf16((1.0f + sc.x) * ((v[i][0] - mu) * rstd) + sh.x);
    o[1] = to_bf16((1.0f + sc.y) * ((v[i][1] - mu) * rstd) + sh.y);
    o[2] = to_bf16((1.0f + sc.z) * ((v[i][2] - mu) * rstd) + sh.z);
    o[3] = to_bf16((1.0f + sc.w) * ((v[i][3] - mu) * rstd) + sh.w);
    *(bf16x4*)(orow + c0) = o;
  }
}

void launch_ln_modulate(const float* x, int ldx, bf16* out, int ldo, int n, const SegTable& seg,
                        const float* mod, int mod_stride, hipStream_t st) {
  if (n <= 0) return;
  dim3 grid((n + kLnRowsPerBlock - 1) / kLnRowsPerBlock);
  hipLaunchKernelGGL(ln_modulate_kernel, grid, dim3(256), 0, st, x, ldx, out, ldo, n, seg, mod,
                     mod_stride);
}

// ---------------------------------------------------------------------------
// RoPE table: (cos, sin) of id_a * 10000^(-2j/32) for the 64 pairs p = 16a+j.
// Angles up to a few thousand radians (text positions) are formed and reduced
// in fp64, then rounded to fp32.
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(const float* __restrict__ ids, int n, float* __restrict__ table) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * 64) return;
  const int tok = t >> 6, p = t & 63, a = p >> 4, j = p & 15;
  const double omega = pow(10000.0, -2.0 * j / 32.0);
  const double ang = (double)ids[tok * 4 + a] * omega;
  table[2 * t] = (float)cos(ang);
  table[2 * t + 1] = (float)sin(ang);
}

void launch_rope_table(const float* ids, int n, float* table, hipStream_t st) {
  if (n <= 0) return;
  const int total = n * 64;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, st, ids, n, table);
}

// ---------------------------------------------------------------------------
// K2: QK RMSNorm + RoPE, in place.  One block (4 waves) per token; 16 lanes
// per 128-wide head vector, 8 dims (4 rotation pairs, all in one axis) per
// lane.  The 48 head vectors of a token (24 q + 24 k) are 12 wave-steps.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(bf16* __restrict__ q, int ldq,
                                                           bf16* __restrict__ k, int ldk, int n,
                                                           const bf16* __restrict__ q_scale,
                                                           const bf16* __restrict__ k_scale,
                                                           const float* __restrict__ table,
                                                           int* __restrict__ zero, int nzero) {
  const int tok = blockIdx.x;
  if (tok >= n) return;
  if (tok == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0;
  const int lane16 = threadIdx.x & 15;
  const int vec_id = threadIdx.x >> 4;  // 0..15 head vectors per pass
  const int d0 = lane16 * 8;
  // rotation for pairs d0/2 .. d0/2+3
  const float* tb = table + (size_t)tok * 128 + d0;
  const float4 t0 = *(const float4*)tb, t1 = *(const float4*)(tb + 4);
  const float cs[4] = {t0.x, t0.z, t1.x, t1.z};
  const float sn[4] = {t0.y, t0.w, t1.y, t1.w};
  const bf16x8 qs = *(const bf16x8*)(q_scale + d0);
  const bf16x8 ks = *(const bf16x8*)(k_scale + d0);
  // All three head vectors are loaded before any is stored: the rows are
  // updated in place, so a load after a store would wait for that store.
  bf16* ptrs[3];
  bf16x8 cv[3];
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int hv = pass * 16 + vec_id;  // 0..47
    const bool is_k = hv >= kHeads;
    const int head = is_k ? hv - kHeads : hv;
    ptrs[pass] = (is_k ? k + (size_t)tok * ldk : q + (size_t)tok * ldq) + head * kHeadDim + d0;
    cv[pass] = *(const bf16x8*)ptrs[pass];
  }
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const bool is_k = pass * 16 + vec_id >= kHeads;
    bf16* ptr = ptrs[pass];
    const bf16x8 c = cv[pass];
    float v[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)c[e];
      ss += v[e] * v[e];
    }
    ss = group_sum<16>(ss);
    const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + 1e-6f);
    const bf16x8 sc = is_k ? ks : qs;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * r * (float)sc[e];
    bf16x8 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = v[2 * p], x1 = v[2 * p + 1];
      o[2 * p] = to_bf16(x0 * cs[p] - x1 * sn[p]);
      o[2 * p + 1] = to_bf16(x0 * sn[p] + x1 * cs[p]);
    }
    *(bf16x8*)ptr = o;
  }
}

void launch_qk_norm_rope(bf16* q, int ldq, bf16* k, int ldk, int n, const bf16* q_scale,
                         const bf16* k_scale, const float* table, hipStream_t st, int* zero,
                         int nzero) {
  if (n <= 0) return;
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3(n), dim3(256), 0, st, q, ldq, k, ldk, n, q_scale,
                     k_scale, table, zero, nzero);
}

}  // namespace flux3
