// Rowwise FP8 quantization for the fp8r projections ("Welcome FLUX.3 Image
// Klein in Diffusers", §Base model and quantized variants: fp8r, rowwise
// FP8): per row, scale = max|x| / 448 and E4M3 codes of x * (448 / max|x|),
// the scale, its inverse and the product in fp32; codes by the hardware
// conversion (OCP E4M3, round to nearest even); a row of zeros gets scale 1.
//   - ln_modulate_fp8_kernel: LayerNorm + modulation (as ln_modulate_kernel)
//     with the quantization of the modulated row fused (the in-projection's
//     input never exists in bf16);
//   - quant_cat_fp8_kernel: the out-projection's input [o | h] (12288 wide,
//     every block), read once into registers, o and h with a scale each
//     (they feed two Linears, attn_out and mlp_out);
//   - quant_rows_fp8_reg_kernel: rows of a multiple of 2048 values up to
//     16384, read once into registers;
//   - quant_rows_fp8_kernel: any other width (the weights, once), two passes.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Four values scaled by inv, as four E4M3 codes in one dword (byte e = value e).
__device__ __forceinline__ unsigned fp8x4(float a, float b, float c, float d, float inv) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a * inv, b * inv, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c * inv, d * inv, w, true);
  return (unsigned)w;
}

// scale = amax / 448 and its inverse 448 / amax (IEEE fp32 divisions).
__device__ __forceinline__ void row_scale(float amax, float& scale, float& inv) {
  if (amax > 0.f) {
    scale = amax / 448.0f;
    inv = 448.0f / amax;
  } else {
    scale = 1.f;
    inv = 1.f;
  }
}

constexpr int kLnRowsPerBlock = 4;

// One wave per row of the fp32 residual stream (3072 values, 48 per lane in
// registers); out: [n][ldo] codes, scale: [n] fp32.
__global__ __launch_bounds__(256) void ln_modulate_fp8_kernel(const float* __restrict__ x, int ldx,
                                                              uint8_t* __restrict__ out, int ldo,
                                                              float* __restrict__ out_scale, int n,
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
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const float4 sh = shv[i], sc = scv[i];
    v[i][0] = (1.0f + sc.x) * ((v[i][0] - mu) * rstd) + sh.x;
    v[i][1] = (1.0f + sc.y) * ((v[i][1] - mu) * rstd) + sh.y;
    v[i][2] = (1.0f + sc.z) * ((v[i][2] - mu) * rstd) + sh.z;
    v[i][3] = (1.0f + sc.w) * ((v[i][3] - mu) * rstd) + sh.w;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3]))));
  }
  float rs, inv;
  row_scale(wave_max(amax), rs, inv);
  uint8_t* orow = out + (size_t)row * ldo;
#pragma unroll
  for (int i = 0; i < 12; ++i)
    *(unsigned*)(orow + (lane + 64 * i) * 4) = fp8x4(v[i][0], v[i][1], v[i][2], v[i][3], inv);
  if (lane == 0) out_scale[row] = rs;
}

// One workgroup per row of `cols` bf16 values (cols a multiple of 8): the
// row max in a first pass, the codes in a second (the row is in cache).
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const bf16* __restrict__ x, int ldx,
                                                             int cols, uint8_t* __restrict__ out,
                                                             int ldo, float* __restrict__ out_scale) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const bf16* xr = x + (size_t)row * ldx;
  float amax = 0.f;
  for (int c = threadIdx.x * 8; c < cols; c += 256 * 8) {
    const bf16x8 t = *(const bf16x8*)(xr + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(to_f32(t[e])));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  float rs, inv;
  row_scale(amax, rs, inv);
  uint8_t* orow = out + (size_t)row * ldo;
  for (int c = threadIdx.x * 8; c < cols; c += 256 * 8) {
    const bf16x8 t = *(const bf16x8*)(xr + c);
    uint2 w;
    w.x = fp8x4(to_f32(t[0]), to_f32(t[1]), to_f32(t[2]), to_f32(t[3]), inv);
    w.y = fp8x4(to_f32(t[4]), to_f32(t[5]), to_f32(t[6]), to_f32(t[7]), inv);
    *(uint2*)(orow + c) = w;
  }
  if (threadIdx.x == 0) out_scale[row] = rs;
}

// One workgroup per row of C * 2048 bf16 values, the row in registers (C
// 16-byte chunks per thread): one read of the row.
template <int C>
__global__ __launch_bounds__(256) void quant_rows_fp8_reg_kernel(const bf16* __restrict__ x, int ldx,
                                                                 uint8_t* __restrict__ out, int ldo,
                                                                 float* __restrict__ out_scale) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const bf16* xr = x + (size_t)row * ldx;
  float v[C][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const bf16x8 t = *(const bf16x8*)(xr + (threadIdx.x + 256 * i) * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[i][e] = to_f32(t[e]);
      amax = fmaxf(amax, fabsf(v[i][e]));
    }
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  float rs, inv;
  row_scale(amax, rs, inv);
  uint8_t* orow = out + (size_t)row * ldo;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    uint2 w;
    w.x = fp8x4(v[i][0], v[i][1], v[i][2], v[i][3], inv);
    w.y = fp8x4(v[i][4], v[i][5], v[i][6], v[i][7], inv);
    *(uint2*)(orow + (threadIdx.x + 256 * i) * 8) = w;
  }
  if (threadIdx.x == 0) out_scale[row] = rs;
}

// One workgroup per row of the block's [o | h] (6 * 2048 bf16 values, in
// registers): o (the first kHidden values) and h (the rest) are the inputs
// of two Linears and get a scale each; ratio = scale of o / scale of h.
__global__ __launch_bounds__(256) void quant_cat_fp8_kernel(const bf16* __restrict__ x, int ldx,
                                                            uint8_t* __restrict__ out, int ldo,
                                                            float* __restrict__ scale0,
                                                            float* __restrict__ scale1,
                                                            float* __restrict__ ratio) {
  constexpr int C = kWOutCols / 2048;
  constexpr int kSplitChunk = kHidden / 8;  // 8-value chunks of o
  static_assert(kWOutCols % 2048 == 0 && kHidden % 8 == 0, "row geometry");
  __shared__ float part[2][4];
  const int row = blockIdx.x;
  const bf16* xr = x + (size_t)row * ldx;
  float v[C][8];
  float amax0 = 0.f, amax1 = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int chunk = threadIdx.x + 256 * i;
    const bf16x8 t = *(const bf16x8*)(xr + chunk * 8);
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[i][e] = to_f32(t[e]);
      m = fmaxf(m, fabsf(v[i][e]));
    }
    if (chunk < kSplitChunk) amax0 = fmaxf(amax0, m);
    else amax1 = fmaxf(amax1, m);
  }
  amax0 = wave_max(amax0);
  amax1 = wave_max(amax1);
  if ((threadIdx.x & 63) == 0) {
    part[0][threadIdx.x >> 6] = amax0;
    part[1][threadIdx.x >> 6] = amax1;
  }
  __syncthreads();
  amax0 = fmaxf(fmaxf(part[0][0], part[0][1]), fmaxf(part[0][2], part[0][3]));
  amax1 = fmaxf(fmaxf(part[1][0], part[1][1]), fmaxf(part[1][2], part[1][3]));
  float rs0, inv0, rs1, inv1;
  row_scale(amax0, rs0, inv0);
  row_scale(amax1, rs1, inv1);
  uint8_t* orow = out + (size_t)row * ldo;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int chunk = threadIdx.x + 256 * i;
    const float inv = chunk < kSplitChunk ? inv0 : inv1;
    uint2 w;
    w.x = fp8x4(v[i][0], v[i][1], v[i][2], v[i][3], inv);
    w.y = fp8x4(v[i][4], v[i][5], v[i][6], v[i][7], inv);
    *(uint2*)(orow + chunk * 8) = w;
  }
  if (threadIdx.x == 0) {
    scale0[row] = rs0;
    scale1[row] = rs1;
    ratio[row] = rs0 / rs1;
  }
}

__global__ __launch_bounds__(256) void scale_ratio_kernel(const float* __restrict__ a,
                                                          const float* __restrict__ b,
                                                          float* __restrict__ out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = a[i] / b[i];
}

}  // namespace

void launch_quant_cat_fp8(const bf16* x, int ldx, int rows, uint8_t* out, int ldo, float* scale0,
                          float* scale1, float* ratio, hipStream_t st) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(quant_cat_fp8_kernel, dim3(rows), dim3(256), 0, st, x, ldx, out, ldo, scale0, scale1,
                     ratio);
}

void launch_scale_ratio(const float* a, const float* b, float* out, int n, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(scale_ratio_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a, b, out, n);
}

void launch_ln_modulate_fp8(const float* x, int ldx, uint8_t* out, int ldo, float* scale, int n,
                            const SegTable& seg, const float* mod, int mod_stride, hipStream_t st) {
  if (n <= 0) return;
  dim3 grid((n + kLnRowsPerBlock - 1) / kLnRowsPerBlock);
  hipLaunchKernelGGL(ln_modulate_fp8_kernel, grid, dim3(256), 0, st, x, ldx, out, ldo, scale, n, seg,
                     mod, mod_stride);
}

void launch_quant_rows_fp8(const bf16* x, int ldx, int rows, int cols, uint8_t* out, int ldo,
                           float* scale, hipStream_t st) {
  if (rows <= 0) return;
#define FLUX3_QUANT_REG(C)                                                                            \
  case C:                                                                                             \
    hipLaunchKernelGGL(quant_rows_fp8_reg_kernel<C>, dim3(rows), dim3(256), 0, st, x, ldx, out, ldo, \
                       scale);                                                                        \
    return;
  if (cols % 2048 == 0) {
    switch (cols / 2048) {
      FLUX3_QUANT_REG(1)
      FLUX3_QUANT_REG(2)
      FLUX3_QUANT_REG(3)
      FLUX3_QUANT_REG(4)
      FLUX3_QUANT_REG(5)
      FLUX3_QUANT_REG(6)
      FLUX3_QUANT_REG(7)
      FLUX3_QUANT_REG(8)
      default: break;
    }
  }
#undef FLUX3_QUANT_REG
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3(rows), dim3(256), 0, st, x, ldx, cols, out, ldo, scale);
}

}  // namespace flux3
