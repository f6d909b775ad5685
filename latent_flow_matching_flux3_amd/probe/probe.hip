// Peak probes for the measurement harness (not part of libflux3_dit): what
// this MI355X sustains on the two resources the kernels are priced against.
//   flux3_probe_mfma_bf16: every wave issues independent
//     v_mfma_f32_32x32x16_bf16 on register operands (random bf16 values, so
//     the power draw is that of real data), 8 accumulator chains per wave,
//     no memory traffic inside the loop.
//   flux3_probe_copy: a streaming copy (16-byte loads and stores, grid
//     stride) between two caller buffers larger than the 256 MB Infinity
//     Cache, i.e. HBM read + write bandwidth; the caller picks the grid (the
//     best rate comes from a few hundred workgroups, not from the most).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ unsigned hash32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// bf16 values in [1, 2) with random mantissas (sign random).
__device__ __forceinline__ bf16x8_t random_frag(unsigned seed) {
  bf16x8_t v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned h = hash32(seed * 8 + e);
    const unsigned short bits = (unsigned short)(0x3F80u | (h & 0x7Fu) | ((h >> 8) & 0x8000u));
    v[e] = __builtin_bit_cast(__bf16, bits);
  }
  return v;
}

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  const unsigned tid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = random_frag(tid * 4 + i);
    b[i] = random_frag(tid * 4 + 2 + i);
  }
  floatx16_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 1], b[(c >> 1) & 1], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[tid] = s;
}

// Each thread moves 2 x 16 bytes per pass (both loads issued before the
// stores), passes grid-strided.
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4_t* __restrict__ src,
                                                         u32x4_t* __restrict__ dst, size_t n) {
  const size_t lanes = (size_t)gridDim.x * blockDim.x;
  for (size_t base = (size_t)blockIdx.x * blockDim.x + threadIdx.x; base < n; base += 2 * lanes) {
    const bool two = base + lanes < n;
    const u32x4_t v0 = src[base];
    const u32x4_t v1 = two ? src[base + lanes] : v0;
    dst[base] = v0;
    if (two) dst[base + lanes] = v1;
  }
}

}  // namespace

extern "C" {

// Launches the MFMA probe: blocks x 4 waves (one block per CU: one wave per
// SIMD), each running iters x 8 MFMAs of 32x32x16 (32768 flop each).  out: device [blocks * 256] fp32 (sums, keeps
// the work live).  Returns 0, or the HIP error code of the launch.
int flux3_probe_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
  return (int)hipGetLastError();
}

// Copies bytes (a multiple of 16, both pointers 16-byte aligned) from src to
// dst with `blocks` workgroups of 256 threads.  Returns 0, -1 for bad
// arguments, or the HIP error code of the launch.
int flux3_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  if (bytes == 0 || bytes % 16 != 0 || blocks <= 0) return -1;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4_t*)src, (u32x4_t*)dst,
                     bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
