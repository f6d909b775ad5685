// Shared device helpers for the gfx950 kernels: bf16 conversion, vector types,
// wave reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux3 {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr int kHidden = 3072;
constexpr int kHeads = 24;
constexpr int kHeadDim = 128;
constexpr int kMlp = 9216;
constexpr int kWInRows = 3 * kHidden + 2 * kMlp;   // 27648
constexpr int kWOutCols = kHidden + kMlp;          // 12288
constexpr int kMaxSeg = 8;

// Row offsets of the modulation segments, passed by value to kernels.
struct SegTable {
  int off[kMaxSeg + 1];
  int n;
};

__device__ __forceinline__ int seg_of_row(const SegTable& s, int row) {
  int m = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i)
    if (i < s.n && row >= s.off[i]) m = i;
  return m;
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf16(float f) { return (bf16)f; }
__device__ __forceinline__ float to_f32(bf16 b) { return (float)b; }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  bf16 b = (bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Sum over the 64 lanes of a wave (butterfly), result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// silu(x) = x / (1 + e^-x) with the hardware reciprocal (1 ulp); -0 for
// x -> -inf, x for x -> +inf.
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace flux3
