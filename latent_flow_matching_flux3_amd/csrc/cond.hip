// Conditioning path and small helpers: timestep embedding, weight-streaming
// GEMVs (time MLPs, stream modulations, final adaLN), the sampler update and
// the one-time weight packing.
//
// Timestep embedding and the time MLPs: "[Feature] FLUX.3 Image Klein support
// #2142", comment §Structure (from dit.py), "Time" paragraph.  Modulation
// vectors: same comment §Tensor names (lin.weight [9216, 3072] = shift,
// scale, gate).  Sampler update: §Sampling (sampling.py, pipeline.py).
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

// emb(t) = [cos(1000 t f_j), sin(1000 t f_j)], f_j = exp(-ln(10000) j / 128).
// Block b computes the embedding of timestep ts.t[b] (fp64 math); the
// timesteps travel as kernel arguments.
__global__ void timestep_embedding_kernel(Timesteps ts, float* __restrict__ out) {
  const int t = blockIdx.x;
  const int j = threadIdx.x;  // 0..127
  const double f = exp(-log(10000.0) * (double)j / 128.0);
  const double arg = 1000.0 * (double)ts.t[t] * f;
  out[t * 256 + j] = (float)cos(arg);
  out[t * 256 + 128 + j] = (float)sin(arg);
}

void launch_timestep_embedding(const Timesteps& ts, int nt, float* out, hipStream_t st) {
  hipLaunchKernelGGL(timestep_embedding_kernel, dim3(nt), dim3(128), 0, st, ts, out);
}

// Batched GEMV: for each batch b, y_b[r] (+)= sum_k W_b[r][k] * f(x_b[k]), with
// f = SiLU or identity.  W bf16 [rows][K] (K % 8 == 0, K <= 4096), x fp32.
// Each wave keeps its slice of f(x) in registers and streams kGemvRows rows of
// W (16-byte loads, 64 lanes across K), one wave reduction per row.
constexpr int kGemvMaxChunksPerLane = 8;  // K <= 64 * 8 * 8 = 4096

// RPW rows per wave, in groups of 4 whose weight loads are issued together.
// Every wave first forms (SiLU of) x in registers, one memory latency; a
// wave then streams its rows.  Four rows per wave (each wave one group of
// loads, many waves) beat 16 (four groups one after another, a quarter of
// the waves) once the preamble waited for x only once: the four streams'
// modulations in the 96-token loop ≈72 → ≈55 µs.
template <int RPW>
__global__ __launch_bounds__(256) void gemv_kernel(GemvBatch batch, int rows, int K, int silu_x,
                                                   int accumulate) {
  const int b = blockIdx.y;
  const bf16* __restrict__ W = batch.w[b];
  const float* __restrict__ x = batch.x[b];
  float* __restrict__ y = batch.y[b];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = K / 8;
  // f(x) in registers: every load issued first (chunks past K read the last
  // chunk again and are then zeroed), so the wave waits for x once, not once
  // per element.
  float xv[kGemvMaxChunksPerLane][8];
#pragma unroll
  for (int i = 0; i < kGemvMaxChunksPerLane; ++i) {
    const float* xp = x + min(lane + 64 * i, nchunk - 1) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[i][e] = xp[e];
  }
#pragma unroll
  for (int i = 0; i < kGemvMaxChunksPerLane; ++i) {
    const bool valid = lane + 64 * i < nchunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float val = xv[i][e];
      if (silu_x) val = val / (1.0f + __expf(-val));
      xv[i][e] = valid ? val : 0.f;
    }
  }
  const int r0 = (blockIdx.x * 4 + wave) * RPW;
#pragma unroll 1
  for (int g = 0; g < RPW; g += 4) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = r0 + g + rr;
      if (r >= rows) break;
      const bf16* wr = W + (size_t)r * K;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kGemvMaxChunksPerLane; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
          bf16x8 w8 = *(const bf16x8*)(wr + c * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc += (float)w8[e] * xv[i][e];
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) y[r] = accumulate ? y[r] + acc : acc;
    }
  }
}

void launch_gemv(const GemvBatch& batch, int nb, int rows, int K, bool silu_x, bool accumulate,
                 hipStream_t st) {
  dim3 grid((rows + 15) / 16, nb);  // 16 rows per workgroup of 4 waves
  hipLaunchKernelGGL(gemv_kernel<4>, grid, dim3(256), 0, st, batch, rows, K, silu_x ? 1 : 0,
                     accumulate ? 1 : 0);
}

// x += (sigma_next - sigma) * v; xb = bf16(x).  v == nullptr: x unchanged,
// only the bf16 copy is written.
__global__ void euler_kernel(float* __restrict__ x, bf16* __restrict__ xb,
                             const float* __restrict__ v, int n, float dt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float y = v ? x[i] + dt * v[i] : x[i];
  if (v) x[i] = y;
  if (xb) xb[i] = to_bf16(y);
}

void launch_euler(float* x, bf16* xb, const float* v, int n, float dt, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(euler_kernel, dim3((n + 255) / 256), dim3(256), 0, st, x, xb, v, n, dt);
}

// Classifier-free guidance: v = vu + g (vc - vu).
__global__ void cfg_combine_kernel(const float* __restrict__ vu, const float* __restrict__ vc,
                                   float* __restrict__ v, int n, float g) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = vu[i];
  v[i] = a + g * (vc[i] - a);
}

void launch_cfg_combine(const float* vu, const float* vc, float* v, int n, float g, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(cfg_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, st, vu, vc, v, n, g);
}

// Weight packing (one-time).  w_in rows: q | k | v, then mlp_in with the a/b
// halves interleaved in groups of 32 rows.  w_out: [attn_out | mlp_out].
// One 16-byte chunk per thread.
__global__ void pack_w_in_kernel(const bf16* __restrict__ wq, const bf16* __restrict__ wk,
                                 const bf16* __restrict__ wv, const bf16* __restrict__ w_mlp_in,
                                 bf16* __restrict__ w_in) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t chunks_per_row = kHidden / 8;
  if (t >= (size_t)kWInRows * chunks_per_row) return;
  const int row = (int)(t / chunks_per_row);
  const int c = (int)(t % chunks_per_row);
  const bf16* src;
  if (row < kHidden) src = wq + (size_t)row * kHidden;
  else if (row < 2 * kHidden) src = wk + (size_t)(row - kHidden) * kHidden;
  else if (row < 3 * kHidden) src = wv + (size_t)(row - 2 * kHidden) * kHidden;
  else {
    const int p = row - 3 * kHidden;
    const int grp = p / 64, w = p % 64;
    const int srow = w < 32 ? grp * 32 + w : kMlp + grp * 32 + (w - 32);
    src = w_mlp_in + (size_t)srow * kHidden;
  }
  *(bf16x8*)(w_in + (size_t)row * kHidden + c * 8) = *(const bf16x8*)(src + c * 8);
}

__global__ void pack_w_out_kernel(const bf16* __restrict__ wo, const bf16* __restrict__ w_mlp_out,
                                  bf16* __restrict__ w_out) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t chunks_per_row = kWOutCols / 8;
  if (t >= (size_t)kHidden * chunks_per_row) return;
  const int row = (int)(t / chunks_per_row);
  const int c = (int)(t % chunks_per_row) * 8;
  const bf16* src = c < kHidden ? wo + (size_t)row * kHidden + c
                                : w_mlp_out + (size_t)row * kMlp + (c - kHidden);
  *(bf16x8*)(w_out + (size_t)row * kWOutCols + c) = *(const bf16x8*)src;
}

void launch_pack_block(const bf16* wq, const bf16* wk, const bf16* wv, const bf16* wo,
                       const bf16* w_mlp_in, const bf16* w_mlp_out, bf16* w_in, bf16* w_out,
                       hipStream_t st) {
  const size_t n_in = (size_t)kWInRows * (kHidden / 8);
  hipLaunchKernelGGL(pack_w_in_kernel, dim3((unsigned)((n_in + 255) / 256)), dim3(256), 0, st, wq,
                     wk, wv, w_mlp_in, w_in);
  const size_t n_out = (size_t)kHidden * (kWOutCols / 8);
  hipLaunchKernelGGL(pack_w_out_kernel, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, st,
                     wo, w_mlp_out, w_out);
}

}  // namespace flux3
