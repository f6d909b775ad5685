// Flash-style attention forward: o = softmax(q k^T / sqrt(128)) v per head,
// no mask ("Welcome FLUX.3 Image Klein in Diffusers", §Two stages: in the
// joint blocks every token attends to every other token; a stage-1 call is
// simply made on one stream's rows).
//
// Design (gfx950, head_dim 128):
//   - One workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//     query rows.  K/V are walked in 64-key tiles staged through LDS (two
//     buffers, register prefetch of the next tile while the current one is
//     consumed).
//   - Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = K from LDS, B = Q^T held in registers for
//     the whole kernel.  A lane then holds one query row (lane % 32) and 32 of
//     the tile's 64 keys, so the row max and row sum are per-lane register
//     reductions plus one exchange with lane ^ 32.
//   - The probabilities stay in registers and feed O^T = V^T P^T directly as
//     the B operand (their register layout is already the B layout, with the
//     keys in a fixed permutation that the V^T reads follow).  V is stored
//     transposed in LDS ([d][key], 8-byte chunks XOR-swizzled by d) so each
//     A-operand read is two 8-byte LDS loads.
//   - Online softmax in base 2: p = exp2(s * log2(e)/sqrt(128) - m); the
//     accumulator is rescaled by exp2(m_old - m_new) when the row max grows.
//   - Workgroups of the same head are placed on the same XCD (3 heads per
//     XCD), so that head's K/V stay in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int kBQ = 128;   // query rows per workgroup
constexpr int kBKV = 64;   // keys per tile
constexpr int kKsChunks = kBKV * 16;     // 16-byte chunks of a K tile
constexpr int kVtChunks = kHeadDim * 16; // 8-byte chunks of a V^T tile

// LDS swizzles (64 banks x 4 bytes: a 128-bit read serves 16 lanes per cycle,
// a 64-bit read 32 lanes).  K rows are 256 bytes = 16 chunks of 16 bytes and
// an operand read puts 16 consecutive rows in one group: chunk c ^ (row & 15).
// V^T rows are 128 bytes = 16 chunks of 8 bytes and a read puts 32
// consecutive d in one group, d and d+1 in opposite 128-byte halves:
// chunk c ^ ((d >> 1) & 15).
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int vt_swz(int d) { return (d >> 1) & 15; }

__global__ __launch_bounds__(256) void attn_fwd_kernel(const bf16* __restrict__ q, int ldq,
                                                       const bf16* __restrict__ k, int ldk,
                                                       const bf16* __restrict__ v, int ldv,
                                                       bf16* __restrict__ o, int ldo, int n,
                                                       float scale_log2) {
  __shared__ bf16x8 ks_lds[2][kKsChunks];
  __shared__ bf16x4 vt_lds[2][kVtChunks];

  const int nqb = (n + kBQ - 1) / kBQ;
  const int total = nqb * kHeads;  // multiple of 8
  const int lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int head = lin / nqb;
  const int qb = lin % nqb;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int hoff = head * kHeadDim;

  // Q^T fragments (B operand): lane holds query row lr, dims 16 s + 8 lh .. +8.
  const int qrow = min(qb * kBQ + wave * 32 + lr, n - 1);
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(q + (size_t)qrow * ldq + hoff + 16 * s + 8 * lh);

  // Staging assignments.  K: chunk ids tid + 256 i -> (row, 16-byte chunk).
  // V: thread covers keys 4 kg .. 4 kg + 3 and dims 8 dg .. 8 dg + 7.
  const int kg = tid >> 4, dg = tid & 15;
  bf16x8 rk[4], rv[4];
  auto load_tile = [&](int key0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int row = min(key0 + (id >> 4), n - 1);
      rk[i] = *(const bf16x8*)(k + (size_t)row * ldk + hoff + (id & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(key0 + 4 * kg + i, n - 1);
      rv[i] = *(const bf16x8*)(v + (size_t)row * ldv + hoff + 8 * dg);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 4, c = id & 15;
      ks_lds[buf][row * 16 + (c ^ k_swz(row))] = rk[i];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = 8 * dg + j;
      bf16x4 t;
      t[0] = rv[0][j];
      t[1] = rv[1][j];
      t[2] = rv[2][j];
      t[3] = rv[3][j];
      vt_lds[buf][d * 16 + (kg ^ vt_swz(d))] = t;
    }
  };

  floatx16 oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_run = -INFINITY;  // running max (scaled, base-2 domain) of row lr
  float l_run = 0.f;        // this lane's partial row sum

  const int ntiles = (n + kBKV - 1) / kBKV;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int key0 = t * kBKV;
    if (t + 1 < ntiles) load_tile(key0 + kBKV);

    // S^T = K Q^T for keys key0 .. key0+63 (two 32-key fragments).
    floatx16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      const int row = kb * 32 + lr;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a = ks_lds[buf][row * 16 + ((2 * s + lh) ^ k_swz(row))];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
      }
    }
    // Keys past the end of the sequence get probability 0.
    if (key0 + kBKV > n) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (key >= n) sacc[kb][r] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pf[4];  // B operand per 16-key step j: keys of fragment j/2, registers 8 (j%2) ..
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], scale_log2, -m_new));
        psum += p;
        pf[kb * 2 + (r >> 3)][r & 7] = to_bf16(p);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

    // O^T += V^T P^T.  Step j covers keys 16 j .. 16 j + 15; lane half lh
    // supplies keys 16 j + {0..3, 8..11} + 4 lh, read from V^T as two 8-byte
    // chunks (16 j + 4 lh) / 4 and (16 j + 8 + 4 lh) / 4.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + lr;
      const int sw = vt_swz(d);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 lo = vt_lds[buf][d * 16 + ((4 * j + lh) ^ sw)];
        const bf16x4 hi = vt_lds[buf][d * 16 + ((4 * j + 2 + lh) ^ sw)];
        bf16x8 a;
        a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
        a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[db], 0, 0, 0);
      }
    }

    // Buffer buf ^ 1 was last read in the previous iteration, before its
    // closing barrier, so it can be refilled now; the barrier below publishes it.
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Normalise and store: lane holds query row lr, dims db*32 + 8 g + 4 lh + 0..3.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int orow = qb * kBQ + wave * 32 + lr;
  if (orow < n) {
    bf16* op = o + (size_t)orow * ldo + hoff;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = to_bf16(oacc[db][4 * g4 + e] * inv);
        *(bf16x4*)(op + db * 32 + 8 * g4 + 4 * lh) = t;
      }
  }
}

}  // namespace

void launch_attention(const bf16* q, int ldq, const bf16* k, int ldk, const bf16* v, int ldv,
                      bf16* o, int ldo, int n, hipStream_t st) {
  if (n <= 0) return;
  const int nqb = (n + kBQ - 1) / kBQ;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHeadDim);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(nqb * kHeads), dim3(256), 0, st, q, ldq, k, ldk, v, ldv,
                     o, ldo, n, scale_log2);
}

}  // namespace flux3
