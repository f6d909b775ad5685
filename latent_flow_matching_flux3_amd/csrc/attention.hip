// Flash-style attention forward: o = softmax(q k^T / sqrt(128)) v per head,
// no mask ("Welcome FLUX.3 Image Klein in Diffusers", §Two stages: in the
// joint blocks every token attends to every other token; a stage-1 call is
// simply made on one stream's rows).
//
// Design (gfx950, head_dim 128):
//   - One workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//     query rows.  K and V are walked in 64-key tiles through a 4-slot LDS
//     ring, filled straight from global memory (global_load_lds_dwordx4),
//     three tiles ahead.
//   - Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = K from LDS, B = Q^T held in registers for
//     the whole kernel.  A lane then holds one query row (lane % 32) and 32 of
//     the tile's 64 keys, so the row max and row sum are per-lane register
//     reductions plus one exchange between the wave halves.
//   - The probabilities stay in registers and feed O^T = V^T P^T directly as
//     the B operand (their register layout is already the B layout, with the
//     keys in a fixed permutation).  V stays row-major in LDS; the A operand
//     V^T is read with ds_read_b64_tr_b16, whose 16-lane transpose hands each
//     lane 4 keys of one head dim, in exactly that key permutation.
//   - Software pipeline inside each wave: the scores of tile t+1 (MFMA) are
//     computed while the softmax of tile t (VALU) runs.
//   - Online softmax in base 2: p = exp2(s * log2(e)/sqrt(128) - m), where the
//     reference m may lag the running row max by up to 8 (p <= 256, exact in
//     the final O / l); the output accumulator is rescaled only when some
//     row's max jumps past that (a wave-uniform test), i.e. almost never
//     after the first tile.
//   - Workgroups of the same head are placed on the same XCD (3 heads per
//     XCD), so that head's K/V stay in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int kBQ = 256;   // query rows per workgroup (8 waves x 32)
constexpr int kWaves = kBQ / 32;
constexpr int kBKV = 64;   // keys per tile
constexpr int kNBuf = 3;   // LDS ring slots
constexpr int kTileChunks = kBKV * 16;  // 16-byte chunks of a 64 x 128 bf16 tile (16 KiB)
constexpr float kSlack = 8.0f;          // allowed lag of the softmax reference max (log2 units)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gmem_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4_t;

// LDS layouts (64 banks x 4 bytes).  Rows are keys, 256 bytes = 16 chunks of
// 16 bytes.
//   K: an operand read puts 16 consecutive rows, same logical chunk, in one
//      16-lane group: chunk c of row r at c ^ (r & 15).
//   V: a transpose read by 32 lanes touches 4 key rows (keys 4a .. 4a+3),
//      64 bytes each at the same offset: the 64-byte quarter q of row r is
//      stored at q ^ (r & 3), i.e. 16-byte chunk c at c ^ 4 (r & 3).
__device__ __forceinline__ int k_phys(int row, int c) { return row * 16 + (c ^ (row & 15)); }
__device__ __forceinline__ int v_phys(int row, int c) { return row * 16 + (c ^ (4 * (row & 3))); }

__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32, 64); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(kBQ * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const bf16* __restrict__ q, int ldq, const bf16* __restrict__ k, int ldk,
                     const bf16* __restrict__ v, int ldv, bf16* __restrict__ o, int ldo, int n,
                     float scale_log2) {
  __shared__ bf16x8 ks_lds[kNBuf][kTileChunks];
  __shared__ bf16x8 vs_lds[kNBuf][kTileChunks];
  __shared__ bf16x8 qs_lds[kBQ * 16];  // this workgroup's queries, 32 KiB

  const int nqb = (n + kBQ - 1) / kBQ;
  const int total = nqb * kHeads;  // multiple of 8
  const int lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int head = lin / nqb;
  const int qb = lin % nqb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int hoff = head * kHeadDim;

  // Q of this wave's 32 rows goes to LDS once (same layout as a K tile, 16
  // rows per 4 KiB... 32 rows = 8 KiB per wave); the Q^T fragments (B
  // operand: query row lr, dims 16 s + 8 lh .. +8) are re-read per tile,
  // which keeps them out of the register file.
  {
    const int sub = lane >> 4, pc = lane & 15;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int row = 4 * b + sub;  // 0..31 within the wave
      const int grow = min(qb * kBQ + wave * 32 + row, n - 1);
      __builtin_amdgcn_global_load_lds(
          (const gmem_void_t*)(q + (size_t)grow * ldq + hoff + (pc ^ (row & 15)) * 8),
          (lds_void_t*)(&qs_lds[wave * 512 + b * 64]), 16, 0, 0);
    }
  }
  const bf16x8* qw = qs_lds + wave * 512;

  // Tile loads: each wave fills 2 KiB of K and 2 KiB of V per tile, 1 KiB
  // (4 key rows) per global_load_lds; lane t lands at row t/16, physical chunk
  // t%16 and so fetches the logical chunk that maps there.
  const int sub_row = lane >> 4, pchunk = lane & 15;
  constexpr int kBlk = kBKV / 4 / kWaves;  // KiB blocks of K (and of V) per wave per tile
  auto issue_tile = [&](int tile, int slot) {
    const int key0 = min(tile, (n - 1) / kBKV) * kBKV;  // a tile past the end reloads the last one
#pragma unroll
    for (int b = 0; b < kBlk; ++b) {
      const int row = (wave * kBlk + b) * 4 + sub_row;   // 0..63
      const int grow = min(key0 + row, n - 1);
      const int kc = pchunk ^ (row & 15);
      const int vc = pchunk ^ (4 * (row & 3));
      __builtin_amdgcn_global_load_lds((const gmem_void_t*)(k + (size_t)grow * ldk + hoff + kc * 8),
                                       (lds_void_t*)(&ks_lds[slot][(wave * kBlk + b) * 64]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const gmem_void_t*)(v + (size_t)grow * ldv + hoff + vc * 8),
                                       (lds_void_t*)(&vs_lds[slot][(wave * kBlk + b) * 64]), 16, 0, 0);
    }
  };
  constexpr int kLoadsPerTile = 2 * kBlk;  // per wave

  // S^T = K Q^T for one tile (two 32-key fragments, interleaved chains).
  auto scores = [&](int slot, floatx16 (&s)[2]) {
    const floatx16 zero = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 qf = qw[k_phys(lr, 2 * st + lh)];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = ks_lds[slot][k_phys(kb * 32 + lr, 2 * st + lh)];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf, st == 0 ? zero : s[kb], 0, 0, 0);
      }
    }
  };

  floatx16 oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_run = -INFINITY;  // running max (scaled, base-2 domain) of row lr
  float l_run = 0.f;        // this lane's partial row sum

  // Transpose-read geometry: within its 16-lane group (g = lane / 16, i =
  // lane % 16) a lane supplies the address of key 4h + i/4 (+ 16 j, + 8 for
  // the second half of the fragment) and head dims 32 db + 16 (g % 2) +
  // 4 (i % 4) .. +3; it receives head dim 32 db + lane % 32 of keys
  // 16 j + 4 h + {0..3} (+ 8), h = lane / 32.
  // The key rows read are tr_key + 16 j (+ 8); adding 16 j or 8 keeps
  // row & 3, so the swizzled address of every read is the j = 0 address of
  // its head-dim block plus a constant.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_key = 4 * lh + (i16 >> 2);
  const int tr_dim = 16 * (g16 & 1) + 4 * (i16 & 3);  // + 32 db
  int tr_off[4];                                        // bf16 element offsets, j = 0
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dim = 32 * db + tr_dim;
    tr_off[db] = v_phys(tr_key, dim >> 3) * 8 + (dim & 7);
  }
  auto pv = [&](int slot, const bf16x8 (&pf)[4]) {
    const bf16* base = (const bf16*)vs_lds[slot];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16* p = base + tr_off[db] + 16 * j * kHeadDim;
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(p));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(p + 8 * kHeadDim));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[db], 0, 0, 0);
      }
  };

  // Softmax of one tile: returns the probabilities as bf16 B operands and
  // updates m_run / l_run / oacc.
  auto softmax = [&](floatx16 (&s)[2], int key0, bf16x8 (&pf)[4]) {
    if (key0 + kBKV > n) {  // keys past the end get probability 0
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (key >= n) s[kb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = half_max(mx) * scale_log2;
    // The reference max may lag the true running max by up to kSlack (base 2),
    // so probabilities stay <= 2^kSlack; O and l share the reference, so the
    // result is unchanged while the rescale (a wave-wide 64-register update)
    // is only needed when some row's max jumps by more than that.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, -m_run));
        psum += p;
        pf[kb * 2 + (r >> 3)][r & 7] = to_bf16(p);
      }
    l_run += psum;
  };

  const int ntiles = (n + kBKV - 1) / kBKV;
  // Prologue: tiles 0..2 in flight, wait for 0 and 1, scores of tile 0.
#pragma unroll
  for (int t = 0; t < kNBuf; ++t) issue_tile(t, t);
  wait_vmcnt<kLoadsPerTile>();
  __syncthreads();
  floatx16 sa[2], sb[2];
  bf16x8 pf[4];
  scores(0, sa);

  // One iteration: scores of tile t+1 into `nxt` while the softmax of tile t
  // (in `cur`) runs, then P V of tile t, then the ring advances.
  // Every step is unconditional (straight-line loop body): a tile index past
  // the end reloads the last tile, and a step on such a tile masks all of its
  // keys, so it adds nothing.  Steps come in pairs (the score buffers swap
  // roles), so an odd tile count runs one fully masked step.
  auto step = [&](int t, floatx16 (&cur)[2], floatx16 (&nxt)[2]) {
    scores((t + 1) % kNBuf, nxt);
    softmax(cur, t * kBKV, pf);
    pv(t % kNBuf, pf);
    // Tile t+2 (the last one issued) landed; after the barrier every wave is
    // done with slot t % 3, which takes tile t+3.
    wait_vmcnt<0>();
    __syncthreads();
    issue_tile(t + kNBuf, t % kNBuf);
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sa, sb);
    step(t + 1, sb, sa);
  }
  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends

  // Normalise and store: lane holds query row lr, dims db*32 + 8 g + 4 lh + 0..3.
  const float inv = 1.0f / half_sum(l_run);
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
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(nqb * kHeads), dim3(kBQ * 2), 0, st, q, ldq, k, ldk, v, ldv,
                     o, ldo, n, scale_log2);
}

}  // namespace flux3
