// Flash-style attention forward: o = softmax(q k^T / sqrt(128)) v per head,
// unmasked over all n rows ("Welcome FLUX.3 Image Klein in Diffusers", §Two
// stages: the joint blocks put the whole concatenated sequence in one
// attention; a stage-1 call passes one stream's rows).
//
// Design (gfx950, head_dim 128):
//   - One workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//     query rows.  Two workgroups share a CU (80 KiB of LDS and at most 256
//     registers per lane each), so each SIMD runs two waves of different
//     workgroups: their per-tile barriers are independent, and one wave's
//     softmax (VALU) overlaps the other's MFMAs.
//   - K and V are walked in 32-key tiles through a 5-slot LDS ring, filled
//     straight from global memory (global_load_lds_dwordx4), three to four
//     tiles ahead.
//   - Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = K from LDS, B = Q^T held in registers for
//     the whole kernel.  A lane then holds one query row (lane % 32) and 16 of
//     the tile's 32 keys, so the row max and row sum are per-lane register
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
//   - Balanced schedule (given a workspace, at 1-3 whole rounds of items plus
//     a part round): the whole rounds as above, then the leftover items' key
//     tiles in equal runs over all 512 workgroups; an item's parts are merged
//     by the workgroup that finishes last (exact: the partial states carry
//     their own reference max).
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace flux3 {

namespace {

constexpr int kBQ = 128;   // query rows per workgroup (4 waves x 32)
constexpr int kWaves = kBQ / 32;
constexpr int kBKV = 32;   // keys per tile
constexpr int kNBuf = 5;   // LDS ring slots
constexpr int kTileChunks = kBKV * 16;  // 16-byte chunks of a 32 x 128 bf16 tile (8 KiB)
constexpr float kSlack = 8.0f;          // allowed lag of the softmax reference max (log2 units)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gmem_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// LDS layouts (64 banks x 4 bytes).  Rows are keys, 256 bytes = 16 chunks of
// 16 bytes.
//   K: an operand read puts 16 consecutive rows, same logical chunk, in one
//      16-lane group: chunk c of row r at c ^ (r & 15).
//   V: a transpose read by 32 lanes touches 4 key rows (keys 4a .. 4a+3),
//      64 bytes each at the same offset: the 64-byte quarter q of row r is
//      stored at q ^ (r & 3), i.e. 16-byte chunk c at c ^ 4 (r & 3).
__device__ __forceinline__ int k_phys(int row, int c) { return row * 16 + (c ^ (row & 15)); }
__device__ __forceinline__ int v_phys(int row, int c) { return row * 16 + (c ^ (4 * (row & 3))); }

// max(x, x of lane ^ 32) with v_permlane32_swap (VALU, no LDS round trip).
// After the swap a = [x_lo | x_lo] and b = [x_hi | x_hi].  Written as one asm
// block: this compiler's folding of the builtin with two copies of the same
// value drops half of the result.  The nops give the cross-lane read of the
// just-written copy, and the max's read of the swap results, their wait states.
__device__ __forceinline__ float half_max(float x) {
  float a = x, b;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(a), "=&v"(b));
  return a;
}
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32, 64); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Partial softmax state of one part of a split item: the 64 accumulator
// registers as 16 groups of four (each group a 16-byte value per thread,
// thread-contiguous), then the row's reference max and partial sum, one value
// per thread.
constexpr int kPartFloats = 64 * kBQ * 2 + 2 * kBQ * 2;

// SPLIT = false: one workgroup per (head, 128-row query block) item, all keys.
// SPLIT = true (items > gridDim.x = 512, not a multiple of it): `rounds` whole
// rounds of items, item r * gridDim.x + slot in round r, then the leftover
// items' key tiles, item-major, cut into runs of `units` tiles (>= a quarter
// of an item, so an item has at most five parts); run j belongs to the slot at
// position j % band of XCD band j / band, so neighbouring runs (parts of one
// item, one head) share an XCD and its L2.  Each part writes its partial state
// to `part`, and the workgroup that brings cnt[item] to the item's part count
// merges all the states in part order, stores the rows and resets the
// counter.
template <bool SPLIT>
__global__ __launch_bounds__(kBQ * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const bf16* __restrict__ q, int ldq, const bf16* __restrict__ k, int ldk,
                     const bf16* __restrict__ v, int ldv, bf16* __restrict__ o, int ldo, int n,
                     float scale_log2, float* __restrict__ part, int* __restrict__ cnt, int rounds,
                     int units, int band) {
  // One LDS object for both rings: with several, the compiler gives each its
  // own alias scope and then waits for every tile load in flight before any
  // LDS read that may alias one (the explicit waits below are exact).
  __shared__ bf16x8 ring_lds[2 * kNBuf * kTileChunks];
  bf16x8 (*ks_lds)[kTileChunks] = (bf16x8 (*)[kTileChunks])ring_lds;
  bf16x8 (*vs_lds)[kTileChunks] = (bf16x8 (*)[kTileChunks])(ring_lds + kNBuf * kTileChunks);

  const int nqb = (n + kBQ - 1) / kBQ;
  const int ntiles = (n + kBKV - 1) / kBKV;
  // Virtual slot: consecutive slots share an XCD (workgroup b runs on XCD b % 8).
  const int band_len = gridDim.x >> 3;
  const int vslot = (blockIdx.x & 7) * band_len + (blockIdx.x >> 3);
  int r = 0;               // whole rounds done
  int run = 0, u = 0, u_end = 0;  // the leftover run: units [u, u_end)
  if constexpr (SPLIT) {
    const int pos = vslot % band_len;
    run = (vslot / band_len) * band + pos;
    if (pos < band) {
      u = run * units;
      u_end = min(u + units, (nqb * kHeads - rounds * (int)gridDim.x) * ntiles);
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int sub_row = lane >> 4, pchunk = lane & 15;
  const unsigned lds_base = (unsigned)(size_t)(lds_void_t*)ring_lds;

  for (;;) {
    int item, k_lo, k_hi;  // this part: key tiles [k_lo, k_hi) of item
    if (!SPLIT) {
      item = vslot;
      k_lo = 0;
      k_hi = ntiles;
    } else if (r < rounds) {
      item = r++ * (int)gridDim.x + vslot;
      k_lo = 0;
      k_hi = ntiles;
    } else {
      if (u >= u_end) return;
      const int it = u / ntiles;
      item = rounds * (int)gridDim.x + it;
      k_lo = u - it * ntiles;
      k_hi = min(ntiles, k_lo + (u_end - u));
      u += k_hi - k_lo;
    }
    const int kend = min(n, k_hi * kBKV);           // keys at or past kend are masked
    const int head = item / nqb;
    const int qb = item - head * nqb;
    const int hoff = head * kHeadDim;

    // Q^T fragments of this wave's 32 rows, in registers for the whole part:
    // the B operand of k-step st is query row lr, dims 16 st + 8 lh .. +8.
    bf16x8 qf[8];
    {
      const int grow = min(qb * kBQ + wave * 32 + lr, n - 1);
      const bf16x8* qp = (const bf16x8*)(q + (size_t)grow * ldq + hoff);
#pragma unroll
      for (int st = 0; st < 8; ++st) qf[st] = qp[2 * st + lh];
    }

    // Tile loads: each wave fills 2 KiB of K and 2 KiB of V per tile, 1 KiB
    // (4 key rows) per global_load_lds_dwordx4; lane t lands at row t/16,
    // physical chunk t%16 and so fetches the logical chunk that maps there.
    // The source is a scalar base (the tile's first key row) plus a fixed
    // 32-bit lane offset; a partial last tile uses lane offsets whose rows are
    // clamped to the last key.  The loads are inline assembly (m0 set, one wait
    // state, load; no register results): the explicit waits and barriers below
    // order them against the LDS reads, and the compiler then adds no waits of
    // its own.
    constexpr int kBlk = kBKV / 4 / kWaves;  // KiB blocks of K (and of V) per wave per tile
    const int last_tile = (n - 1) / kBKV;
    const int last_rows = n - last_tile * kBKV;  // keys in the last tile (1 .. 32)
    unsigned voff_k[kBlk], voff_v[kBlk], voff_kl[kBlk], voff_vl[kBlk];
#pragma unroll
    for (int b = 0; b < kBlk; ++b) {
      const int row = (wave * kBlk + b) * 4 + sub_row;  // 0..31
      const int rl = min(row, last_rows - 1);
      const int kc = pchunk ^ (row & 15);
      const int vc = pchunk ^ (4 * (row & 3));
      voff_k[b] = (unsigned)((row * ldk + hoff + kc * 8) * 2);
      voff_v[b] = (unsigned)((row * ldv + hoff + vc * 8) * 2);
      voff_kl[b] = (unsigned)((rl * ldk + hoff + kc * 8) * 2);
      voff_vl[b] = (unsigned)((rl * ldv + hoff + vc * 8) * 2);
    }
    auto dma = [&](unsigned voff, const void* base, unsigned dst) __attribute__((always_inline)) {
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(base), "s"(dst) : "m0");
    };
    auto issue_tile = [&](int tile, auto SLOT) __attribute__((always_inline)) {
      constexpr int slot = decltype(SLOT)::value;
      const int tt = min(tile, k_hi - 1);  // a tile past the part's end reloads its last one
      const char* kb = (const char*)(k + (size_t)tt * kBKV * ldk);
      const char* vb = (const char*)(v + (size_t)tt * kBKV * ldv);
      const unsigned dk = lds_base + (unsigned)(slot * kTileChunks + wave * kBlk * 64) * 16u;
      const unsigned dv = dk + (unsigned)(kNBuf * kTileChunks) * 16u;
      if (tt == last_tile) {
#pragma unroll
        for (int b = 0; b < kBlk; ++b) {
          dma(voff_kl[b], kb, dk + b * 1024u);
          dma(voff_vl[b], vb, dv + b * 1024u);
        }
      } else {
#pragma unroll
        for (int b = 0; b < kBlk; ++b) {
          dma(voff_k[b], kb, dk + b * 1024u);
          dma(voff_v[b], vb, dv + b * 1024u);
        }
      }
    };
    constexpr int kLoadsPerTile = 2 * kBlk;  // per wave

    // S^T = K Q^T for one tile (one 32-key fragment).
    auto scores = [&](int slot, floatx16& s) {
      const floatx16 zero = {};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 a = ks_lds[slot][k_phys(lr, 2 * st + lh)];
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], st == 0 ? zero : s, 0, 0, 0);
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
    // its head-dim block in slot 0 plus a constant (the slot's offset and
    // 2048 bytes per 8 keys), which goes into the instruction's offset field.
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_key = 4 * lh + (i16 >> 2);
    const int tr_dim = 16 * (g16 & 1) + 4 * (i16 & 3);  // + 32 db
    unsigned tr_addr[4];                                 // LDS byte addresses, slot 0, j = 0
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dim = 32 * db + tr_dim;
      tr_addr[db] = lds_base + (unsigned)(kNBuf * kTileChunks) * 16u +
                    2u * (unsigned)(v_phys(tr_key, dim >> 3) * 8 + (dim & 7));
    }
    // The 16 transpose reads of a tile (4 head-dim blocks x 2 key groups x two
    // 8-key halves) are issued as one batch and waited for inside the same asm
    // block.  Through the builtin, the compiler would wait for every tile load
    // in flight before the first of them; the explicit waits and barriers below
    // already order them after the tile's data landed.
    auto pv = [&](auto SLOT, const bf16x8 (&pf)[2]) __attribute__((always_inline)) {
      constexpr int o0 = decltype(SLOT)::value * kTileChunks * 16;
      short4_t r[4][4];  // [db][j * 2 + half]
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
          "ds_read_b64_tr_b16 %1, %16 offset:%21\n\t"
          "ds_read_b64_tr_b16 %2, %16 offset:%22\n\t"
          "ds_read_b64_tr_b16 %3, %16 offset:%23\n\t"
          "ds_read_b64_tr_b16 %4, %17 offset:%20\n\t"
          "ds_read_b64_tr_b16 %5, %17 offset:%21\n\t"
          "ds_read_b64_tr_b16 %6, %17 offset:%22\n\t"
          "ds_read_b64_tr_b16 %7, %17 offset:%23\n\t"
          "ds_read_b64_tr_b16 %8, %18 offset:%20\n\t"
          "ds_read_b64_tr_b16 %9, %18 offset:%21\n\t"
          "ds_read_b64_tr_b16 %10, %18 offset:%22\n\t"
          "ds_read_b64_tr_b16 %11, %18 offset:%23\n\t"
          "ds_read_b64_tr_b16 %12, %19 offset:%20\n\t"
          "ds_read_b64_tr_b16 %13, %19 offset:%21\n\t"
          "ds_read_b64_tr_b16 %14, %19 offset:%22\n\t"
          "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]),
            "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3]),
            "=&v"(r[2][0]), "=&v"(r[2][1]), "=&v"(r[2][2]), "=&v"(r[2][3]),
            "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[3][2]), "=&v"(r[3][3])
          : "v"(tr_addr[0]), "v"(tr_addr[1]), "v"(tr_addr[2]), "v"(tr_addr[3]),
            "i"(o0), "i"(o0 + 2048), "i"(o0 + 4096), "i"(o0 + 6144)
          : "memory");
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(r[db][2 * j], r[db][2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[db], 0, 0, 0);
        }
    };

    // Softmax of tile t, first part: mask keys past the end, row max, and the
    // (rare) move of the reference max with the rescale of O and l.  Both tests
    // are wave-uniform branches, kept ahead of the branch-free part below.
    auto softmax_head = [&](floatx16& s, int key0) {
      if (key0 + kBKV > kend) {  // keys past the part's end get probability 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (key >= kend) s[r] = -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
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
    };

    // Prologue: tiles k_lo .. k_lo+4 in flight, wait for the first three,
    // scores of the first.  Tile t sits in ring slot (t - k_lo) % 5.
    issue_tile(k_lo, std::integral_constant<int, 0>{});
    issue_tile(k_lo + 1, std::integral_constant<int, 1>{});
    issue_tile(k_lo + 2, std::integral_constant<int, 2>{});
    issue_tile(k_lo + 3, std::integral_constant<int, 3>{});
    issue_tile(k_lo + 4, std::integral_constant<int, 4>{});
    wait_vmcnt<(kNBuf - 3) * kLoadsPerTile>();
    __syncthreads();
    floatx16 sa, sb;
    bf16x8 pf[2];
    scores(0, sa);

    // One step: scores of tile t+1 into `nxt` while the softmax of tile t (in
    // `cur`) runs, then P V of tile t.  Tile t sits in ring slot t % 5; the
    // loop below is unrolled over the ring's cycle (five pairs of steps), so
    // every slot is a compile-time constant and each LDS address is a
    // loop-invariant register plus an immediate offset.  Steps come in pairs
    // (the score buffers swap roles); a pair starts with tiles t .. t+2 landed
    // for every wave, and the ring is refilled once per pair, at its end, with
    // the two tiles whose slots the pair freed.  Every step is unconditional: a
    // tile index past the end reloads the last tile, and a step on such a tile
    // masks all of its keys, so it adds nothing; an odd tile count runs one
    // fully masked step.
    auto step = [&](int t, auto CS, floatx16& cur, floatx16& nxt) __attribute__((always_inline)) {
      constexpr int cs = decltype(CS)::value;
      constexpr int ns = (cs + 1) % kNBuf;
      // K fragments of tile t+1, read ahead of the softmax's branches.
      bf16x8 kf[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) kf[st] = ks_lds[ns][k_phys(lr, 2 * st + lh)];
      softmax_head(cur, t * kBKV);
      // One branch-free region: the score MFMAs of tile t+1 with the
      // exponentials of tile t between them (two per MFMA).
      const floatx16 zero = {};
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], st == 0 ? zero : nxt, 0, 0, 0);
#pragma unroll
        for (int r = 2 * st; r < 2 * st + 2; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(cur[r], scale_log2, -m_run));
          psum += p;
          pf[r >> 3][r & 7] = to_bf16(p);
        }
      }
      l_run += psum;
      pv(CS, pf);
    };
    auto pair = [&](int t, auto S0) __attribute__((always_inline)) {
      constexpr int s0 = decltype(S0)::value;
      constexpr int s1 = (s0 + 1) % kNBuf;
      step(t, std::integral_constant<int, s0>{}, sa, sb);
      step(t + 1, std::integral_constant<int, s1>{}, sb, sa);
      // Tiles t+3 and t+4 landed; every wave is done with the slots of tiles t
      // and t+1, which take tiles t+5 and t+6.
      wait_vmcnt<0>();
      __syncthreads();
      issue_tile(t + kNBuf, std::integral_constant<int, s0>{});
      issue_tile(t + 1 + kNBuf, std::integral_constant<int, s1>{});
    };
    for (int t = k_lo;;) {
      pair(t, std::integral_constant<int, 0>{});
      if ((t += 2) >= k_hi) break;
      pair(t, std::integral_constant<int, 2>{});
      if ((t += 2) >= k_hi) break;
      pair(t, std::integral_constant<int, 4>{});
      if ((t += 2) >= k_hi) break;
      pair(t, std::integral_constant<int, 1>{});
      if ((t += 2) >= k_hi) break;
      pair(t, std::integral_constant<int, 3>{});
      if ((t += 2) >= k_hi) break;
    }
    // No load may still be writing LDS when the part (or the workgroup) ends.
    wait_vmcnt<0>();

    if (SPLIT && (k_lo > 0 || k_hi < ntiles)) {
      // A part of a split item.  A run holds at most two partial parts: one
      // starting inside an item (its first part, side 0) and one starting at
      // an item's first tile (its last part, side 1).  The parts of an item are
      // in runs first .. last: side 1 of run first, side 0 of the others.
      const int side = k_lo > 0 ? 0 : 1;
      // The workgroups of an item may run on different XCDs, whose L2s are not
      // coherent with each other: the state goes out through stores that write
      // through to memory and comes back through loads that bypass the
      // non-coherent caches (system-coherent cache policy, SC1), so no fence
      // has to write back or invalidate a whole L2 (which would also evict the
      // K and V tiles other workgroups are streaming).  Every store is complete
      // (vmcnt 0) before the barrier and the counter is bumped after it, so the
      // workgroup that arrives last sees every state.
      constexpr int kSC1 = 16;  // buffer cache-policy bit
      const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
          part + ((size_t)run * 2 + side) * kPartFloats, (short)0, kPartFloats * 4, 0x00020000);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const floatx16& a = oacc[c >> 2];
        const int e = 4 * (c & 3);
        const u32x4 d = {__float_as_uint(a[e]), __float_as_uint(a[e + 1]), __float_as_uint(a[e + 2]),
                         __float_as_uint(a[e + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(d, mine, tid * 16, c * kBQ * 2 * 16, kSC1);
      }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), mine, tid * 4, 64 * kBQ * 2 * 4, kSC1);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_run), mine, tid * 4, 65 * kBQ * 2 * 4, kSC1);
      wait_vmcnt<0>();
      __syncthreads();
      int* flag = (int*)ring_lds;  // the count is passed on through the (drained) ring
      if (tid == 0)
        flag[0] = __hip_atomic_fetch_add(cnt + item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int arrived = flag[0];
      __syncthreads();  // every wave has read the flag before the ring is reused
      const int t0 = (item - rounds * (int)gridDim.x) * ntiles;  // the item's first leftover unit
      const int first = t0 / units, last = (t0 + ntiles - 1) / units;
      if (arrived != last - first) continue;
      // Last to arrive: merge every part's state, its own included (read
      // back), in part order, so the rounding does not depend on which part
      // finished last.  The start state (reference max -inf, sum 0, O 0)
      // takes the first part's state over exactly (factors 0 and 1).
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[c][e] = 0.f;
      for (int j = first; j <= last; ++j) {
        const __amdgpu_buffer_rsrc_t other = __builtin_amdgcn_make_buffer_rsrc(
            part + ((size_t)j * 2 + (j == first ? 1 : 0)) * kPartFloats, (short)0, kPartFloats * 4,
            0x00020000);
        const float m_o =
            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(other, tid * 4, 64 * kBQ * 2 * 4, kSC1));
        const float l_o =
            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(other, tid * 4, 65 * kBQ * 2 * 4, kSC1));
        const float m_new = fmaxf(m_run, m_o);
        const float fa = __builtin_amdgcn_exp2f(m_run - m_new);
        const float fb = __builtin_amdgcn_exp2f(m_o - m_new);
        m_run = m_new;
        l_run = l_run * fa + l_o * fb;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(other, tid * 16, c * kBQ * 2 * 16, kSC1);
          floatx16& a = oacc[c >> 2];
          const int e0 = 4 * (c & 3);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e0 + e] = a[e0 + e] * fa + __uint_as_float(t[e]) * fb;
        }
      }
      if (tid == 0) __hip_atomic_store(cnt + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

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
    if (!SPLIT) break;
  }  // parts
}

}  // namespace

namespace {

// Two workgroups on each of the 256 CUs.
constexpr int kSplitSlots = 512;

int attn_items(int n) { return (n + kBQ - 1) / kBQ * kHeads; }

struct SplitPlan {
  int rounds = 0;  // whole rounds of items
  int units = 0;   // key tiles per leftover run (0: no split)
  int band = 0;    // leftover runs per XCD band
};

// The split schedule for n rows: none where the items fill whole rounds of
// the slots, or less than one round, or where the leftover items would take
// nearly a whole round anyway.  Nor past three whole rounds: the kernel runs
// at its power limit, so a partly filled last round runs at a higher clock
// and costs less than its share of the rounds, and after many rounds the
// parts' extra loads and merges cost more than the idle slots (measured:
// 2817 rows -16%, 4096 -9%, 4608 -2%, 8272 -8%, but 20992 rows, 7 whole
// rounds, +1%).
SplitPlan attn_split_plan(int n) {
  SplitPlan p;
  const int items = attn_items(n);
  if (items <= kSplitSlots || items % kSplitSlots == 0 || items / kSplitSlots > 3) return p;
  const long T = (n + kBKV - 1) / kBKV;
  const long tail_units = (long)(items % kSplitSlots) * T;
  const long units = std::max((tail_units + kSplitSlots - 1) / kSplitSlots, (T + 3) / 4);
  if (units * 8 > T * 7) return p;
  const long runs = (tail_units + units - 1) / units;
  p.rounds = items / kSplitSlots;
  p.units = (int)units;
  p.band = (int)((runs + 7) / 8);
  return p;
}

}  // namespace

bool attn_split_used(int n) { return n > 0 && attn_split_plan(n).units > 0; }

static_assert(kAttnSplitMaxBytes == (size_t)kSplitSlots * 2 * kPartFloats * sizeof(float) +
                                        (size_t)4 * kSplitSlots * sizeof(int),
              "largest split workspace: partial states + counters of < 4 rounds of items");

size_t attn_split_ws_bytes(int n) {
  if (n <= 0 || attn_items(n) <= kSplitSlots) return 0;
  return (size_t)kSplitSlots * 2 * kPartFloats * sizeof(float) +
         ((size_t)attn_items(n) * sizeof(int) + 255) / 256 * 256;
}

int* attn_split_counters(void* ws) {
  return ws ? (int*)((char*)ws + (size_t)kSplitSlots * 2 * kPartFloats * sizeof(float)) : nullptr;
}

int attn_split_counter_count(int n) { return attn_split_ws_bytes(n) ? attn_items(n) : 0; }

namespace {
__global__ void zero_ints_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
}  // namespace

void launch_zero_ints(int* p, int n, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
}

void launch_attention(const bf16* q, int ldq, const bf16* k, int ldk, const bf16* v, int ldv,
                      bf16* o, int ldo, int n, hipStream_t st, void* split_ws) {
  if (n <= 0) return;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHeadDim);
  const SplitPlan plan = split_ws ? attn_split_plan(n) : SplitPlan{};
  if (plan.units > 0) {
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(kSplitSlots), dim3(kBQ * 2), 0, st, q, ldq, k, ldk,
                       v, ldv, o, ldo, n, scale_log2, (float*)split_ws, attn_split_counters(split_ws),
                       plan.rounds, plan.units, plan.band);
    return;
  }
  hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(attn_items(n)), dim3(kBQ * 2), 0, st, q, ldq, k, ldk,
                     v, ldv, o, ldo, n, scale_log2, nullptr, nullptr, 0, 0, 0);
}

}  // namespace flux3
