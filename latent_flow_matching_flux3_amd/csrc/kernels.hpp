// Internal launch interface between the C ABI and the kernels.
#pragma once

#include "common.hpp"

namespace flux3 {

struct GemvBatch {
  const bf16* w[kMaxSeg];
  const float* x[kMaxSeg];
  float* y[kMaxSeg];
};

// Epilogue selector of the bf16 MFMA GEMM  C = A B^T  (A [M][K], B [N][K]).
enum class GemmEpi {
  kStoreBf16,     // C bf16 [M][N], stride ldc
  kStoreF32,      // C fp32 [M][N], stride ldc
  kInProj,        // cols < 9216: q|k|v store; cols >= 9216: SwiGLU of interleaved a/b -> h
  kGatedResidual,  // x[row][col] += gate[seg(row)][col] * acc, x fp32
  // One of ksplit K ranges of a kGatedResidual or kStoreF32 product: the
  // fp32 partial product goes to rows split * Mpad + row of C (Mpad = M
  // rounded up to the tile height); a reduction kernel then adds
  // gate * (sum of the partials) to x, or stores the sum.
  kSplitPartial
};

struct GemmArgs {
  const bf16* A;
  int lda;
  const bf16* B;
  int ldb;
  int M, N, K;
  GemmEpi epi;
  // kStoreBf16 / kStoreF32 / kInProj(q|k|v part) / kGatedResidual (x)
  void* C;
  int ldc;
  // kInProj: h output (bf16, stride ldh)
  bf16* H;
  int ldh;
  // kGatedResidual: gate of segment s at mod + s * mod_stride + gate_offset
  const float* mod;
  int mod_stride;
  int gate_offset;
  SegTable seg;
  // kGatedResidual / kStoreF32: optional scratch that lets a product with too
  // few tiles to fill the chip be split over K (null: no split).
  void* split_ws;
  size_t split_ws_bytes;
  // kSplitPartial: number of K ranges (divides K / 32)
  int ksplit;
  // fp8 products (gemm_fp8.hip): A8 [M][lda], B8 [N][ldb] E4M3 codes; the
  // product of row r and column c is scaled by a_scale[r] * w_scale[c].
  const uint8_t* A8;
  const uint8_t* B8;
  const float* a_scale;
  const float* w_scale;
  // fp8 products over two Linears side by side along K (the block's
  // [o | h] against [attn_out | mlp_out]): K columns below k_part belong to
  // the first, whose products are scaled by a_scale0[r] * w_scale0[c]; the
  // rest by a_scale[r] * w_scale[c].  a_ratio = a_scale0 / a_scale per row
  // and w_ratio = w_scale0 / w_scale per column (k_part = 0: one Linear).
  int k_part;
  const float* a_scale0;
  const float* w_scale0;
  const float* a_ratio;
  const float* w_ratio;
  // kGatedResidual on 256x256 tiles: optional stream-K scratch (gemm_sk_ws_bytes,
  // carved by gemm_sk_carve).  Every workgroup then takes an equal run of the
  // product's K slices in tile order, and a tile split between workgroups is
  // finished by the last of its parts to arrive.  sk_cnt: one arrival counter
  // per (tile, wave), zero before a launch and zero again after it; sk_part:
  // the parts' fp32 partial products.  Null: whole tiles per workgroup.
  int* sk_cnt;
  float* sk_part;
  size_t sk_bytes;
  // stream-K: tile rows per group of its tile order (0: 3)
  int group_m;
  // kInProj where gemm_fuses_qk_norm holds: optional QK RMSNorm + RoPE in
  // the epilogue (q_scale / k_scale bf16 [128], rope_table [M][64][2] as for
  // launch_qk_norm_rope): the q and k columns are stored normalised and
  // rotated, so no separate norm kernel runs.  Null: plain q | k | v stores.
  // zero[0 .. nzero), if given, is cleared by the 256x256 kernel's first
  // workgroup (the counters launch_qk_norm_rope would otherwise clear; the
  // skinny kernel clears none).
  const bf16* qk_scale_q;
  const bf16* qk_scale_k;
  const float* rope_table;
  int* zero;
  int nzero;
  // kGatedResidual on the skinny kernel split over K: optional output of the
  // next block's LayerNorm + modulation of the updated rows (same mod and
  // segments: shift at mod + s * mod_stride, scale 3072 further), bf16 with
  // row stride ln_ldo, written by the reduce (gemm_fuses_next_ln tells when).
  bf16* ln_out;
  int ln_ldo;
};

// Scratch bytes a kGatedResidual or kStoreF32 product of this shape uses when
// split over K (0: it is not split).
size_t gemm_split_ws_bytes(int m, int n, int k);
// Stream-K scratch of a kGatedResidual product of this shape on this device:
// 0 where the whole tiles already fill the CUs evenly (or too few tiles for
// a split), else counters (gemm_sk_counters of them, first) and partial
// slots.  The counters must be zero before the first launch.
size_t gemm_sk_ws_bytes(int m, int n, int k);
// True where launch_gemm runs the skinny kernel (M <= 128 rows).
bool gemm_skinny_used(int m, int n, int k);
// True where a kInProj product of this shape runs on a kernel whose
// epilogue applies the QK norm (GemmArgs::rope_table): the skinny kernel, or
// the 256x256 kernel (each wave's 128 columns of q or k are one head).
bool gemm_fuses_qk_norm(int m, int n, int k);
// True where that kernel is the 256x256 one (it clears GemmArgs::zero).
bool gemm_ring_used(int m, int n, int k);
// True where a kGatedResidual product of this shape, lent `scratch_bytes` of
// split scratch, runs split over K on the skinny kernel and so applies
// GemmArgs::ln_out in its reduce.
bool gemm_fuses_next_ln(int m, int n, int k, size_t scratch_bytes);
int gemm_sk_counters(int m, int n, int k);

// fp8 (E4M3, rowwise-scaled) products: shapes the kernel takes, and launch.
bool gemm_fp8_shape_ok(int m, int n, int k);
void launch_gemm_fp8(const GemmArgs& g, hipStream_t st);
void launch_ln_modulate_fp8(const float* x, int ldx, uint8_t* out, int ldo, float* scale, int n,
                            const SegTable& seg, const float* mod, int mod_stride, hipStream_t st);
void launch_quant_rows_fp8(const bf16* x, int ldx, int rows, int cols, uint8_t* out, int ldo,
                           float* scale, hipStream_t st);
// Rows of the block's [o | h] (12288 wide): the first 3072 and the last 9216
// values quantized as two rows of their own: codes, scale0 (o), scale1 (h)
// and ratio = scale0 / scale1 per row.
void launch_quant_cat_fp8(const bf16* x, int ldx, int rows, uint8_t* out, int ldo, float* scale0,
                          float* scale1, float* ratio, hipStream_t st);
// out[i] = a[i] / b[i] (fp32 division), i < n.
void launch_scale_ratio(const float* a, const float* b, float* out, int n, hipStream_t st);

void launch_ln_modulate(const float* x, int ldx, bf16* out, int ldo, int n, const SegTable& seg,
                        const float* mod, int mod_stride, hipStream_t st);
void launch_rope_table(const float* ids, int n, float* table, hipStream_t st);
// zero[0 .. nzero) is cleared on the way (the split attention's counters).
void launch_qk_norm_rope(bf16* q, int ldq, bf16* k, int ldk, int n, const bf16* q_scale,
                         const bf16* k_scale, const float* table, hipStream_t st, int* zero = nullptr,
                         int nzero = 0);
// split_ws: attn_split_ws_bytes(n') bytes for some n' >= n, whose counters
// (attn_split_counters) are zero; they are zero again when the launch ends.
// With split_ws == nullptr (or a row count that fills whole rounds of
// workgroups) every workgroup takes whole items.
void launch_attention(const bf16* q, int ldq, const bf16* k, int ldk, const bf16* v, int ldv,
                      bf16* o, int ldo, int n, hipStream_t st, void* split_ws = nullptr);
// The balanced schedule is used for n (given a workspace); the workspace
// (attn_split_ws_bytes) is sized for every row count up to n.
bool attn_split_used(int n);
size_t attn_split_ws_bytes(int n);
// The largest workspace the balanced schedule uses, over every n: partial
// states of 512 runs (two sides of 16896 floats each) plus one counter per
// item; it runs only below four whole rounds of items (fewer than 2048).
constexpr size_t kAttnSplitMaxBytes = (size_t)512 * 2 * 16896 * 4 + 2048 * 4;
int* attn_split_counters(void* ws);
int attn_split_counter_count(int n);
void launch_zero_ints(int* p, int n, hipStream_t st);
void launch_gemm(const GemmArgs& a, hipStream_t st);
struct Timesteps {
  float t[4];
};
void launch_timestep_embedding(const Timesteps& ts, int nt, float* out, hipStream_t st);
void launch_gemv(const GemvBatch& batch, int nb, int rows, int K, bool silu_x, bool accumulate,
                 hipStream_t st);
void launch_cfg_combine(const float* vu, const float* vc, float* v, int n, float g, hipStream_t st);
void launch_euler(float* x, bf16* xb, const float* v, int n, float dt, hipStream_t st);
void launch_pack_block(const bf16* wq, const bf16* wk, const bf16* wv, const bf16* wo,
                       const bf16* w_mlp_in, const bf16* w_mlp_out, bf16* w_in, bf16* w_out,
                       hipStream_t st);

}  // namespace flux3
