/*
 * flux3_dit — the FLUX.3 Image Klein denoiser transformer on AMD Instinct
 * MI355X (gfx950): C ABI.
 *
 * Sources (cited by page title and section):
 *   [blog]  "Welcome FLUX.3 Image Klein in Diffusers" (Hugging Face blog),
 *           sections "Two stages", "Inside one block", "Every token gets its
 *           own timestep", "Positions in four dimensions", "The denoising loop".
 *   [issue] "[Feature] FLUX.3 Image Klein support #2142" (stable-diffusion.cpp
 *           issue): the part/size table of the description and the comment's
 *           subsections "Tensor names (distilled checkpoint)", "Structure
 *           (from dit.py)", "Sampling (sampling.py, pipeline.py)".
 *
 * Conventions shared by every entry point
 *   - bf16 values are passed as uint16_t bit patterns; fp32 as float.
 *   - Matrices are row-major.  Weights keep the checkpoint's [out, in] shape,
 *     so every projection is Y = X W^T.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory owned by the caller.  The library
 *     never frees or keeps a caller's pointer after a call returns.
 *   - Device pointers must be 16-byte aligned; leading dimensions are in
 *     elements and must be multiples of 8.
 *   - Every call that takes a hipStream_t only enqueues work on that stream
 *     (the null stream is allowed) and returns without synchronising.
 *   - Errors: every int-returning call returns FLUX3_OK (0) or a FLUX3_E*
 *     code and never aborts.  flux3_last_error() gives a message for the last
 *     failing call of the calling thread.  On error nothing was enqueued,
 *     except FLUX3_EHIP, which reports a HIP launch failure.
 *   - Token order inside one sample is image, image_cond (every reference),
 *     text.  Stage-2 results for a token do not depend on this order (the
 *     attention has no mask and positions and modulation travel with the
 *     token), see [blog] "Two stages" and [issue] "Structure".
 */
#ifndef FLUX3_DIT_H
#define FLUX3_DIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define FLUX3_OK 0
#define FLUX3_EINVAL 1        /* bad argument: null pointer, bad size, misalignment */
#define FLUX3_EUNSUPPORTED 2  /* a shape the kernels do not handle */
#define FLUX3_EWORKSPACE 3    /* workspace missing or smaller than required */
#define FLUX3_EHIP 4          /* a HIP call or kernel launch failed */

/* ---- model constants ([issue] description table and "Tensor names") ---- */
#define FLUX3_HIDDEN 3072     /* transformer width */
#define FLUX3_HEADS 24
#define FLUX3_HEAD_DIM 128
#define FLUX3_MLP_HIDDEN 9216 /* mlp_ratio 3; mlp_in produces 2 x 9216 */
#define FLUX3_LATENT_CH 128   /* one latent token = 32 VAE channels x 2x2 */
#define FLUX3_TXT_FEAT 20480  /* 8 text-encoder layers x 2560 */
#define FLUX3_TIME_DIM 256    /* sinusoidal timestep embedding width */
#define FLUX3_MAX_SEG 8       /* at most this many modulation segments per call */

/* Message for the last failing call on this thread ("" if none). */
const char* flux3_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int flux3_version(void);

/* ---- a1: positions ------------------------------------------------------
 * flux3_build_ids: position ids (t, h, w, l) of one sample, host only.
 * [blog] "Positions in four dimensions" (table) and [issue] "Structure":
 *   image token (row, col)      -> (0, 0.5*row, 0.5*col, 0)
 *   reference k token (row,col) -> (0, 0.5*row, 0.5*col, -(k+1))
 *   text token i                -> (0, 0, 0, i)
 * rows/cols are 0-based token-grid indices, row-major; text index 0-based.
 *   img_h, img_w : image token grid (>= 0 each)
 *   n_refs       : number of references; ref_hw (host, [n_refs][2]) their grids
 *   n_txt        : text tokens (>= 0)
 *   ids          : host output [N][4] fp32, N = img_h*img_w + sum(ref) + n_txt;
 *                  may be NULL to query N only
 *   n_out        : host output, N
 * Every id is an exact multiple of 1/2, so the fp32 values are exact.
 */
int flux3_build_ids(int img_h, int img_w, int n_refs, const int* ref_hw, int n_txt,
                    float* ids, int* n_out);

/* flux3_rope_table: per-token rotation table for the 4-axis RoPE, on device.
 * Axis a (t, h, w, l) owns head dims 32a..32a+31; its pair j = dims
 * (32a+2j, 32a+2j+1) is rotated by angle id_a * 10000^(-2j/32)
 * ([issue] description table: 4 axes of 32, theta 10000).
 *   ids   : device [n][4] fp32 (from flux3_build_ids)
 *   table : device output [n][64][2] fp32 = (cos, sin) per pair p = 16a + j;
 *           angles and sin/cos are evaluated in fp64, then rounded to fp32
 */
int flux3_rope_table(const float* ids, int n, float* table, hipStream_t stream);

/* ---- a2: modulation --------------------------------------------------------
 * (shift, scale, gate) = chunk3(lin . silu(vec)) for each of n_seg vectors
 * ([issue] "Tensor names": *.lin.weight [9216, 3072] = shift, scale, gate;
 * SiLU on vec as in the final layer's adaLN, a reading of [issue] "Structure").
 *   vec   : device [n_seg][3072] fp32
 *   w_lin : host array of n_seg device pointers, each [9216][3072] bf16
 *   mod   : device output [n_seg][3][3072] fp32 (shift, scale, gate)
 */
int flux3_modulate(const float* vec, const uint16_t* const* w_lin, int n_seg, float* mod,
                   hipStream_t stream);

/* ---- a3: LayerNorm + modulation --------------------------------------------
 * out = (1 + scale[m]) * LN(x) + shift[m], LN without affine, eps 1e-6, where
 * m is the segment of the row ([blog] "Inside one block"; [issue] "Structure").
 *   x       : device [n][3072] fp32 residual stream (row stride ldx)
 *   out     : device [n][3072] bf16 (row stride ldo)
 *   seg_off : host [n_seg+1] int, 0 = seg_off[0] < ... < seg_off[n_seg] = n
 *   mod     : device, segment s uses shift = mod + s*mod_stride and
 *             scale = shift + 3072 (fp32); mod_stride >= 6144
 */
int flux3_ln_modulate(const float* x, int ldx, uint16_t* out, int ldo, int n,
                      const int* seg_off, int n_seg, const float* mod, int mod_stride,
                      hipStream_t stream);

/* ---- a6: QK RMSNorm + RoPE ---------------------------------------------------
 * In place on q and k of every head ([issue] "Structure"):
 *   q <- rope(q / sqrt(mean_128(q^2) + 1e-6) * q_scale), same for k.
 *   q, k    : device [n][24][128] bf16 with row strides ldq, ldk (elements)
 *   q_scale, k_scale : device [128] bf16 (norm.query_norm / key_norm scale)
 *   table   : device rope table from flux3_rope_table, [n][64][2] fp32
 */
int flux3_qk_norm_rope(uint16_t* q, int ldq, uint16_t* k, int ldk, int n, const uint16_t* q_scale,
                       const uint16_t* k_scale, const float* table, hipStream_t stream);

/* ---- a7: attention -------------------------------------------------------------
 * o = softmax(q k^T / sqrt(128)) v per head over all n keys, no mask
 * ([blog] "Two stages": the joint blocks run one attention over the whole
 * concatenated sequence; stage-1 calls pass one stream's rows only).
 *   q, k, v : device [n][24][128] bf16, row strides ldq, ldk, ldv
 *   o       : device output [n][24][128] bf16, row stride ldo
 * fp32 accumulation; probabilities are rounded to bf16 for the P.V product.
 */
int flux3_attention(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* v,
                    int ldv, uint16_t* o, int ldo, int n, hipStream_t stream);

/* flux3_attention_ws: the same operation on a balanced schedule.  The work is
 * 24 * ceil(n/128) items (head, 128-row query block) of ceil(n/32) key tiles
 * each; flux3_attention runs one workgroup per item, two per CU (512 at a
 * time), so an item count a little past a multiple of 512 leaves most CUs
 * idle in the last round.  Here, for more than 512 items, no multiple of 512,
 * and at most three whole rounds, 512 workgroups run the whole rounds and
 * then share the leftover items' key tiles in equal runs (at least a quarter
 * of an item each, so at most five parts an item); the workgroup that finishes
 * an item's last part merges the other parts' partial softmax states (running
 * max, sum and unnormalised output, fp32) from the workspace.
 * flux3_block_forward attends this way inside its workspace.
 *   workspace: device, >= flux3_attention_workspace_size(n) bytes (0: the plain
 *              schedule, workspace may be NULL); no contents expected on entry
 *              (its counters are cleared on the stream first).  Calls that
 *              overlap on one workspace race.
 */
size_t flux3_attention_workspace_size(int n);
int flux3_attention_ws(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* v,
                       int ldv, uint16_t* o, int ldo, int n, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/* flux3_attention_noalloc: flux3_attention_ws with the workspace in static
 * device memory of the library instead of a caller buffer, for callers that
 * cannot allocate device memory (code being captured into a graph, tight
 * serving loops, harnesses that forbid hipMalloc).  Same operation, kernels
 * and results as flux3_attention_ws with a workspace.
 *   q, k, v, o, ld*, n : as flux3_attention
 * The library holds one static scratch array per GPU of
 * FLUX3_ATTENTION_SCRATCH_BYTES (about 69 MB: the balanced schedule's
 * partial states and counters), from the first call on that GPU until the
 * process ends; it allocates nothing.  The first call on a device looks the
 * array's address up (hipGetSymbolAddress), so make one call before capturing
 * a graph.  The array keeps the last call's contents; the counters are
 * cleared on the stream by each call.  Every call on one GPU shares the
 * array, so calls that overlap on one GPU (other streams, other threads)
 * race.  A row count whose schedule would need more scratch than the array
 * holds is rejected with FLUX3_EUNSUPPORTED (none does: the balanced
 * schedule is used only below 2048 items). */
#define FLUX3_ATTENTION_SCRATCH_BYTES ((size_t)512 * 2 * 16896 * 4 + 2048 * 4)
int flux3_attention_noalloc(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* v,
                            int ldv, uint16_t* o, int ldo, int n, hipStream_t stream);

/* ---- projections -------------------------------------------------------------
 * flux3_linear: Y = X W^T, fp32 accumulation, rounded to bf16 (or fp32 when
 * y_f32 is set, then y is ignored).
 *   x : device [m][k] bf16 (row stride ldx), w : device [n][k] bf16 (stride ldw)
 *   y : device [m][n] bf16 (stride ldy) or y_f32 : device [m][n] fp32
 * Requires k % 64 == 0 and n % 64 == 0 (every projection of the model does).
 */
int flux3_linear(const uint16_t* x, int ldx, const uint16_t* w, int ldw, uint16_t* y, int ldy,
                 float* y_f32, int m, int n, int k, hipStream_t stream);

/* ---- packed block weights ------------------------------------------------------
 * One block's weights in the layout the block kernels read (made once by
 * flux3_pack_block from the checkpoint tensors):
 *   w_in  [27648][3072]: rows 0..9215 = q_proj | k_proj | v_proj, rows
 *         9216.. = mlp_in with its two halves interleaved in groups of 32
 *         rows (a0..a31, b0..b31, a32..a63, b32..b63, ...), so the SwiGLU
 *         partner columns of one output tile are computed together;
 *   w_out [3072][12288]: [attn_out | mlp_out] concatenated along the input
 *         dimension, so attn_out(o) + mlp_out(h) is one product with [o | h].
 */
typedef struct flux3_block_weights {
  const uint16_t* w_in;     /* device [27648][3072] bf16 (NULL when w_in_fp8 is set) */
  const uint16_t* w_out;    /* device [3072][12288] bf16 (NULL when w_out_fp8 is set) */
  const uint16_t* q_scale;  /* device [128] bf16 */
  const uint16_t* k_scale;  /* device [128] bf16 */
  /* fp8r ([blog] "Base model and quantized variants": rowwise FP8): when set
   * (from flux3_pack_block_fp8), the block's six Linears run as rowwise
   * E4M3 products, each Linear's input quantized per token on the fly and
   * its weight per output row ([issue] "Tensor names": one scale per row of
   * each tensor). */
  const uint8_t* w_in_fp8;  /* device [27648][3072] OCP E4M3 codes */
  const float* w_in_scale;  /* device [27648] fp32 (row scales of q|k|v|mlp_in) */
  const uint8_t* w_out_fp8; /* device [3072][12288]: attn_out codes | mlp_out codes */
  const float* w_out_scale; /* device [3][3072]: attn_out row scales, mlp_out row
                             * scales, and attn_out's over mlp_out's (fp32) */
} flux3_block_weights;

#define FLUX3_W_IN_ROWS 27648
#define FLUX3_W_OUT_COLS 12288

/* flux3_pack_block: build w_in and w_out (device outputs, caller-allocated)
 * from the checkpoint's q_proj, k_proj, v_proj, attn_out [3072][3072],
 * mlp_in [18432][3072] and mlp_out [3072][9216] (all device bf16). */
int flux3_pack_block(const uint16_t* q_proj, const uint16_t* k_proj, const uint16_t* v_proj,
                     const uint16_t* attn_out, const uint16_t* mlp_in, const uint16_t* mlp_out,
                     uint16_t* w_in, uint16_t* w_out, hipStream_t stream);

/* ---- fp8r: rowwise FP8 ([blog] "Base model and quantized variants") --------------
 * A row's scale is max|row| / 448 and its codes are OCP E4M3 (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits, largest 448) of
 * row * (448 / max|row|), rounded to nearest even; scale, inverse and product
 * in fp32; a row of zeros gets scale 1.  A product of two such operands is
 * (codes_a codes_w^T) scaled by scale_a[row] * scale_w[col], accumulated in
 * fp32.
 *
 * flux3_quantize_rows_fp8: rows x [rows][cols] bf16 (ldx elements, cols a
 *   multiple of 8, 16-byte aligned rows) -> q [rows][ldq] codes (ldq a
 *   multiple of 8, q 8-byte aligned), scale [rows]. */
int flux3_quantize_rows_fp8(const uint16_t* x, int ldx, int rows, int cols, uint8_t* q, int ldq,
                            float* scale, hipStream_t stream);

/* flux3_pack_block_fp8: quantize a packed block's w_in and w_out (from
 * flux3_pack_block) into the fp8 fields' buffers (caller-allocated, sizes as
 * in flux3_block_weights): w_in per row; w_out's first 3072 columns
 * (attn_out) and its last 9216 (mlp_out) per row as two tensors, plus the
 * ratio of their row scales. */
int flux3_pack_block_fp8(const uint16_t* w_in, const uint16_t* w_out, uint8_t* w_in_fp8,
                         float* w_in_scale, uint8_t* w_out_fp8, float* w_out_scale, hipStream_t stream);

/* flux3_linear_fp8: y = (a w^T) * a_scale[row] * w_scale[col] for quantized
 * a [m][k] (lda bytes) and w [n][k] (ldw bytes), into y (bf16, ldy elements)
 * or y_f32 (exactly one non-NULL).  Requires n % 256 == 0, k % 128 == 0,
 * k >= 256, lda and ldw multiples of 16, 16-byte aligned pointers. */
int flux3_linear_fp8(const uint8_t* a, int lda, const float* a_scale, const uint8_t* w, int ldw,
                     const float* w_scale, uint16_t* y, float* y_f32, int ldy, int m, int n, int k,
                     hipStream_t stream);

/* ---- a4 + a5: the block's input projections, one fused product ------------------
 * [q | k | v] = xm [Wq; Wk; Wv]^T and h = silu(a) * b with [a | b] = xm mlp_in^T
 * ([blog] "Inside one block": q, k, v and the SwiGLU MLP all read the same
 * modulated input; [issue] "Structure": a, b = mlp_in(x_mod).chunk(2)).
 *   xm    : device [n][3072] bf16 (modulated input, contiguous rows)
 *   w_in  : device packed [27648][3072] (flux3_pack_block)
 *   qkv   : device output [n][9216] bf16 (q | k | v, contiguous rows)
 *   h     : device output [n][9216] bf16, row stride ldh (>= 9216)
 */
int flux3_block_in_proj(const uint16_t* xm, int n, const uint16_t* w_in, uint16_t* qkv, uint16_t* h,
                        int ldh, hipStream_t stream);

/* ---- a8: the block's output projection and gated residual --------------------------
 * x <- x + gate[m] * ([o | h] [attn_out | mlp_out]^T), m = segment of the row
 * ([blog] "Inside one block"; [issue] "Structure": x + gate * (attn_out(attn)
 * + mlp_out(silu(a) * b))).
 *   cat   : device [n][12288] bf16 = [o | h] (contiguous rows)
 *   w_out : device packed [3072][12288] (flux3_pack_block)
 *   x     : device [n][3072] fp32 residual stream, updated in place
 *   seg_off, n_seg, mod : as flux3_block_forward (gate = mod + s*9216 + 6144)
 */
int flux3_block_out_proj(const uint16_t* cat, int n, const uint16_t* w_out, float* x,
                         const int* seg_off, int n_seg, const float* mod, hipStream_t stream);

/* ---- a3..a8: one block -----------------------------------------------------------
 * x <- x + gate * (attn_out(attention(rope(rms(q)), rope(rms(k)), v)) +
 *                  mlp_out(silu(a) * b)),  with q, k, v, [a|b] projections of
 * h = (1 + scale) LN(x) + shift ([blog] "Inside one block"; [issue] "Structure").
 *   x        : device [n][3072] fp32 residual stream, updated in place (the
 *              residual is kept in fp32 across the 33 blocks; every GEMM
 *              operand is bf16)
 *   seg_off  : host [n_seg+1] row offsets; segment s uses mod + s*9216
 *              (shift, scale, gate) fp32 (device)
 *   table    : device rope table of these n rows
 *   workspace: device, >= flux3_block_workspace_size(n) bytes, sized for the
 *              current device (its CU count fixes the output projection's
 *              stream-K split); no initial contents needed, and calls that
 *              share a workspace must not overlap
 * Attention covers all n rows: a stage-1 call passes one stream's rows.
 */
size_t flux3_block_workspace_size(int n);
int flux3_block_forward(float* x, int n, const int* seg_off, int n_seg, const float* mod,
                        const flux3_block_weights* w, const float* table, void* workspace,
                        size_t ws_bytes, hipStream_t stream);

/* ---- conditioning ------------------------------------------------------------------
 * flux3_time_vectors: per-mode conditioning vectors ([blog] "Every token gets
 * its own timestep"; [issue] "Structure"):
 *   vec[image] = time_in(emb(sigma)), vec[other modes] = time_in(emb(0)),
 *   plus ref_time_in(emb(sigma_next)) on every mode when ref_time_in is given
 *   (the flow-map checkpoint).  emb(t) = [cos, sin](1000 t f_j),
 *   f_j = 10000^(-j/128), j < 128; time_in = Linear, SiLU, Linear (no bias).
 *   w_time   : device {in [3072][256], out [3072][3072]} bf16
 *   w_ref    : same for ref_time_in, or NULLs for the base checkpoint
 *   mode_is_image : host [n_modes] (1 for the image mode)
 *   vec      : device output [n_modes][3072] fp32
 */
int flux3_time_vectors(const uint16_t* w_time_in, const uint16_t* w_time_out,
                       const uint16_t* w_ref_in, const uint16_t* w_ref_out, float sigma,
                       float sigma_next, const int* mode_is_image, int n_modes, float* vec,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- a9..a12: the whole transformer ---------------------------------------------- */
typedef struct flux3_model_weights {
  const uint16_t* emb_in_image;       /* [3072][128] */
  const uint16_t* emb_in_image_cond;  /* [3072][128] */
  const uint16_t* txt_in;             /* [3072][20480] */
  const uint16_t* time_in_w1;         /* [3072][256] */
  const uint16_t* time_in_w2;         /* [3072][3072] */
  const uint16_t* ref_time_in_w1;     /* [3072][256], NULL for the base checkpoint */
  const uint16_t* ref_time_in_w2;     /* [3072][3072], NULL for the base checkpoint */
  const uint16_t* early_mod[3];       /* image, image_cond, txt: [9216][3072] */
  const uint16_t* single_mod[3];      /* image, image_cond, txt: [9216][3072] */
  const flux3_block_weights* early[3];/* host arrays of n_early packed blocks per mode */
  const flux3_block_weights* single;  /* host array of n_single packed blocks */
  int n_early;                        /* 5 in the checkpoint */
  int n_single;                       /* 28 in the checkpoint */
  const uint16_t* final_ada;          /* [6144][3072] adaLN_modulation.1 */
  const uint16_t* final_linear;       /* [128][3072] */
} flux3_model_weights;

/* flux3_stack_workspace_size: bytes of workspace for flux3_stack_forward
 * with these token counts. */
size_t flux3_stack_workspace_size(int n_img, int n_cond, int n_txt);

/* flux3_stack_forward: velocity of the image tokens ([blog] "Two stages";
 * [issue] "Structure"):
 *   embed (emb_in.image, emb_in.image_cond, txt_in) -> stage 1: each stream
 *   through its own n_early blocks with its early modulation, attending only
 *   to itself -> streams concatenated (image, image_cond, text) -> stage 2:
 *   n_single shared blocks, each token modulated by its stream's single
 *   modulation -> final layer on the image tokens -> v.
 *   img   : device [n_img][128] bf16 latents
 *   cond  : device [n_cond][128] bf16 reference latents (NULL if n_cond = 0)
 *   txt   : device [n_txt][20480] bf16 text features
 *   table : device rope table [n_img + n_cond + n_txt][64][2] for the ids of
 *           flux3_build_ids (same token order)
 *   sigma, sigma_next : the step's noise level and the one it jumps to
 *   v     : device output [n_img][128] fp32
 * Stage 1's streams after the image one (references, text) run on a second
 * HIP stream that the library keeps per device, forked from `stream` and
 * joined back to it before stage 2 (so the call stays ordered on `stream`;
 * under graph capture the fork and join are part of the captured graph).
 * That stream is created by the first call on a device that is not under
 * capture; until then everything runs on `stream`.
 */
int flux3_stack_forward(const flux3_model_weights* w, const uint16_t* img, int n_img,
                        const uint16_t* cond, int n_cond, const uint16_t* txt, int n_txt,
                        const float* table, float sigma, float sigma_next, float* v,
                        void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- a13: sampler update ------------------------------------------------------------
 * x <- x + (sigma_next - sigma) v, and x_bf16 <- bf16(x) for the next call
 * ([issue] "Sampling").  x, v: device [n] fp32; x_bf16: device [n] bf16.
 */
int flux3_euler_step(float* x, uint16_t* x_bf16, const float* v, int n, float sigma,
                     float sigma_next, hipStream_t stream);

/* flux3_sample: the whole flow-map sampling loop in one call ([issue]
 * "Sampling"; [blog] "The denoising loop"): for k = 0..steps-1,
 *   v = flux3_stack_forward(bf16(x), sigmas[k], sigmas[k+1]);
 *   x <- x + (sigmas[k+1] - sigmas[k]) v.
 * Everything is enqueued on `stream` (stage 1 as in flux3_stack_forward) with
 * no host synchronisation and no allocation, so the call can be captured into
 * one HIP graph by the caller (the sigmas are read on the host at call time
 * and baked into the launches).
 *   x      : device [n_img][128] fp32 latents, in/out (the final x on return)
 *   cond, txt, table : as for flux3_stack_forward, constant over the loop
 *   sigmas : host [steps+1] fp32 (e.g. from flux3_sigmas), all finite
 *   steps  : >= 0 (0 leaves x untouched)
 *   workspace : device, >= flux3_sample_workspace_size(n_img, n_cond, n_txt)
 * The conditioning vectors (time MLPs, modulations, final adaLN), which
 * depend on the sigmas only, are computed for up to eight steps at a time
 * before those steps run, each weight read once per launch for several steps.
 * The result equals steps calls of flux3_stack_forward + flux3_euler_step
 * bit for bit. */
size_t flux3_sample_workspace_size(int n_img, int n_cond, int n_txt);
int flux3_sample(const flux3_model_weights* w, float* x, int n_img, const uint16_t* cond,
                 int n_cond, const uint16_t* txt, int n_txt, const float* table,
                 const float* sigmas, int steps, void* workspace, size_t ws_bytes,
                 hipStream_t stream);

/* ---- base checkpoint: guided sampling on a two-sample pack ----------------------
 * [issue] "Sampling": the base checkpoint runs 50 steps of the same Euler update
 * with classifier-free guidance 3.5 on a pack of two samples, [empty prompt,
 * prompt], and has no ref_time_in.  Guidance: v = v0 + g (v1 - v0), sample 0
 * the empty prompt, sample 1 the prompt (the usual formula; the pages give the
 * scale only).  Both samples share the image latents and references.
 *
 * flux3_build_ids_cfg: ids (as flux3_build_ids) of the packed rows, host only:
 *   sample 0: image | references | text 0 (indices 0 ..),
 *   sample 1: text 1 (indices 0 ..) | image | references.
 *   ids: host [n][4] fp32 or NULL (then only *n_out is set). */
int flux3_build_ids_cfg(int img_h, int img_w, int n_refs, const int* ref_hw, int n_txt0, int n_txt1,
                        float* ids, int* n_out);

/* flux3_stack_forward_cfg: the guided velocity of one step.  The image and
 * reference streams go through stage 1 once (they are the same for both
 * samples); the texts run side by side, each attending to itself; stage 2 runs
 * both samples in one pass, each attending within itself; the final layer
 * gives v0 and v1, and v = v0 + guidance (v1 - v0).  The reference and text
 * streams' stage 1 runs on the library's side stream as in
 * flux3_stack_forward.
 *   w        : model weights; ref_time_in NULL for the base checkpoint (if
 *              given, ref_time_in(emb(sigma_next)) is added as in the flow map)
 *   img      : device [n_img][128] bf16;  cond: device [n_cond][128] or NULL
 *   txt0/txt1: device [n_txt][20480] bf16 (empty prompt / prompt)
 *   table    : device rope table of the flux3_build_ids_cfg ids
 *   v        : device output [n_img][128] fp32
 *   workspace: device, >= flux3_stack_cfg_workspace_size(...) */
size_t flux3_stack_cfg_workspace_size(int n_img, int n_cond, int n_txt0, int n_txt1);
int flux3_stack_forward_cfg(const flux3_model_weights* w, const uint16_t* img, int n_img,
                            const uint16_t* cond, int n_cond, const uint16_t* txt0, int n_txt0,
                            const uint16_t* txt1, int n_txt1, const float* table, float sigma,
                            float sigma_next, float guidance, float* v, void* workspace,
                            size_t ws_bytes, hipStream_t stream);

/* flux3_sample_cfg: the whole guided loop in one call: for k < steps,
 * v = flux3_stack_forward_cfg(bf16(x), sigmas[k], sigmas[k+1], guidance),
 * x <- x + (sigmas[k+1] - sigmas[k]) v.  As flux3_sample: no host
 * synchronisation, no allocation, capturable into one HIP graph.
 *   x: device [n_img][128] fp32 in/out; sigmas: host [steps+1] fp32. */
size_t flux3_sample_cfg_workspace_size(int n_img, int n_cond, int n_txt0, int n_txt1);
int flux3_sample_cfg(const flux3_model_weights* w, float* x, int n_img, const uint16_t* cond,
                     int n_cond, const uint16_t* txt0, int n_txt0, const uint16_t* txt1, int n_txt1,
                     const float* table, const float* sigmas, int steps, float guidance,
                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* flux3_sigmas: the shifted schedule, host only ([issue] "Sampling"):
 * t_k = 1 - k/steps, sigma_k = alpha t_k / (1 + (alpha - 1) t_k), k = 0..steps.
 *   out: host [steps+1] fp32 (computed in fp64). */
int flux3_sigmas(int steps, double alpha, float* out);

/* ---- launch timing (profiling) -------------------------------------------------------
 * Measures the block's kernels where they actually run: inside
 * flux3_block_forward, flux3_stack_forward(_cfg) and flux3_sample(_cfg), on
 * whichever stream each launch is made (the caller's, or the library's own
 * stage-1 side stream).  Not a step of the pages' method: an instrument for
 * per-kernel rooflines of a whole stack step.
 *
 * flux3_timer_start: arm the timer for the kinds in the bit mask `kinds`
 * (1 << FLUX3_TIMER_*) and up to `capacity` launches.  Creates 2 x capacity
 * timing HIP events.  While armed, each launch of an armed kind records one
 * event before it and one after it on its stream; launches past `capacity`
 * and launches on a stream under graph capture are not recorded.  One timer
 * per process; FLUX3_EINVAL if it is already armed, kinds is 0 or capacity is
 * outside 1..1048576.  Recording adds two event packets per timed launch to
 * the stream.
 *
 * flux3_timer_stop: disarm, wait for every recorded event, and write per
 * launch, in launch order: ms[i] = elapsed time between its two events,
 * kind[i] = FLUX3_TIMER_*, rows[i] = the rows (tokens) of the launch.
 * Host arrays of `capacity` entries (each may be NULL); *count = entries
 * written, min(launches recorded, capacity).  Destroys the events and
 * disarms even when it fails.  FLUX3_EINVAL if the timer is not armed;
 * FLUX3_EHIP if an event could not be read (its entry is 0). */
#define FLUX3_TIMER_IN_PROJ 0       /* a4 + a5: the fused input projection (bf16 blocks of at
                                       most 128 or over 256 rows: with a6 in its epilogue) */
#define FLUX3_TIMER_QK_NORM_ROPE 1  /* a6 where it runs as a kernel of its own (bf16 blocks of
                                       129..256 rows, fp8r blocks) */
#define FLUX3_TIMER_ATTENTION 2     /* a7, every row group of the call */
#define FLUX3_TIMER_OUT_PROJ 3      /* a8, with its split-K reduce when one runs (at most 128
                                       rows, inside a stage: with the next block's a3) */
#define FLUX3_TIMER_LN_MODULATE 4   /* a3 where it runs as a kernel of its own */
int flux3_timer_start(unsigned kinds, int capacity);
int flux3_timer_stop(float* ms, int* kind, int* rows, int capacity, int* count);

#ifdef __cplusplus
}
#endif

#endif /* FLUX3_DIT_H */
