// C ABI of flux3_dit: argument checks, workspace layout and the block / stack
// drivers.  The declarations and their citations are in include/flux3_dit.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <new>

#include "../../include/flux3_dit.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace flux3;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FLUX3_EHIP, "%s: %s", what, hipGetErrorString(e));
  return FLUX3_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr && aligned16(p), FLUX3_EINVAL, "%s: null or not 16-byte aligned", #p)
#define REQUIRE_LD(ld, minv) REQUIRE((ld) >= (minv) && (ld) % 8 == 0, FLUX3_EINVAL, "%s=%d must be >= %d and a multiple of 8", #ld, (int)(ld), (int)(minv))

int make_segs(const int* seg_off, int n_seg, int n, SegTable* out) {
  REQUIRE(seg_off != nullptr, FLUX3_EINVAL, "seg_off is null");
  REQUIRE(n_seg >= 1 && n_seg <= kMaxSeg, FLUX3_EINVAL, "n_seg=%d must be in 1..%d", n_seg, kMaxSeg);
  REQUIRE(seg_off[0] == 0 && seg_off[n_seg] == n, FLUX3_EINVAL,
          "seg_off must start at 0 and end at n=%d", n);
  for (int i = 0; i < n_seg; ++i)
    REQUIRE(seg_off[i] < seg_off[i + 1], FLUX3_EINVAL, "seg_off must be strictly increasing");
  memset(out, 0, sizeof(*out));
  for (int i = 0; i <= n_seg; ++i) out->off[i] = seg_off[i];
  out->n = n_seg;
  return FLUX3_OK;
}

const bf16* B(const uint16_t* p) { return reinterpret_cast<const bf16*>(p); }
bf16* B(uint16_t* p) { return reinterpret_cast<bf16*>(p); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Block workspace: xm [n][3072] | qkv [n][9216] | cat [n][12288], bf16, then
// for fp8 blocks cat8 [n][12288] codes and four row-scale vectors [n]: the
// input's, o's, h's and o's over h's (the fp8 xm codes reuse the xm region).  The q|k|v region is dead once
// attention has run, so the output projection borrows it as scratch for a
// K-split product (sized for that too).
struct BlockWs {
  bf16* xm;
  bf16* qkv;
  size_t qkv_bytes;
  bf16* cat;
  uint8_t* cat8;
  float* scale_in;
  float* scale_o;
  float* scale_h;
  float* ratio_oh;
  void* attn_split;  // split attention's partial states and counters (or null)
  int attn_counters;
  // the output projection's stream-K counters and partial products (or null)
  int* sk_cnt;
  float* sk_part;
  size_t sk_bytes;
  // counters qk_norm_rope clears before each attention and output projection:
  // the attention's (when split) and the stream-K ones, one contiguous range
  int* zero;
  int nzero;
};

size_t qkv_region_bytes(int n) {
  return align256(std::max((size_t)n * 3 * kHidden * 2, gemm_split_ws_bytes(n, kHidden, kWOutCols)));
}

size_t block_ws_bytes(int n) {
  return align256((size_t)n * kHidden * 2) + qkv_region_bytes(n) + align256((size_t)n * kWOutCols * 2) +
         align256((size_t)n * kWOutCols) + 4 * align256((size_t)n * 4) + attn_split_ws_bytes(n) +
         gemm_sk_ws_bytes(n, kHidden, kWOutCols);
}

BlockWs carve_block_ws(void* ws, int n) {
  char* p = (char*)ws;
  BlockWs w;
  w.xm = (bf16*)p;
  p += align256((size_t)n * kHidden * 2);
  w.qkv = (bf16*)p;
  w.qkv_bytes = qkv_region_bytes(n);
  p += w.qkv_bytes;
  w.cat = (bf16*)p;
  p += align256((size_t)n * kWOutCols * 2);
  w.cat8 = (uint8_t*)p;
  p += align256((size_t)n * kWOutCols);
  w.scale_in = (float*)p;
  p += align256((size_t)n * 4);
  w.scale_o = (float*)p;
  p += align256((size_t)n * 4);
  w.scale_h = (float*)p;
  p += align256((size_t)n * 4);
  w.ratio_oh = (float*)p;
  p += align256((size_t)n * 4);
  w.attn_split = attn_split_ws_bytes(n) ? p : nullptr;
  w.attn_counters = attn_split_counter_count(n);
  p += attn_split_ws_bytes(n);
  w.sk_bytes = gemm_sk_ws_bytes(n, kHidden, kWOutCols);
  const int sk_counters = gemm_sk_counters(n, kHidden, kWOutCols);
  w.sk_cnt = w.sk_bytes ? (int*)p : nullptr;
  w.sk_part = w.sk_bytes ? (float*)(p + align256((size_t)sk_counters * 4)) : nullptr;
  // attention counters end where the stream-K counters begin
  w.zero = w.attn_split ? attn_split_counters(w.attn_split) : w.sk_cnt;
  w.nzero = w.zero ? (int)(((char*)(w.sk_bytes ? (char*)w.sk_part : p) - (char*)w.zero) / 4) : 0;
  return w;
}

int check_block_weights(const flux3_block_weights* w) {
  REQUIRE(w != nullptr, FLUX3_EINVAL, "block weights are null");
  if (w->w_in_fp8 || w->w_out_fp8) {
    REQUIRE_PTR(w->w_in_fp8);
    REQUIRE_PTR(w->w_in_scale);
    REQUIRE_PTR(w->w_out_fp8);
    REQUIRE_PTR(w->w_out_scale);
  } else {
    REQUIRE_PTR(w->w_in);
    REQUIRE_PTR(w->w_out);
  }
  REQUIRE_PTR(w->q_scale);
  REQUIRE_PTR(w->k_scale);
  return FLUX3_OK;
}

// Launch timer (flux3_timer_start / flux3_timer_stop): while armed, a
// TimedLaunch around a launch of an armed kind records one event before and
// one after it on the launch's stream.  `kinds` is read without the lock on
// every launch (0 when disarmed); slots are taken under the lock.
struct LaunchTimer {
  std::mutex mu;
  std::atomic<unsigned> kinds{0};
  hipEvent_t* ev = nullptr;  // [2 * capacity]: begin, end of slot i at 2i, 2i+1
  int* kind = nullptr;
  int* rows = nullptr;
  int capacity = 0;
  int count = 0;
};
LaunchTimer g_timer;

class TimedLaunch {
 public:
  TimedLaunch(int kind, int rows, hipStream_t st) {
    if ((g_timer.kinds.load(std::memory_order_acquire) & (1u << kind)) == 0) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    std::lock_guard<std::mutex> lock(g_timer.mu);
    if ((g_timer.kinds.load(std::memory_order_relaxed) & (1u << kind)) == 0 ||
        g_timer.count >= g_timer.capacity)
      return;
    const int i = g_timer.count;
    if (hipEventRecord(g_timer.ev[2 * i], st) != hipSuccess) return;
    g_timer.kind[i] = kind;
    g_timer.rows[i] = rows;
    g_timer.count = i + 1;
    end_ = g_timer.ev[2 * i + 1];
    st_ = st;
  }
  ~TimedLaunch() {
    if (end_ != nullptr) (void)hipEventRecord(end_, st_);
  }
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  hipEvent_t end_ = nullptr;
  hipStream_t st_ = nullptr;
};

// a4 + a5: [q | k | v] and h_mlp = silu(a) * b in one product over w_in;
// with q_scale (where gemm_fuses_qk_norm holds), also a6 on q and k in the
// epilogue, and zero[0 .. nzero) cleared on the 256x256 kernel.
void in_proj(const bf16* xm, int n, const bf16* w_in, bf16* qkv, bf16* h, int ldh, hipStream_t st,
             const bf16* q_scale = nullptr, const bf16* k_scale = nullptr, const float* table = nullptr,
             int* zero = nullptr, int nzero = 0) {
  GemmArgs g{};
  g.A = xm;
  g.lda = kHidden;
  g.B = w_in;
  g.ldb = kHidden;
  g.M = n;
  g.N = kWInRows;
  g.K = kHidden;
  g.epi = GemmEpi::kInProj;
  g.C = qkv;
  g.ldc = 3 * kHidden;
  g.H = h;
  g.ldh = ldh;
  g.qk_scale_q = q_scale;
  g.qk_scale_k = k_scale;
  g.rope_table = q_scale ? table : nullptr;
  g.zero = nzero > 0 ? zero : nullptr;
  g.nzero = nzero;
  launch_gemm(g, st);
}

// a8: x += gate * ([o | h] [W_o | W_out]^T).
void out_proj(const bf16* cat, int n, const bf16* w_out, float* x, const SegTable& seg,
              const float* mod, hipStream_t st, void* scratch = nullptr, size_t scratch_bytes = 0,
              const BlockWs* ws = nullptr, bf16* ln_out = nullptr) {
  GemmArgs o{};
  o.A = cat;
  o.lda = kWOutCols;
  o.B = w_out;
  o.ldb = kWOutCols;
  o.M = n;
  o.N = kHidden;
  o.K = kWOutCols;
  o.epi = GemmEpi::kGatedResidual;
  o.C = x;
  o.ldc = kHidden;
  o.mod = mod;
  o.mod_stride = 3 * kHidden;
  o.gate_offset = 2 * kHidden;
  o.seg = seg;
  o.split_ws = scratch;
  o.split_ws_bytes = scratch_bytes;
  if (ws != nullptr) {
    o.sk_cnt = ws->sk_cnt;
    o.sk_part = ws->sk_part;
    o.sk_bytes = ws->sk_bytes;
  }
  o.ln_out = ln_out;
  o.ln_ldo = kHidden;
  launch_gemm(o, st);
}

// a3..a8 with arguments already checked.
// attn: row groups that attend only within themselves (the samples of a
// pack, or two text streams in stage 1); nullptr = all n rows together.
// ln_ready: ws.xm already holds a3 of x (the previous block's output
// projection wrote it).  next_ln: the next block uses the same workspace,
// rows, segments and mod, so this block may write its a3 into ws.xm.
// Returns whether it did (then the next block is called with ln_ready).
bool block_forward_unchecked(float* x, int n, const SegTable& seg, const float* mod,
                             const flux3_block_weights* w, const float* table, const BlockWs& ws,
                             hipStream_t st, const SegTable* attn = nullptr, bool ln_ready = false,
                             bool next_ln = false) {
  const bool fp8 = w->w_in_fp8 != nullptr;
  // a6 in the in-projection's epilogue: on the 256x256 kernel, which also
  // clears the workspace's counters, or on the skinny kernel where there are
  // none to clear.
  const bool ring_qk = !fp8 && gemm_ring_used(n, kWInRows, kHidden);
  const bool fuse_qk = ring_qk || (!fp8 && ws.nzero == 0 && gemm_skinny_used(n, kWInRows, kHidden));
  uint8_t* const xm8 = (uint8_t*)ws.xm;
  if (fp8) {
    // a3 with the rowwise FP8 quantization fused; a4 + a5 as an fp8r product
    {
      TimedLaunch t(FLUX3_TIMER_LN_MODULATE, n, st);
      launch_ln_modulate_fp8(x, kHidden, xm8, kHidden, ws.scale_in, n, seg, mod, 3 * kHidden, st);
    }
    GemmArgs g{};
    g.A8 = xm8;
    g.lda = kHidden;
    g.B8 = w->w_in_fp8;
    g.ldb = kHidden;
    g.a_scale = ws.scale_in;
    g.w_scale = w->w_in_scale;
    g.M = n;
    g.N = kWInRows;
    g.K = kHidden;
    g.epi = GemmEpi::kInProj;
    g.C = ws.qkv;
    g.ldc = 3 * kHidden;
    g.H = ws.cat + kHidden;
    g.ldh = kWOutCols;
    TimedLaunch t(FLUX3_TIMER_IN_PROJ, n, st);
    launch_gemm_fp8(g, st);
  } else {
    // a3: h = (1 + scale) LN(x) + shift
    if (!ln_ready) {
      TimedLaunch t(FLUX3_TIMER_LN_MODULATE, n, st);
      launch_ln_modulate(x, kHidden, ws.xm, kHidden, n, seg, mod, 3 * kHidden, st);
    }
    // a4 + a5: q | k | v into qkv; SwiGLU output into the last 9216 columns of
    // cat.  Except on the mid-size kernel (129 .. 256 rows), the epilogue also
    // applies a6.
    TimedLaunch t(FLUX3_TIMER_IN_PROJ, n, st);
    if (fuse_qk)
      in_proj(ws.xm, n, B(w->w_in), ws.qkv, ws.cat + kHidden, kWOutCols, st, B(w->q_scale), B(w->k_scale),
              table, ring_qk ? ws.zero : nullptr, ring_qk ? ws.nzero : 0);
    else
      in_proj(ws.xm, n, B(w->w_in), ws.qkv, ws.cat + kHidden, kWOutCols, st);
  }
  // a6: RMSNorm + RoPE on q and k
  if (!fuse_qk) {
    TimedLaunch t(FLUX3_TIMER_QK_NORM_ROPE, n, st);
    launch_qk_norm_rope(ws.qkv, 3 * kHidden, ws.qkv + kHidden, 3 * kHidden, n, B(w->q_scale),
                        B(w->k_scale), table, st, ws.zero, ws.nzero);
  }
  // a7: attention -> first 3072 columns of cat, per row group
  {
    const int ng = attn ? attn->n : 1;
    TimedLaunch t(FLUX3_TIMER_ATTENTION, n, st);
    for (int gi = 0; gi < ng; ++gi) {
      const int r0 = attn ? attn->off[gi] : 0, r1 = attn ? attn->off[gi + 1] : n;
      if (r1 <= r0) continue;
      const bf16* q = ws.qkv + (size_t)r0 * 3 * kHidden;
      launch_attention(q, 3 * kHidden, q + kHidden, 3 * kHidden, q + 2 * kHidden, 3 * kHidden,
                       ws.cat + (size_t)r0 * kWOutCols, kWOutCols, r1 - r0, st, ws.attn_split);
    }
  }
  // a8: gated residual
  if (fp8) {
    // attn_out(o) + mlp_out(h): two Linears, each with its own scales, in
    // one product over [o | h]
    launch_quant_cat_fp8(ws.cat, kWOutCols, n, ws.cat8, kWOutCols, ws.scale_o, ws.scale_h, ws.ratio_oh,
                         st);
    GemmArgs o{};
    o.A8 = ws.cat8;
    o.lda = kWOutCols;
    o.B8 = w->w_out_fp8;
    o.ldb = kWOutCols;
    o.k_part = kHidden;
    o.a_scale0 = ws.scale_o;
    o.a_scale = ws.scale_h;
    o.a_ratio = ws.ratio_oh;
    o.w_scale0 = w->w_out_scale;
    o.w_scale = w->w_out_scale + kHidden;
    o.w_ratio = w->w_out_scale + 2 * kHidden;
    o.M = n;
    o.N = kHidden;
    o.K = kWOutCols;
    o.epi = GemmEpi::kGatedResidual;
    o.C = x;
    o.ldc = kHidden;
    o.mod = mod;
    o.mod_stride = 3 * kHidden;
    o.gate_offset = 2 * kHidden;
    o.seg = seg;
    o.split_ws = ws.qkv;
    o.split_ws_bytes = ws.qkv_bytes;
    TimedLaunch t(FLUX3_TIMER_OUT_PROJ, n, st);
    launch_gemm_fp8(o, st);
  } else {
    // products of at most 128 rows split over K: the reduce also writes the
    // next block's a3 (xm is dead once the input projection has run)
    const bool ln_next = next_ln && gemm_fuses_next_ln(n, kHidden, kWOutCols, ws.qkv_bytes);
    TimedLaunch t(FLUX3_TIMER_OUT_PROJ, n, st);
    out_proj(ws.cat, n, B(w->w_out), x, seg, mod, st, ws.qkv, ws.qkv_bytes, &ws, ln_next ? ws.xm : nullptr);
    return ln_next;
  }
  return false;
}

}  // namespace

// Scratch of flux3_attention_noalloc: the balanced attention schedule's
// workspace (partial softmax states and per-item counters) in static device
// memory, one copy per GPU, held until the process ends.  In host code
// `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[kAttnSplitMaxBytes];
static_assert(kAttnSplitMaxBytes == FLUX3_ATTENTION_SCRATCH_BYTES, "header's scratch size");

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on each device), or null with the error recorded.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(FLUX3_EHIP, "no current HIP device (or device index >= %d)", kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      fail(FLUX3_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_dev[dev] = p;
  }
  return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

const char* flux3_last_error(void) { return g_err; }

int flux3_version(void) { return 100; }

int flux3_build_ids(int img_h, int img_w, int n_refs, const int* ref_hw, int n_txt, float* ids,
                    int* n_out) {
  REQUIRE(img_h >= 0 && img_w >= 0 && n_txt >= 0 && n_refs >= 0, FLUX3_EINVAL,
          "sizes must be non-negative");
  REQUIRE(n_refs == 0 || ref_hw != nullptr, FLUX3_EINVAL, "ref_hw is null");
  REQUIRE(n_out != nullptr, FLUX3_EINVAL, "n_out is null");
  long n = (long)img_h * img_w + n_txt;
  for (int k = 0; k < n_refs; ++k) {
    REQUIRE(ref_hw[2 * k] >= 0 && ref_hw[2 * k + 1] >= 0, FLUX3_EINVAL, "bad reference grid");
    n += (long)ref_hw[2 * k] * ref_hw[2 * k + 1];
  }
  REQUIRE(n < (1L << 30), FLUX3_EINVAL, "too many tokens");
  *n_out = (int)n;
  if (!ids) return FLUX3_OK;
  float* p = ids;
  for (int r = 0; r < img_h; ++r)
    for (int c = 0; c < img_w; ++c) {
      p[0] = 0.f; p[1] = 0.5f * r; p[2] = 0.5f * c; p[3] = 0.f;
      p += 4;
    }
  for (int k = 0; k < n_refs; ++k)
    for (int r = 0; r < ref_hw[2 * k]; ++r)
      for (int c = 0; c < ref_hw[2 * k + 1]; ++c) {
        p[0] = 0.f; p[1] = 0.5f * r; p[2] = 0.5f * c; p[3] = -(float)(k + 1);
        p += 4;
      }
  for (int i = 0; i < n_txt; ++i) {
    p[0] = 0.f; p[1] = 0.f; p[2] = 0.f; p[3] = (float)i;
    p += 4;
  }
  return FLUX3_OK;
}

int flux3_rope_table(const float* ids, int n, float* table, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(ids);
  REQUIRE_PTR(table);
  launch_rope_table(ids, n, table, stream);
  return check_launch("rope_table");
}

int flux3_modulate(const float* vec, const uint16_t* const* w_lin, int n_seg, float* mod,
                   hipStream_t stream) {
  REQUIRE(n_seg >= 1 && n_seg <= kMaxSeg, FLUX3_EINVAL, "n_seg=%d must be in 1..%d", n_seg, kMaxSeg);
  REQUIRE_PTR(vec);
  REQUIRE_PTR(mod);
  REQUIRE(w_lin != nullptr, FLUX3_EINVAL, "w_lin is null");
  GemvBatch b{};
  for (int s = 0; s < n_seg; ++s) {
    REQUIRE(w_lin[s] != nullptr && aligned16(w_lin[s]), FLUX3_EINVAL, "w_lin[%d] null or misaligned", s);
    b.w[s] = B(w_lin[s]);
    b.x[s] = vec + (size_t)s * kHidden;
    b.y[s] = mod + (size_t)s * 3 * kHidden;
  }
  launch_gemv(b, n_seg, 3 * kHidden, kHidden, true, false, stream);
  return check_launch("modulate");
}

int flux3_ln_modulate(const float* x, int ldx, uint16_t* out, int ldo, int n,
                      const int* seg_off, int n_seg, const float* mod, int mod_stride,
                      hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(out);
  REQUIRE_PTR(mod);
  REQUIRE_LD(ldx, kHidden);
  REQUIRE_LD(ldo, kHidden);
  REQUIRE(mod_stride >= 2 * kHidden && mod_stride % 4 == 0, FLUX3_EINVAL, "mod_stride=%d", mod_stride);
  SegTable seg;
  int rc = make_segs(seg_off, n_seg, n, &seg);
  if (rc) return rc;
  launch_ln_modulate(x, ldx, B(out), ldo, n, seg, mod, mod_stride, stream);
  return check_launch("ln_modulate");
}

int flux3_qk_norm_rope(uint16_t* q, int ldq, uint16_t* k, int ldk, int n, const uint16_t* q_scale,
                       const uint16_t* k_scale, const float* table, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(q_scale);
  REQUIRE_PTR(k_scale);
  REQUIRE_PTR(table);
  REQUIRE_LD(ldq, kHidden);
  REQUIRE_LD(ldk, kHidden);
  launch_qk_norm_rope(B(q), ldq, B(k), ldk, n, B(q_scale), B(k_scale), table, stream);
  return check_launch("qk_norm_rope");
}

int flux3_attention(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* v,
                    int ldv, uint16_t* o, int ldo, int n, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_LD(ldq, kHidden);
  REQUIRE_LD(ldk, kHidden);
  REQUIRE_LD(ldv, kHidden);
  REQUIRE_LD(ldo, kHidden);
  launch_attention(B(q), ldq, B(k), ldk, B(v), ldv, B(o), ldo, n, stream);
  return check_launch("attention");
}

size_t flux3_attention_workspace_size(int n) { return n > 0 && attn_split_used(n) ? attn_split_ws_bytes(n) : 0; }

int flux3_attention_ws(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* v,
                       int ldv, uint16_t* o, int ldo, int n, void* workspace, size_t ws_bytes,
                       hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_LD(ldq, kHidden);
  REQUIRE_LD(ldk, kHidden);
  REQUIRE_LD(ldv, kHidden);
  REQUIRE_LD(ldo, kHidden);
  const size_t need = flux3_attention_workspace_size(n);
  REQUIRE(ws_bytes >= need, FLUX3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (need) {
    REQUIRE_PTR(workspace);
    launch_zero_ints(attn_split_counters(workspace), attn_split_counter_count(n), stream);
  }
  launch_attention(B(q), ldq, B(k), ldk, B(v), ldv, B(o), ldo, n, stream, need ? workspace : nullptr);
  return check_launch("attention");
}

int flux3_attention_noalloc(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* v,
                            int ldv, uint16_t* o, int ldo, int n, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_LD(ldq, kHidden);
  REQUIRE_LD(ldk, kHidden);
  REQUIRE_LD(ldv, kHidden);
  REQUIRE_LD(ldo, kHidden);
  const size_t need = flux3_attention_workspace_size(n);
  REQUIRE(need <= kAttnSplitMaxBytes, FLUX3_EUNSUPPORTED,
          "n=%d needs %zu bytes of scratch, more than the static %zu", n, need, kAttnSplitMaxBytes);
  void* ws = nullptr;
  if (need) {
    ws = scratch_ptr();
    if (ws == nullptr) return FLUX3_EHIP;
    // the counters must start at zero (a fill kernel, no memset node)
    launch_zero_ints(attn_split_counters(ws), attn_split_counter_count(n), stream);
  }
  launch_attention(B(q), ldq, B(k), ldk, B(v), ldv, B(o), ldo, n, stream, ws);
  return check_launch("attention_noalloc");
}

int flux3_linear(const uint16_t* x, int ldx, const uint16_t* w, int ldw, uint16_t* y, int ldy,
                 float* y_f32, int m, int n, int k, hipStream_t stream) {
  REQUIRE(m >= 0 && n > 0 && k > 0, FLUX3_EINVAL, "m=%d n=%d k=%d", m, n, k);
  REQUIRE(k % 64 == 0 && n % 64 == 0, FLUX3_EUNSUPPORTED, "k=%d and n=%d must be multiples of 64", k, n);
  if (m == 0) return FLUX3_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w);
  REQUIRE_LD(ldx, k);
  REQUIRE_LD(ldw, k);
  GemmArgs g{};
  g.A = B(x);
  g.lda = ldx;
  g.B = B(w);
  g.ldb = ldw;
  g.M = m;
  g.N = n;
  g.K = k;
  if (y_f32) {
    REQUIRE_PTR(y_f32);
    REQUIRE(ldy >= n && ldy % 4 == 0, FLUX3_EINVAL, "ldy=%d", ldy);
    g.epi = GemmEpi::kStoreF32;
    g.C = y_f32;
  } else {
    REQUIRE_PTR(y);
    REQUIRE_LD(ldy, n);
    g.epi = GemmEpi::kStoreBf16;
    g.C = y;
  }
  g.ldc = ldy;
  launch_gemm(g, stream);
  return check_launch("linear");
}

int flux3_pack_block(const uint16_t* q_proj, const uint16_t* k_proj, const uint16_t* v_proj,
                     const uint16_t* attn_out, const uint16_t* mlp_in, const uint16_t* mlp_out,
                     uint16_t* w_in, uint16_t* w_out, hipStream_t stream) {
  REQUIRE_PTR(q_proj);
  REQUIRE_PTR(k_proj);
  REQUIRE_PTR(v_proj);
  REQUIRE_PTR(attn_out);
  REQUIRE_PTR(mlp_in);
  REQUIRE_PTR(mlp_out);
  REQUIRE_PTR(w_in);
  REQUIRE_PTR(w_out);
  launch_pack_block(B(q_proj), B(k_proj), B(v_proj), B(attn_out), B(mlp_in), B(mlp_out), B(w_in),
                    B(w_out), stream);
  return check_launch("pack_block");
}

int flux3_block_in_proj(const uint16_t* xm, int n, const uint16_t* w_in, uint16_t* qkv, uint16_t* h,
                        int ldh, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(xm);
  REQUIRE_PTR(w_in);
  REQUIRE_PTR(qkv);
  REQUIRE_PTR(h);
  REQUIRE_LD(ldh, kMlp);
  in_proj(B(xm), n, B(w_in), B(qkv), B(h), ldh, stream);
  return check_launch("block_in_proj");
}

int flux3_block_out_proj(const uint16_t* cat, int n, const uint16_t* w_out, float* x,
                         const int* seg_off, int n_seg, const float* mod, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(cat);
  REQUIRE_PTR(w_out);
  REQUIRE_PTR(x);
  REQUIRE_PTR(mod);
  SegTable seg;
  int rc = make_segs(seg_off, n_seg, n, &seg);
  if (rc) return rc;
  out_proj(B(cat), n, B(w_out), x, seg, mod, stream);
  return check_launch("block_out_proj");
}

size_t flux3_block_workspace_size(int n) { return n > 0 ? block_ws_bytes(n) : 0; }

int flux3_block_forward(float* x, int n, const int* seg_off, int n_seg, const float* mod,
                        const flux3_block_weights* w, const float* table, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(mod);
  REQUIRE_PTR(table);
  int rc = check_block_weights(w);
  if (rc) return rc;
  SegTable seg;
  rc = make_segs(seg_off, n_seg, n, &seg);
  if (rc) return rc;
  REQUIRE(workspace != nullptr && aligned16(workspace), FLUX3_EWORKSPACE, "workspace missing or misaligned");
  REQUIRE(ws_bytes >= block_ws_bytes(n), FLUX3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
          block_ws_bytes(n));
  block_forward_unchecked(x, n, seg, mod, w, table, carve_block_ws(workspace, n), stream);
  return check_launch("block_forward");
}

int flux3_quantize_rows_fp8(const uint16_t* x, int ldx, int rows, int cols, uint8_t* q, int ldq,
                            float* scale, hipStream_t stream) {
  REQUIRE(rows >= 0 && cols > 0 && cols % 8 == 0, FLUX3_EINVAL, "rows=%d cols=%d", rows, cols);
  if (rows == 0) return FLUX3_OK;
  REQUIRE_PTR(x);
  REQUIRE(q != nullptr, FLUX3_EINVAL, "q is null");
  REQUIRE(scale != nullptr, FLUX3_EINVAL, "scale is null");
  REQUIRE_LD(ldx, cols);
  REQUIRE(ldq >= cols && ldq % 8 == 0 && ((uintptr_t)q & 7) == 0, FLUX3_EINVAL,
          "ldq=%d must be >= cols and a multiple of 8 (q 8-byte aligned)", ldq);
  launch_quant_rows_fp8(B(x), ldx, rows, cols, q, ldq, scale, stream);
  return check_launch("quantize_rows_fp8");
}

int flux3_pack_block_fp8(const uint16_t* w_in, const uint16_t* w_out, uint8_t* w_in_fp8,
                         float* w_in_scale, uint8_t* w_out_fp8, float* w_out_scale, hipStream_t stream) {
  REQUIRE_PTR(w_in);
  REQUIRE_PTR(w_out);
  REQUIRE_PTR(w_in_fp8);
  REQUIRE_PTR(w_out_fp8);
  REQUIRE(w_in_scale != nullptr && w_out_scale != nullptr, FLUX3_EINVAL, "scale buffers are null");
  launch_quant_rows_fp8(B(w_in), kHidden, kWInRows, kHidden, w_in_fp8, kHidden, w_in_scale, stream);
  // attn_out and mlp_out are quantized as the tensors they are, with the
  // ratio of their row scales for the product over [o | h]
  launch_quant_rows_fp8(B(w_out), kWOutCols, kHidden, kHidden, w_out_fp8, kWOutCols, w_out_scale, stream);
  launch_quant_rows_fp8(B(w_out) + kHidden, kWOutCols, kHidden, kMlp, w_out_fp8 + kHidden, kWOutCols,
                        w_out_scale + kHidden, stream);
  launch_scale_ratio(w_out_scale, w_out_scale + kHidden, w_out_scale + 2 * kHidden, kHidden, stream);
  return check_launch("pack_block_fp8");
}

int flux3_linear_fp8(const uint8_t* a, int lda, const float* a_scale, const uint8_t* w, int ldw,
                     const float* w_scale, uint16_t* y, float* y_f32, int ldy, int m, int n, int k,
                     hipStream_t stream) {
  REQUIRE(m >= 0, FLUX3_EINVAL, "m=%d", m);
  if (m == 0) return FLUX3_OK;
  REQUIRE(gemm_fp8_shape_ok(m, n, k), FLUX3_EUNSUPPORTED,
          "fp8 product needs n %% 256 == 0, k %% 128 == 0, k >= 256 (m=%d n=%d k=%d)", m, n, k);
  REQUIRE_PTR(a);
  REQUIRE_PTR(w);
  REQUIRE(a_scale != nullptr && w_scale != nullptr, FLUX3_EINVAL, "scales are null");
  REQUIRE(lda >= k && lda % 16 == 0 && ldw >= k && ldw % 16 == 0, FLUX3_EINVAL,
          "lda=%d ldw=%d must be >= k and multiples of 16", lda, ldw);
  REQUIRE((y == nullptr) != (y_f32 == nullptr), FLUX3_EINVAL, "give exactly one of y, y_f32");
  REQUIRE(y == nullptr || aligned16(y), FLUX3_EINVAL, "y misaligned");
  REQUIRE(y_f32 == nullptr || aligned16(y_f32), FLUX3_EINVAL, "y_f32 misaligned");
  REQUIRE(ldy >= n && ldy % 8 == 0, FLUX3_EINVAL, "ldy=%d", ldy);
  GemmArgs g{};
  g.A8 = a;
  g.lda = lda;
  g.B8 = w;
  g.ldb = ldw;
  g.a_scale = a_scale;
  g.w_scale = w_scale;
  g.M = m;
  g.N = n;
  g.K = k;
  g.epi = y ? GemmEpi::kStoreBf16 : GemmEpi::kStoreF32;
  g.C = y ? (void*)y : (void*)y_f32;
  g.ldc = ldy;
  launch_gemm_fp8(g, stream);
  return check_launch("linear_fp8");
}

// ---- conditioning and the whole stack -----------------------------------------------

namespace {
// Scratch of flux3_time_vectors: emb [3][256] | hidden [2][8][3072] (fp32).
constexpr size_t kTimeWsBytes = 3 * 256 * 4 + 2 * kMaxSeg * kHidden * 4;

// vec[m] = time_in(emb(t_m)) (+ ref_time_in(emb(sigma_next))), t_m = sigma for
// image, 0 otherwise.  Embeddings: index 0 = emb(sigma), 1 = emb(0),
// 2 = emb(sigma_next).
int time_vectors_unchecked(const uint16_t* w1, const uint16_t* w2, const uint16_t* r1,
                           const uint16_t* r2, float sigma, float sigma_next,
                           const int* is_image, int n_modes, float* vec, char* ws,
                           hipStream_t st) {
  float* emb = (float*)ws;
  float* hid = emb + 3 * 256;
  const Timesteps ts{{sigma, 0.f, sigma_next, 0.f}};
  launch_timestep_embedding(ts, 3, emb, st);
  GemvBatch b{};
  for (int m = 0; m < n_modes; ++m) {
    b.w[m] = B(w1);
    b.x[m] = emb + (is_image[m] ? 0 : 256);
    b.y[m] = hid + (size_t)m * kHidden;
  }
  launch_gemv(b, n_modes, kHidden, 256, false, false, st);
  for (int m = 0; m < n_modes; ++m) {
    b.w[m] = B(w2);
    b.x[m] = hid + (size_t)m * kHidden;
    b.y[m] = vec + (size_t)m * kHidden;
  }
  launch_gemv(b, n_modes, kHidden, kHidden, true, false, st);
  if (r1 && r2) {
    float* rh = hid + (size_t)kMaxSeg * kHidden;
    GemvBatch r{};
    r.w[0] = B(r1);
    r.x[0] = emb + 512;
    r.y[0] = rh;
    launch_gemv(r, 1, kHidden, 256, false, false, st);
    for (int m = 0; m < n_modes; ++m) {
      b.w[m] = B(r2);
      b.x[m] = rh;
      b.y[m] = vec + (size_t)m * kHidden;
    }
    launch_gemv(b, n_modes, kHidden, kHidden, true, true, st);
  }
  return check_launch("time_vectors");
}

// Stack workspace layout.
struct StackWs {
  float* x;         // [N][3072] fp32 residual stream, tokens image | image_cond | txt
  float* vec;       // [3][3072]
  float* mod_early; // [3][9216]
  float* mod_single;// [3][9216]
  float* mod_final; // [6144]
  char* time_ws;    // kTimeWsBytes
  void* block_ws;   // block workspace for N rows
  size_t block_ws_bytes;
  void* side_ws;    // block workspace of the stage-1 side stream (largest non-image stream)
};

// Stage 1 runs each stream on its own rows with its own blocks, so the
// non-image streams (references, text) do not depend on the image stream
// until stage 2: they run on a second HIP stream beside it and fill CUs the
// image stream's kernels leave idle (at 4096 image rows the output projection
// has 192 tiles for 256 CUs, and the attention's second round of workgroups
// is half full; at 64 + 32 rows both streams' weight streams overlap).  One
// side stream and one pair of fork / join events per device, created on
// first use, and not while the caller's stream is being captured (then
// stage 1 runs on the caller's stream alone).  side_fork takes the device's
// side-stream lock and side_join releases it: between them no other call can
// queue work on the side stream, which under capture would land in the
// caller's graph, and no other call can record the fork event in between
// (that would let this call's side work start before its inputs are ready).
// Under capture the fork's event record and wait put the side stream into the
// capture, and the join brings its work back before the capture ends.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
std::mutex g_side_mu;  // guards creation
SideStream g_side[64];

// The current device's side stream, made to wait for everything queued on
// `main` so far, with its lock held; null when there is none to use (HIP
// failure, or not created yet while `main` is being captured).
SideStream* side_fork(hipStream_t main) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(main, &cs) != hipSuccess) return nullptr;
  const bool capturing = cs != hipStreamCaptureStatusNone;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& sd = g_side[dev];
  {
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (sd.s == nullptr) {
      if (capturing) return nullptr;
      hipStream_t st = nullptr;
      hipEvent_t f = nullptr, j = nullptr;
      if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
      if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
        if (f) (void)hipEventDestroy(f);
        (void)hipStreamDestroy(st);
        return nullptr;
      }
      sd.fork = f;
      sd.join = j;
      sd.s = st;
    }
  }
  sd.mu.lock();
  if (hipEventRecord(sd.fork, main) != hipSuccess || hipStreamWaitEvent(sd.s, sd.fork, 0) != hipSuccess) {
    sd.mu.unlock();
    return nullptr;
  }
  return &sd;
}

// `main` waits for everything queued on the side stream so far; releases the
// lock side_fork took (also when it fails).
int side_join(SideStream* sd, hipStream_t main) {
  const hipError_t e = hipEventRecord(sd->join, sd->s);
  const hipError_t f = e == hipSuccess ? hipStreamWaitEvent(main, sd->join, 0) : e;
  sd->mu.unlock();
  REQUIRE(e == hipSuccess, FLUX3_EHIP, "stage-1 join record: %s", hipGetErrorString(e));
  REQUIRE(f == hipSuccess, FLUX3_EHIP, "stage-1 join wait: %s", hipGetErrorString(f));
  return FLUX3_OK;
}

// Rows of the largest stream that stage 1 may run beside the image stream.
int side_rows(int n_cond, int n_txt) { return std::max(n_cond, n_txt); }

size_t stack_ws_bytes(int n_img, int n_cond, int n_txt) {
  const int n_total = n_img + n_cond + n_txt;
  const int side = side_rows(n_cond, n_txt);
  return align256((size_t)n_total * kHidden * 4) + align256(3 * kHidden * 4) +
         2 * align256(3 * 3 * kHidden * 4) + align256(2 * kHidden * 4) + align256(kTimeWsBytes) +
         block_ws_bytes(n_total) + (side > 0 ? block_ws_bytes(side) : 0);
}

StackWs carve_stack_ws(void* ws, int n_total) {
  char* p = (char*)ws;
  StackWs s;
  s.x = (float*)p;
  p += align256((size_t)n_total * kHidden * 4);
  s.vec = (float*)p;
  p += align256(3 * kHidden * 4);
  s.mod_early = (float*)p;
  p += align256(3 * 3 * kHidden * 4);
  s.mod_single = (float*)p;
  p += align256(3 * 3 * kHidden * 4);
  s.mod_final = (float*)p;
  p += align256(2 * kHidden * 4);
  s.time_ws = p;
  p += align256(kTimeWsBytes);
  s.block_ws = p;
  s.block_ws_bytes = block_ws_bytes(n_total);
  s.side_ws = p + s.block_ws_bytes;
  return s;
}
}  // namespace

int flux3_time_vectors(const uint16_t* w_time_in, const uint16_t* w_time_out,
                       const uint16_t* w_ref_in, const uint16_t* w_ref_out, float sigma,
                       float sigma_next, const int* mode_is_image, int n_modes, float* vec,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  REQUIRE_PTR(w_time_in);
  REQUIRE_PTR(w_time_out);
  REQUIRE((w_ref_in == nullptr) == (w_ref_out == nullptr), FLUX3_EINVAL,
          "ref_time_in weights: give both or neither");
  if (w_ref_in) {
    REQUIRE_PTR(w_ref_in);
    REQUIRE_PTR(w_ref_out);
  }
  REQUIRE(n_modes >= 1 && n_modes <= kMaxSeg, FLUX3_EINVAL, "n_modes=%d", n_modes);
  REQUIRE(mode_is_image != nullptr, FLUX3_EINVAL, "mode_is_image is null");
  REQUIRE_PTR(vec);
  REQUIRE(workspace != nullptr && aligned16(workspace) && ws_bytes >= kTimeWsBytes,
          FLUX3_EWORKSPACE, "time_vectors needs %zu bytes of workspace", kTimeWsBytes);
  return time_vectors_unchecked(w_time_in, w_time_out, w_ref_in, w_ref_out, sigma, sigma_next,
                                mode_is_image, n_modes, vec, (char*)workspace, stream);
}

size_t flux3_stack_workspace_size(int n_img, int n_cond, int n_txt) {
  const long n = (long)n_img + n_cond + n_txt;
  if (n_img <= 0 || n_cond < 0 || n_txt < 0 || n >= (1L << 30)) return 0;
  return stack_ws_bytes(n_img, n_cond, n_txt);
}

}  // extern "C"

namespace {
// Argument checks shared by flux3_stack_forward and flux3_sample (everything
// but the workspace size).
int check_stack_args(const flux3_model_weights* w, const uint16_t* img, int n_img,
                     const uint16_t* cond, int n_cond, const uint16_t* txt, int n_txt,
                     const float* table, const float* v, const void* workspace) {
  REQUIRE(w != nullptr, FLUX3_EINVAL, "weights are null");
  REQUIRE(n_img > 0 && n_cond >= 0 && n_txt >= 0, FLUX3_EINVAL, "n_img=%d n_cond=%d n_txt=%d",
          n_img, n_cond, n_txt);
  REQUIRE_PTR(img);
  REQUIRE(n_cond == 0 || (cond != nullptr && aligned16(cond)), FLUX3_EINVAL, "cond null or misaligned");
  REQUIRE(n_txt == 0 || (txt != nullptr && aligned16(txt)), FLUX3_EINVAL, "txt null or misaligned");
  REQUIRE_PTR(table);
  REQUIRE_PTR(v);
  REQUIRE(w->n_early >= 0 && w->n_single >= 0, FLUX3_EINVAL, "block counts");
  REQUIRE_PTR(w->emb_in_image);
  REQUIRE(n_cond == 0 || (w->emb_in_image_cond && aligned16(w->emb_in_image_cond)), FLUX3_EINVAL,
          "emb_in_image_cond missing");
  REQUIRE(n_txt == 0 || (w->txt_in && aligned16(w->txt_in)), FLUX3_EINVAL, "txt_in missing");
  REQUIRE_PTR(w->time_in_w1);
  REQUIRE_PTR(w->time_in_w2);
  REQUIRE((w->ref_time_in_w1 == nullptr) == (w->ref_time_in_w2 == nullptr), FLUX3_EINVAL,
          "ref_time_in weights: give both or neither");
  REQUIRE_PTR(w->final_ada);
  REQUIRE_PTR(w->final_linear);
  REQUIRE(workspace != nullptr && aligned16(workspace), FLUX3_EWORKSPACE, "workspace missing");
  const int all_counts[3] = {n_img, n_cond, n_txt};
  for (int m = 0; m < 3; ++m) {
    if (all_counts[m] == 0) continue;
    REQUIRE(w->early_mod[m] && aligned16(w->early_mod[m]), FLUX3_EINVAL, "early_mod[%d] missing", m);
    REQUIRE(w->single_mod[m] && aligned16(w->single_mod[m]), FLUX3_EINVAL, "single_mod[%d] missing", m);
    REQUIRE(w->n_early == 0 || w->early[m] != nullptr, FLUX3_EINVAL, "early[%d] missing", m);
    for (int b = 0; b < w->n_early; ++b) {
      int rc = check_block_weights(&w->early[m][b]);
      if (rc) return rc;
    }
  }
  REQUIRE(w->n_single == 0 || w->single != nullptr, FLUX3_EINVAL, "single blocks missing");
  for (int b = 0; b < w->n_single; ++b) {
    int rc = check_block_weights(&w->single[b]);
    if (rc) return rc;
  }
  return FLUX3_OK;
}

// The modulation vectors of one stack pass: per present mode i (in token
// order) early and single (shift, scale, gate) at mod_early / mod_single +
// i * 9216, and the final layer's (shift, scale) at mod_final.
struct CondSlot {
  float* vec;  // [n_modes][3072]
  float* mod_early;
  float* mod_single;
  float* mod_final;
};

// Present modes in token order (image, image_cond, text) and their rows.
int present_modes(int n_img, int n_cond, int n_txt, int* modes, int* counts) {
  const int all_counts[3] = {n_img, n_cond, n_txt};
  int n = 0;
  for (int m = 0; m < 3; ++m)
    if (all_counts[m] > 0) {
      modes[n] = m;
      if (counts) counts[n] = all_counts[m];
      ++n;
    }
  return n;
}

// GEMV items y_i (+)= W_i f(x_i), launched in batches of kMaxSeg (items of
// one batch must not depend on each other).
struct GemvItems {
  GemvBatch b{};
  int n = 0;
  int rows, K;
  bool silu, acc;
  hipStream_t st;
  GemvItems(int rows_, int K_, bool silu_, bool acc_, hipStream_t st_)
      : rows(rows_), K(K_), silu(silu_), acc(acc_), st(st_) {}
  void add(const bf16* w, const float* x, float* y) {
    b.w[n] = w;
    b.x[n] = x;
    b.y[n] = y;
    if (++n == kMaxSeg) flush();
  }
  void flush() {
    if (n > 0) launch_gemv(b, n, rows, K, silu, acc, st);
    n = 0;
  }
};

// Conditioning of sampling steps k0 .. k0 + nk - 1 (nk <= kCondChunk) into
// slots[0 .. nk): the same GEMVs as a stack pass makes for each step (each
// row's sum in the same order, so the same bits), batched over the steps so
// that a launch reads each weight for several steps at once.  The time
// embeddings of sigma_k0 .. sigma_{k0+nk} and of 0 go to emb.
constexpr int kCondChunk = 8;
size_t cond_slot_bytes() {
  return align256(3 * kHidden * 4) + 2 * align256(3 * 3 * kHidden * 4) + align256(2 * kHidden * 4);
}
size_t cond_chunk_bytes() {
  return kCondChunk * cond_slot_bytes() + align256((kCondChunk + 2) * 256 * 4) +
         align256((size_t)kCondChunk * 3 * kHidden * 4) + align256((size_t)kCondChunk * kHidden * 4);
}
int precompute_cond(const flux3_model_weights* w, const int* modes, int n_modes, const float* sigmas, int k0,
                    int nk, char* buf, CondSlot* slots, hipStream_t st) {
  for (int j = 0; j < nk; ++j) {
    char* p = buf + j * cond_slot_bytes();
    slots[j].vec = (float*)p;
    p += align256(3 * kHidden * 4);
    slots[j].mod_early = (float*)p;
    p += align256(3 * 3 * kHidden * 4);
    slots[j].mod_single = (float*)p;
    p += align256(3 * 3 * kHidden * 4);
    slots[j].mod_final = (float*)p;
  }
  char* p = buf + kCondChunk * cond_slot_bytes();
  float* emb = (float*)p;  // [nk + 2][256]: emb(sigma_{k0+j}), j <= nk, then emb(0)
  p += align256((kCondChunk + 2) * 256 * 4);
  float* hid = (float*)p;  // [nk][n_modes][3072]
  p += align256((size_t)kCondChunk * 3 * kHidden * 4);
  float* rh = (float*)p;   // [nk][3072]
  for (int j0 = 0; j0 < nk + 2; j0 += 4) {  // four embeddings per launch
    Timesteps ts{};
    const int nt = std::min(4, nk + 2 - j0);
    for (int t = 0; t < nt; ++t) ts.t[t] = j0 + t <= nk ? sigmas[k0 + j0 + t] : 0.f;
    launch_timestep_embedding(ts, nt, emb + (size_t)j0 * 256, st);
  }
  const float* emb0 = emb + (size_t)(nk + 1) * 256;
  // time_in: vec[j][m] = W2 silu(W1 emb(t)), t = sigma_{k0+j} for the image mode, else 0
  GemvItems l1(kHidden, 256, false, false, st);
  for (int j = 0; j < nk; ++j)
    for (int i = 0; i < n_modes; ++i)
      l1.add(B(w->time_in_w1), modes[i] == 0 ? emb + (size_t)j * 256 : emb0,
             hid + ((size_t)j * 3 + i) * kHidden);
  l1.flush();
  GemvItems l2(kHidden, kHidden, true, false, st);
  for (int j = 0; j < nk; ++j)
    for (int i = 0; i < n_modes; ++i)
      l2.add(B(w->time_in_w2), hid + ((size_t)j * 3 + i) * kHidden, slots[j].vec + (size_t)i * kHidden);
  l2.flush();
  if (w->ref_time_in_w1 && w->ref_time_in_w2) {
    // + ref_time_in(emb(sigma_{k0+j+1})) on every mode
    GemvItems r1(kHidden, 256, false, false, st);
    for (int j = 0; j < nk; ++j) r1.add(B(w->ref_time_in_w1), emb + (size_t)(j + 1) * 256, rh + (size_t)j * kHidden);
    r1.flush();
    GemvItems r2(kHidden, kHidden, true, true, st);
    for (int j = 0; j < nk; ++j)
      for (int i = 0; i < n_modes; ++i)
        r2.add(B(w->ref_time_in_w2), rh + (size_t)j * kHidden, slots[j].vec + (size_t)i * kHidden);
    r2.flush();
  }
  // modulations: early and single per mode, final adaLN on the image vector;
  // weight by weight, so that a launch's items share one weight
  GemvItems mods(3 * kHidden, kHidden, true, false, st);
  for (int i = 0; i < n_modes; ++i)
    for (int single = 0; single < 2; ++single)
      for (int j = 0; j < nk; ++j)
        mods.add(B(single ? w->single_mod[modes[i]] : w->early_mod[modes[i]]),
                 slots[j].vec + (size_t)i * kHidden,
                 (single ? slots[j].mod_single : slots[j].mod_early) + (size_t)i * 3 * kHidden);
  mods.flush();
  GemvItems fin(2 * kHidden, kHidden, true, false, st);
  for (int j = 0; j < nk; ++j) fin.add(B(w->final_ada), slots[j].vec, slots[j].mod_final);
  fin.flush();
  return check_launch("sample conditioning");
}

// One pass of the transformer on checked arguments; workspace = StackWs.
// pre: this step's conditioning, already computed (precompute_cond), or null.
int stack_forward_unchecked(const flux3_model_weights* w, const uint16_t* img, int n_img,
                            const uint16_t* cond, int n_cond, const uint16_t* txt, int n_txt,
                            const float* table, float sigma, float sigma_next, float* v,
                            void* workspace, hipStream_t stream, const CondSlot* pre = nullptr) {
  const int n_total = n_img + n_cond + n_txt;
  // Streams present, in token order.
  int modes[3], counts[3], n_modes = 0;
  const int all_counts[3] = {n_img, n_cond, n_txt};
  for (int m = 0; m < 3; ++m)
    if (all_counts[m] > 0) {
      modes[n_modes] = m;
      counts[n_modes] = all_counts[m];
      ++n_modes;
    }

  StackWs s = carve_stack_ws(workspace, n_total);
  const BlockWs bws = carve_block_ws(s.block_ws, n_total);

  // a13 / conditioning: per-mode vectors, then the 2 x n_modes modulations and
  // the final adaLN (SiLU then Linear), unless the caller computed them.
  int rc = FLUX3_OK;
  if (pre != nullptr) {
    s.vec = pre->vec;
    s.mod_early = pre->mod_early;
    s.mod_single = pre->mod_single;
    s.mod_final = pre->mod_final;
  } else {
  int is_image[3];
  for (int i = 0; i < n_modes; ++i) is_image[i] = modes[i] == 0;
  rc = time_vectors_unchecked(w->time_in_w1, w->time_in_w2, w->ref_time_in_w1,
                              w->ref_time_in_w2, sigma, sigma_next, is_image, n_modes, s.vec,
                              s.time_ws, stream);
  if (rc) return rc;
  GemvBatch mb{};
  for (int i = 0; i < n_modes; ++i) {
    mb.w[i] = B(w->early_mod[modes[i]]);
    mb.x[i] = s.vec + (size_t)i * kHidden;
    mb.y[i] = s.mod_early + (size_t)i * 3 * kHidden;
    mb.w[n_modes + i] = B(w->single_mod[modes[i]]);
    mb.x[n_modes + i] = s.vec + (size_t)i * kHidden;
    mb.y[n_modes + i] = s.mod_single + (size_t)i * 3 * kHidden;
  }
  launch_gemv(mb, 2 * n_modes, 3 * kHidden, kHidden, true, false, stream);
  GemvBatch fb{};
  fb.w[0] = B(w->final_ada);
  fb.x[0] = s.vec;  // the image mode is always first
  fb.y[0] = s.mod_final;
  launch_gemv(fb, 1, 2 * kHidden, kHidden, true, false, stream);
  }

  // a9: embeddings into the residual stream.
  const uint16_t* inputs[3] = {img, cond, txt};
  const uint16_t* emb_w[3] = {w->emb_in_image, w->emb_in_image_cond, w->txt_in};
  const int in_dim[3] = {128, 128, 20480};
  int row0[3];
  {
    int r = 0;
    for (int i = 0; i < n_modes; ++i) {
      row0[i] = r;
      r += counts[i];
    }
  }
  for (int i = 0; i < n_modes; ++i) {
    const int m = modes[i];
    GemmArgs g{};
    g.A = B(inputs[m]);
    g.lda = in_dim[m];
    g.B = B(emb_w[m]);
    g.ldb = in_dim[m];
    g.M = counts[i];
    g.N = kHidden;
    g.K = in_dim[m];
    g.epi = GemmEpi::kStoreF32;
    g.C = s.x + (size_t)row0[i] * kHidden;
    g.ldc = kHidden;
    g.split_ws = bws.qkv;  // free until the first block
    g.split_ws_bytes = bws.qkv_bytes;
    launch_gemm(g, stream);
  }

  // a10: stage 1, each stream on its own rows with its own blocks; the
  // streams after the image one on the side stream when there is one.
  SideStream* side = n_modes > 1 ? side_fork(stream) : nullptr;
  const BlockWs sws = side ? carve_block_ws(s.side_ws, side_rows(n_cond, n_txt)) : bws;
  for (int i = 0; i < n_modes; ++i) {
    const int m = modes[i];
    const bool beside = side != nullptr && i > 0;
    SegTable seg{};
    seg.off[0] = 0;
    seg.off[1] = counts[i];
    seg.n = 1;
    bool ln = false;  // a3 of the next block already in the workspace
    for (int b = 0; b < w->n_early; ++b)
      ln = block_forward_unchecked(s.x + (size_t)row0[i] * kHidden, counts[i], seg,
                                   s.mod_early + (size_t)i * 3 * kHidden, &w->early[m][b],
                                   table + (size_t)row0[i] * 128, beside ? sws : bws,
                                   beside ? side->s : stream, nullptr, ln, b + 1 < w->n_early);
  }
  if (side != nullptr) {
    rc = side_join(side, stream);
    if (rc) return rc;
  }

  // a11: stage 2, all tokens, per-row modulation by stream.
  SegTable seg{};
  for (int i = 0; i < n_modes; ++i) seg.off[i] = row0[i];
  seg.off[n_modes] = n_total;
  seg.n = n_modes;
  bool ln = false;
  for (int b = 0; b < w->n_single; ++b)
    ln = block_forward_unchecked(s.x, n_total, seg, s.mod_single, &w->single[b], table, bws, stream, nullptr,
                                 ln, b + 1 < w->n_single);

  // a12: final layer on the image rows.
  SegTable one{};
  one.off[1] = n_img;
  one.n = 1;
  launch_ln_modulate(s.x, kHidden, bws.xm, kHidden, n_img, one, s.mod_final, 2 * kHidden, stream);
  GemmArgs f{};
  f.A = bws.xm;
  f.lda = kHidden;
  f.B = B(w->final_linear);
  f.ldb = kHidden;
  f.M = n_img;
  f.N = 128;
  f.K = kHidden;
  f.epi = GemmEpi::kStoreF32;
  f.C = v;
  f.ldc = 128;
  launch_gemm(f, stream);
  return check_launch("stack_forward");
}

// flux3_sample's workspace: the stack's, then v [n_img][128] fp32 and the
// bf16 copy of x [n_img][128] the embedding reads.
size_t sample_ws_bytes(int n_img, int n_cond, int n_txt) {
  return stack_ws_bytes(n_img, n_cond, n_txt) + align256((size_t)n_img * 128 * 4) +
         align256((size_t)n_img * 128 * 2) + cond_chunk_bytes();
}
}  // namespace

extern "C" {

int flux3_stack_forward(const flux3_model_weights* w, const uint16_t* img, int n_img,
                        const uint16_t* cond, int n_cond, const uint16_t* txt, int n_txt,
                        const float* table, float sigma, float sigma_next, float* v,
                        void* workspace, size_t ws_bytes, hipStream_t stream) {
  int rc = check_stack_args(w, img, n_img, cond, n_cond, txt, n_txt, table, v, workspace);
  if (rc) return rc;
  REQUIRE(ws_bytes >= stack_ws_bytes(n_img, n_cond, n_txt), FLUX3_EWORKSPACE,
          "workspace %zu < %zu bytes", ws_bytes, stack_ws_bytes(n_img, n_cond, n_txt));
  return stack_forward_unchecked(w, img, n_img, cond, n_cond, txt, n_txt, table, sigma,
                                 sigma_next, v, workspace, stream);
}

size_t flux3_sample_workspace_size(int n_img, int n_cond, int n_txt) {
  const long n = (long)n_img + n_cond + n_txt;
  if (n_img <= 0 || n_cond < 0 || n_txt < 0 || n >= (1L << 30)) return 0;
  return sample_ws_bytes(n_img, n_cond, n_txt);
}

int flux3_sample(const flux3_model_weights* w, float* x, int n_img, const uint16_t* cond,
                 int n_cond, const uint16_t* txt, int n_txt, const float* table,
                 const float* sigmas, int steps, void* workspace, size_t ws_bytes,
                 hipStream_t stream) {
  REQUIRE(steps >= 0, FLUX3_EINVAL, "steps=%d", steps);
  REQUIRE(steps == 0 || sigmas != nullptr, FLUX3_EINVAL, "sigmas is null");
  for (int k = 0; k <= steps && steps > 0; ++k)
    REQUIRE(std::isfinite(sigmas[k]), FLUX3_EINVAL, "sigmas[%d] is not finite", k);
  REQUIRE_PTR(x);
  // x doubles as the velocity pointer for the shared checks (only non-null
  // and alignment are checked there).
  int rc = check_stack_args(w, (const uint16_t*)x, n_img, cond, n_cond, txt, n_txt, table, x,
                            workspace);
  if (rc) return rc;
  REQUIRE(ws_bytes >= sample_ws_bytes(n_img, n_cond, n_txt), FLUX3_EWORKSPACE,
          "workspace %zu < %zu bytes", ws_bytes, sample_ws_bytes(n_img, n_cond, n_txt));
  if (steps == 0) return FLUX3_OK;
  char* p = (char*)workspace + stack_ws_bytes(n_img, n_cond, n_txt);
  float* v = (float*)p;
  bf16* xb = (bf16*)(p + align256((size_t)n_img * 128 * 4));
  const int n_lat = n_img * 128;
  char* cond_buf = (char*)xb + align256((size_t)n_img * 128 * 2);
  launch_euler(x, xb, nullptr, n_lat, 0.f, stream);  // xb = bf16(x)
  // The conditioning depends on the step's sigmas only: computed for up to
  // kCondChunk steps at a time, each weight read once per launch for them.
  int modes[3];
  const int n_modes = present_modes(n_img, n_cond, n_txt, modes, nullptr);
  CondSlot slots[kCondChunk];
  for (int k0 = 0; k0 < steps; k0 += kCondChunk) {
    const int nk = std::min(kCondChunk, steps - k0);
    rc = precompute_cond(w, modes, n_modes, sigmas, k0, nk, cond_buf, slots, stream);
    if (rc) return rc;
    for (int j = 0; j < nk; ++j) {
      const int k = k0 + j;
      rc = stack_forward_unchecked(w, (const uint16_t*)xb, n_img, cond, n_cond, txt, n_txt, table,
                                   sigmas[k], sigmas[k + 1], v, workspace, stream, &slots[j]);
      if (rc) return rc;
      launch_euler(x, k + 1 < steps ? xb : nullptr, v, n_lat, sigmas[k + 1] - sigmas[k], stream);
    }
  }
  return check_launch("sample");
}

int flux3_euler_step(float* x, uint16_t* x_bf16, const float* v, int n, float sigma,
                     float sigma_next, hipStream_t stream) {
  REQUIRE(n >= 0, FLUX3_EINVAL, "n=%d", n);
  if (n == 0) return FLUX3_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(v);
  REQUIRE(x_bf16 == nullptr || aligned16(x_bf16), FLUX3_EINVAL, "x_bf16 misaligned");
  launch_euler(x, B(x_bf16), v, n, sigma_next - sigma, stream);
  return check_launch("euler_step");
}

int flux3_sigmas(int steps, double alpha, float* out) {
  REQUIRE(steps >= 1 && out != nullptr && alpha > 0, FLUX3_EINVAL, "steps=%d alpha=%g", steps, alpha);
  for (int k = 0; k <= steps; ++k) {
    const double t = 1.0 - (double)k / steps;
    out[k] = (float)(alpha * t / (1.0 + (alpha - 1.0) * t));
  }
  return FLUX3_OK;
}

int flux3_timer_start(unsigned kinds, int capacity) {
  REQUIRE(kinds != 0 && kinds < (1u << 5), FLUX3_EINVAL, "kinds=0x%x", kinds);
  REQUIRE(capacity >= 1 && capacity <= (1 << 20), FLUX3_EINVAL, "capacity=%d", capacity);
  std::lock_guard<std::mutex> lock(g_timer.mu);
  REQUIRE(g_timer.ev == nullptr, FLUX3_EINVAL, "the launch timer is already armed");
  hipEvent_t* ev = new (std::nothrow) hipEvent_t[2 * (size_t)capacity]();
  int* kind = new (std::nothrow) int[capacity];
  int* rows = new (std::nothrow) int[capacity];
  int made = 0;
  hipError_t e = hipSuccess;
  if (ev != nullptr && kind != nullptr && rows != nullptr)
    for (; made < 2 * capacity; ++made)
      if ((e = hipEventCreate(&ev[made])) != hipSuccess) break;
  if (ev == nullptr || kind == nullptr || rows == nullptr || made < 2 * capacity) {
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    delete[] ev;
    delete[] kind;
    delete[] rows;
    return fail(FLUX3_EHIP, "timer events: %s", e != hipSuccess ? hipGetErrorString(e) : "out of host memory");
  }
  g_timer.ev = ev;
  g_timer.kind = kind;
  g_timer.rows = rows;
  g_timer.capacity = capacity;
  g_timer.count = 0;
  g_timer.kinds.store(kinds, std::memory_order_release);
  return FLUX3_OK;
}

int flux3_timer_stop(float* ms, int* kind, int* rows, int capacity, int* count) {
  REQUIRE(capacity >= 0, FLUX3_EINVAL, "capacity=%d", capacity);
  std::lock_guard<std::mutex> lock(g_timer.mu);
  REQUIRE(g_timer.ev != nullptr, FLUX3_EINVAL, "the launch timer is not armed");
  g_timer.kinds.store(0, std::memory_order_release);
  const int n = g_timer.count;
  hipError_t err = hipSuccess;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[2 * i + 1]);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]);
    if (e != hipSuccess && err == hipSuccess) err = e;
    if (i < capacity) {
      if (ms) ms[i] = t;
      if (kind) kind[i] = g_timer.kind[i];
      if (rows) rows[i] = g_timer.rows[i];
    }
  }
  for (int i = 0; i < 2 * g_timer.capacity; ++i) (void)hipEventDestroy(g_timer.ev[i]);
  delete[] g_timer.ev;
  delete[] g_timer.kind;
  delete[] g_timer.rows;
  g_timer.ev = nullptr;
  g_timer.kind = g_timer.rows = nullptr;
  g_timer.capacity = g_timer.count = 0;
  if (count) *count = std::min(n, capacity);
  REQUIRE(err == hipSuccess, FLUX3_EHIP, "timer events: %s", hipGetErrorString(err));
  return FLUX3_OK;
}

}  // extern "C"

// ---- base checkpoint: the guided two-sample pack ---------------------------------
//
// Both samples of the pack [empty prompt, prompt] share the image latents and
// references, so their image and image_cond streams are identical through
// stage 1 (those streams attend only to themselves and carry the same
// modulation): they run once.  Rows of the packed residual stream:
//   sample 0: image | image_cond | text 0,   sample 1: text 1 | image | image_cond
// so each sample is one contiguous row range (its attention group in stage 2)
// and the two text streams are adjacent (one stage-1 call, two groups).

namespace {

struct CfgRows {
  int n_img, n_cond, n_t0, n_t1;
  int txt0() const { return n_img + n_cond; }
  int n0() const { return n_img + n_cond + n_t0; }
  int img1() const { return n0() + n_t1; }
  int n() const { return img1() + n_img + n_cond; }
};

struct CfgWs {
  float* x;          // [n][3072]
  float* vec;        // [3][3072]
  float* mod_early;  // [3][9216]
  float* mod_seg;    // [5][9216] stage-2 modulation per packed segment
  float* mod_final;  // [6144]
  char* time_ws;
  float* v_pair;     // [2][n_img][128]
  void* block_ws;
  void* side_ws;     // block workspace of the stage-1 side stream
};

size_t cfg_ws_bytes(const CfgRows& r) {
  return align256((size_t)r.n() * kHidden * 4) + align256(3 * kHidden * 4) +
         align256(3 * 3 * kHidden * 4) + align256(5 * 3 * kHidden * 4) + align256(2 * kHidden * 4) +
         align256(kTimeWsBytes) + align256((size_t)2 * r.n_img * 128 * 4) + block_ws_bytes(r.n()) +
         (side_rows(r.n_cond, r.n_t0 + r.n_t1) > 0 ? block_ws_bytes(side_rows(r.n_cond, r.n_t0 + r.n_t1))
                                                    : 0);
}

CfgWs carve_cfg_ws(void* ws, const CfgRows& r) {
  char* p = (char*)ws;
  CfgWs s;
  s.x = (float*)p;
  p += align256((size_t)r.n() * kHidden * 4);
  s.vec = (float*)p;
  p += align256(3 * kHidden * 4);
  s.mod_early = (float*)p;
  p += align256(3 * 3 * kHidden * 4);
  s.mod_seg = (float*)p;
  p += align256(5 * 3 * kHidden * 4);
  s.mod_final = (float*)p;
  p += align256(2 * kHidden * 4);
  s.time_ws = p;
  p += align256(kTimeWsBytes);
  s.v_pair = (float*)p;
  p += align256((size_t)2 * r.n_img * 128 * 4);
  s.block_ws = p;
  s.side_ws = p + block_ws_bytes(r.n());
  return s;
}

int check_cfg_args(const flux3_model_weights* w, const uint16_t* img, const CfgRows& r,
                   const uint16_t* cond, const uint16_t* txt0, const uint16_t* txt1,
                   const float* table, const float* v, const void* ws) {
  REQUIRE(r.n_t0 >= 0 && r.n_t1 >= 0, FLUX3_EINVAL, "n_txt0=%d n_txt1=%d", r.n_t0, r.n_t1);
  REQUIRE(r.n_t0 == 0 || (txt0 != nullptr && aligned16(txt0)), FLUX3_EINVAL, "txt0 null or misaligned");
  REQUIRE(r.n_t1 == 0 || (txt1 != nullptr && aligned16(txt1)), FLUX3_EINVAL, "txt1 null or misaligned");
  REQUIRE((long)r.n_img * 2 + (long)r.n_cond * 2 + r.n_t0 + r.n_t1 < (1L << 30), FLUX3_EINVAL,
          "too many tokens");
  // the shared checks see one text stream of n_t0 + n_t1 rows
  return check_stack_args(w, img, r.n_img, cond, r.n_cond, r.n_t0 ? txt0 : txt1, r.n_t0 + r.n_t1,
                          table, v, ws);
}

// One guided velocity evaluation on checked arguments.
int stack_cfg_unchecked(const flux3_model_weights* w, const uint16_t* img, const uint16_t* cond,
                        const uint16_t* txt0, const uint16_t* txt1, const CfgRows& r,
                        const float* table, float sigma, float sigma_next, float guidance, float* v,
                        void* workspace, hipStream_t stream) {
  const int n = r.n();
  const CfgWs s = carve_cfg_ws(workspace, r);
  const BlockWs bws = carve_block_ws(s.block_ws, n);

  // Modes present (image, image_cond, txt) and their conditioning.
  int modes[3], n_modes = 0;
  modes[n_modes++] = 0;
  if (r.n_cond > 0) modes[n_modes++] = 1;
  if (r.n_t0 + r.n_t1 > 0) modes[n_modes++] = 2;
  int is_image[3];
  for (int i = 0; i < n_modes; ++i) is_image[i] = modes[i] == 0;
  int rc = time_vectors_unchecked(w->time_in_w1, w->time_in_w2, w->ref_time_in_w1,
                                  w->ref_time_in_w2, sigma, sigma_next, is_image, n_modes, s.vec,
                                  s.time_ws, stream);
  if (rc) return rc;
  // Early modulation per mode; single modulation per mode straight into the
  // first n_modes packed segments (sample 0 holds every mode, in mode order).
  GemvBatch mb{};
  for (int i = 0; i < n_modes; ++i) {
    mb.w[i] = B(w->early_mod[modes[i]]);
    mb.x[i] = s.vec + (size_t)i * kHidden;
    mb.y[i] = s.mod_early + (size_t)i * 3 * kHidden;
    mb.w[n_modes + i] = B(w->single_mod[modes[i]]);
    mb.x[n_modes + i] = s.vec + (size_t)i * kHidden;
    mb.y[n_modes + i] = s.mod_seg + (size_t)i * 3 * kHidden;
  }
  launch_gemv(mb, 2 * n_modes, 3 * kHidden, kHidden, true, false, stream);
  GemvBatch fb{};
  fb.w[0] = B(w->final_ada);
  fb.x[0] = s.vec;
  fb.y[0] = s.mod_final;
  launch_gemv(fb, 1, 2 * kHidden, kHidden, true, false, stream);

  // Stage-2 segments in row order; sample 1's image (and image_cond)
  // segments reuse the modulation of the same modes.
  SegTable seg2{};
  int ns = 0;
  seg2.off[ns++] = 0;
  if (r.n_cond > 0) seg2.off[ns++] = r.n_img;
  if (r.n_t0 + r.n_t1 > 0) seg2.off[ns++] = r.txt0();
  const int img_seg1 = ns;
  seg2.off[ns++] = r.img1();
  if (r.n_cond > 0) seg2.off[ns++] = r.img1() + r.n_img;
  seg2.off[ns] = n;
  seg2.n = ns;
  const size_t mod_bytes = 3 * kHidden * sizeof(float);
  for (int i = 0; img_seg1 + i < ns; ++i) {
    const hipError_t e = hipMemcpyAsync(s.mod_seg + (size_t)(img_seg1 + i) * 3 * kHidden,
                                        s.mod_seg + (size_t)i * 3 * kHidden, mod_bytes,
                                        hipMemcpyDeviceToDevice, stream);
    REQUIRE(e == hipSuccess, FLUX3_EHIP, "modulation copy: %s", hipGetErrorString(e));
  }

  // a9: embeddings (image and references once, both texts).
  struct Emb { const uint16_t* in; const uint16_t* w; int rows, k, row0; };
  const Emb embs[4] = {{img, w->emb_in_image, r.n_img, 128, 0},
                       {cond, w->emb_in_image_cond, r.n_cond, 128, r.n_img},
                       {txt0, w->txt_in, r.n_t0, 20480, r.txt0()},
                       {txt1, w->txt_in, r.n_t1, 20480, r.n0()}};
  for (const Emb& e : embs) {
    if (e.rows == 0) continue;
    GemmArgs g{};
    g.A = B(e.in);
    g.lda = e.k;
    g.B = B(e.w);
    g.ldb = e.k;
    g.M = e.rows;
    g.N = kHidden;
    g.K = e.k;
    g.epi = GemmEpi::kStoreF32;
    g.C = s.x + (size_t)e.row0 * kHidden;
    g.ldc = kHidden;
    g.split_ws = bws.qkv;  // free until the first block
    g.split_ws_bytes = bws.qkv_bytes;
    launch_gemm(g, stream);
  }

  // a10: stage 1.  Image and references once (sample 0's rows), then both
  // texts in one call with one attention group each; then sample 1 gets a
  // copy of the shared streams.  References and texts run on the side stream
  // when there is one.
  const int nt = r.n_t0 + r.n_t1;
  SideStream* side = (r.n_cond > 0 || nt > 0) ? side_fork(stream) : nullptr;
  const BlockWs sws = side ? carve_block_ws(s.side_ws, side_rows(r.n_cond, nt)) : bws;
  hipStream_t s1 = side ? side->s : stream;
  SegTable one{};
  one.n = 1;
  int mi = 0;
  {
    one.off[1] = r.n_img;
    bool ln = false;
    for (int b = 0; b < w->n_early; ++b)
      ln = block_forward_unchecked(s.x, r.n_img, one, s.mod_early, &w->early[0][b], table, bws, stream, nullptr,
                                   ln, b + 1 < w->n_early);
    ++mi;
  }
  if (r.n_cond > 0) {
    one.off[1] = r.n_cond;
    bool ln = false;
    for (int b = 0; b < w->n_early; ++b)
      ln = block_forward_unchecked(s.x + (size_t)r.n_img * kHidden, r.n_cond, one,
                                   s.mod_early + (size_t)mi * 3 * kHidden, &w->early[1][b],
                                   table + (size_t)r.n_img * 128, sws, s1, nullptr, ln, b + 1 < w->n_early);
    ++mi;
  }
  if (nt > 0) {
    one.off[1] = nt;
    SegTable groups{};
    groups.off[0] = 0;
    groups.off[1] = r.n_t0;
    groups.off[2] = nt;
    groups.n = 2;
    bool ln = false;
    for (int b = 0; b < w->n_early; ++b)
      ln = block_forward_unchecked(s.x + (size_t)r.txt0() * kHidden, nt, one,
                                   s.mod_early + (size_t)mi * 3 * kHidden, &w->early[2][b],
                                   table + (size_t)r.txt0() * 128, sws, s1, &groups, ln, b + 1 < w->n_early);
  }
  if (side != nullptr) {
    rc = side_join(side, stream);
    if (rc) return rc;
  }
  {
    const hipError_t e = hipMemcpyAsync(s.x + (size_t)r.img1() * kHidden, s.x,
                                        (size_t)(r.n_img + r.n_cond) * kHidden * sizeof(float),
                                        hipMemcpyDeviceToDevice, stream);
    REQUIRE(e == hipSuccess, FLUX3_EHIP, "stream copy: %s", hipGetErrorString(e));
  }

  // a11: stage 2 on both samples at once; each sample attends within itself.
  SegTable samples{};
  samples.off[0] = 0;
  samples.off[1] = r.n0();
  samples.off[2] = n;
  samples.n = 2;
  bool ln = false;
  for (int b = 0; b < w->n_single; ++b)
    ln = block_forward_unchecked(s.x, n, seg2, s.mod_seg, &w->single[b], table, bws, stream, &samples, ln,
                                 b + 1 < w->n_single);

  // a12: final layer on both samples' image rows, then guidance.
  one.off[1] = r.n_img;
  launch_ln_modulate(s.x, kHidden, bws.xm, kHidden, r.n_img, one, s.mod_final, 2 * kHidden, stream);
  launch_ln_modulate(s.x + (size_t)r.img1() * kHidden, kHidden, bws.xm + (size_t)r.n_img * kHidden,
                     kHidden, r.n_img, one, s.mod_final, 2 * kHidden, stream);
  GemmArgs f{};
  f.A = bws.xm;
  f.lda = kHidden;
  f.B = B(w->final_linear);
  f.ldb = kHidden;
  f.M = 2 * r.n_img;
  f.N = 128;
  f.K = kHidden;
  f.epi = GemmEpi::kStoreF32;
  f.C = s.v_pair;
  f.ldc = 128;
  launch_gemm(f, stream);
  launch_cfg_combine(s.v_pair, s.v_pair + (size_t)r.n_img * 128, v, r.n_img * 128, guidance, stream);
  return check_launch("stack_forward_cfg");
}

size_t sample_cfg_ws_bytes(const CfgRows& r) {
  return cfg_ws_bytes(r) + align256((size_t)r.n_img * 128 * 4) + align256((size_t)r.n_img * 128 * 2);
}

bool cfg_rows_ok(int n_img, int n_cond, int n_t0, int n_t1) {
  return n_img > 0 && n_cond >= 0 && n_t0 >= 0 && n_t1 >= 0 &&
         (long)n_img * 2 + (long)n_cond * 2 + n_t0 + n_t1 < (1L << 30);
}
}  // namespace

extern "C" {

int flux3_build_ids_cfg(int img_h, int img_w, int n_refs, const int* ref_hw, int n_txt0, int n_txt1,
                        float* ids, int* n_out) {
  REQUIRE(n_txt0 >= 0 && n_txt1 >= 0, FLUX3_EINVAL, "text lengths must be non-negative");
  REQUIRE(n_out != nullptr, FLUX3_EINVAL, "n_out is null");
  int n0 = 0, nshared = 0;
  int rc = flux3_build_ids(img_h, img_w, n_refs, ref_hw, n_txt0, nullptr, &n0);
  if (rc) return rc;
  rc = flux3_build_ids(img_h, img_w, n_refs, ref_hw, 0, nullptr, &nshared);
  if (rc) return rc;
  const long n = (long)n0 + n_txt1 + nshared;
  REQUIRE(n < (1L << 30), FLUX3_EINVAL, "too many tokens");
  *n_out = (int)n;
  if (!ids) return FLUX3_OK;
  // sample 0: image | references | text 0 (text index 0 ..)
  rc = flux3_build_ids(img_h, img_w, n_refs, ref_hw, n_txt0, ids, &n0);
  if (rc) return rc;
  float* p = ids + (size_t)n0 * 4;
  // sample 1: text 1 | image | references
  for (int i = 0; i < n_txt1; ++i) {
    p[0] = 0.f; p[1] = 0.f; p[2] = 0.f; p[3] = (float)i;
    p += 4;
  }
  return flux3_build_ids(img_h, img_w, n_refs, ref_hw, 0, p, &nshared);
}

size_t flux3_stack_cfg_workspace_size(int n_img, int n_cond, int n_txt0, int n_txt1) {
  if (!cfg_rows_ok(n_img, n_cond, n_txt0, n_txt1)) return 0;
  return cfg_ws_bytes(CfgRows{n_img, n_cond, n_txt0, n_txt1});
}

int flux3_stack_forward_cfg(const flux3_model_weights* w, const uint16_t* img, int n_img,
                            const uint16_t* cond, int n_cond, const uint16_t* txt0, int n_txt0,
                            const uint16_t* txt1, int n_txt1, const float* table, float sigma,
                            float sigma_next, float guidance, float* v, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  const CfgRows r{n_img, n_cond, n_txt0, n_txt1};
  REQUIRE(std::isfinite(guidance), FLUX3_EINVAL, "guidance is not finite");
  int rc = check_cfg_args(w, img, r, cond, txt0, txt1, table, v, workspace);
  if (rc) return rc;
  REQUIRE(ws_bytes >= cfg_ws_bytes(r), FLUX3_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
          cfg_ws_bytes(r));
  return stack_cfg_unchecked(w, img, cond, txt0, txt1, r, table, sigma, sigma_next, guidance, v,
                             workspace, stream);
}

size_t flux3_sample_cfg_workspace_size(int n_img, int n_cond, int n_txt0, int n_txt1) {
  if (!cfg_rows_ok(n_img, n_cond, n_txt0, n_txt1)) return 0;
  return sample_cfg_ws_bytes(CfgRows{n_img, n_cond, n_txt0, n_txt1});
}

int flux3_sample_cfg(const flux3_model_weights* w, float* x, int n_img, const uint16_t* cond,
                     int n_cond, const uint16_t* txt0, int n_txt0, const uint16_t* txt1, int n_txt1,
                     const float* table, const float* sigmas, int steps, float guidance,
                     void* workspace, size_t ws_bytes, hipStream_t stream) {
  const CfgRows r{n_img, n_cond, n_txt0, n_txt1};
  REQUIRE(steps >= 0, FLUX3_EINVAL, "steps=%d", steps);
  REQUIRE(steps == 0 || sigmas != nullptr, FLUX3_EINVAL, "sigmas is null");
  for (int k = 0; k <= steps && steps > 0; ++k)
    REQUIRE(std::isfinite(sigmas[k]), FLUX3_EINVAL, "sigmas[%d] is not finite", k);
  REQUIRE(std::isfinite(guidance), FLUX3_EINVAL, "guidance is not finite");
  REQUIRE_PTR(x);
  // x doubles as the latent and velocity pointers for the shared checks.
  int rc = check_cfg_args(w, (const uint16_t*)x, r, cond, txt0, txt1, table, x, workspace);
  if (rc) return rc;
  REQUIRE(ws_bytes >= sample_cfg_ws_bytes(r), FLUX3_EWORKSPACE, "workspace %zu < %zu bytes",
          ws_bytes, sample_cfg_ws_bytes(r));
  if (steps == 0) return FLUX3_OK;
  char* p = (char*)workspace + cfg_ws_bytes(r);
  float* v = (float*)p;
  bf16* xb = (bf16*)(p + align256((size_t)n_img * 128 * 4));
  const int n_lat = n_img * 128;
  launch_euler(x, xb, nullptr, n_lat, 0.f, stream);  // xb = bf16(x)
  for (int k = 0; k < steps; ++k) {
    rc = stack_cfg_unchecked(w, (const uint16_t*)xb, cond, txt0, txt1, r, table, sigmas[k],
                             sigmas[k + 1], guidance, v, workspace, stream);
    if (rc) return rc;
    launch_euler(x, k + 1 < steps ? xb : nullptr, v, n_lat, sigmas[k + 1] - sigmas[k], stream);
  }
  return check_launch("sample_cfg");
}

}  // extern "C"
