"""Plain CPU oracle of the FLUX.3 Image Klein denoiser (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
bench's CPU-baseline leg may import or run this module.  The HIP library never
calls it, and it shares no code with the HIP library.

Everything is NumPy in float64: inputs are the exact bf16 values (upcast), and
no intermediate value is rounded.  The code follows the pages' statement of the
model step by step, with no blocking or fusion beyond row chunking of the
attention score matrix (which does not change any value's definition).

Sources (cited by page title and section):
  [blog]  "Welcome FLUX.3 Image Klein in Diffusers" (Hugging Face blog):
          §From pixels to tokens, §From prompt to tokens, §Two stages,
          §Inside one block, §Every token gets its own timestep,
          §Positions in four dimensions, §The denoising loop.
  [issue] "[Feature] FLUX.3 Image Klein support #2142" (stable-diffusion.cpp
          issue): the part/size table of the description; the follow-up
          comment's subsections "Tensor names (distilled checkpoint)",
          "Structure (from dit.py)" and "Sampling (sampling.py, pipeline.py)".

Readings taken where the pages are silent or disagree (each restated at the
function that uses it):
  R1  token order image, image_cond, text ([issue] Structure); the blog's
      [text | image | reference] order gives the same per-token results,
      because stage 2 has no mask and positions/modulation travel with tokens.
  R2  the reference offset lives on the l axis, t is 0 for every token.
  R3  image_rope_scale multiplies the h and w ids only (id = 0.5*row).
  R4  row/col are 0-based token-grid indices, row-major; text index 0-based.
  R5  RoPE: per axis 16 frequencies theta^(-2j/32); rotated pairs are adjacent
      dims (2j, 2j+1); axis chunks in head-dim order t, h, w, l.
  R7  the RMSNorm scale multiplies (no 1+scale).
  R8  softmax scale 1/sqrt(128).
  R9  SiLU is applied to vec before every modulation `lin` (as the final
      layer's adaLN does).
  R10 chunk orders: (shift, scale, gate); final layer (shift, scale); SwiGLU
      silu(first half) * second half.
  R12 all references of a sample form one image_cond stream in stage 1.
  R14 attn_out is applied to the attention output (a listed tensor), though
      the blog's block sketch folds it away.
  R17 fp8r ("rowwise FP8"): every Linear of the checkpoint is quantized on
      its own, as a per-tensor checkpoint stores it: its weight per output
      row and its input per token, scale = row max / 448, codes rounded to
      OCP E4M3; the dot products are exact and scaled afterwards.  attn_out
      and mlp_out are two Linears with their own weight scales and their own
      input scales (o and swiglu); q_proj, k_proj, v_proj and mlp_in read
      the same input, so they share its codes and scales.

Parity unpinned against the trained checkpoint: R5 (which head dims a RoPE
pair rotates) and R9 (SiLU before `lin`) are readings no page fixes and no
trained weights or reference outputs exist to check them; apply_rope and
modulation are pinned only to the pages' parameters and to invariants.
"""
from __future__ import annotations

import math

import numpy as np

HIDDEN = 3072
HEADS = 24
HEAD_DIM = 128
MLP_HIDDEN = 9216
AXES = (32, 32, 32, 32)      # t, h, w, l   ([issue] description table, RoPE row)
THETA = 10000.0              # ([issue] description table, RoPE row)
IMAGE_ROPE_SCALE = 0.5       # ([issue] Structure; [blog] positions table "row / 2")
EPS = 1e-6                   # LayerNorm and RMSNorm ([issue] Structure)
TIME_DIM = 256               # timestep embedding width ([issue] Structure)
TIME_FACTOR = 1000.0
MAX_PERIOD = 10000.0
SHIFT_ALPHA = 6.93           # ([issue] Sampling; [blog] §The denoising loop)
PATCH_PX = 16                # one token per 16x16 pixels ([blog] §From pixels to tokens)
TEXT_PAD_MULTIPLE = 80       # ([blog] §From prompt to tokens)


# ----------------------------------------------------------------------------
# Tokens and positions
# ----------------------------------------------------------------------------

def token_grid(height_px: int, width_px: int):
    """Token grid of an image: 8x VAE downsampling then 2x2 packing, so one
    token per 16x16 pixels ([blog] §From pixels to tokens)."""
    assert height_px % PATCH_PX == 0 and width_px % PATCH_PX == 0
    return height_px // PATCH_PX, width_px // PATCH_PX


def padded_text_len(n_prompt_tokens: int) -> int:
    """Prompt right-padded to a multiple of 80 tokens; the pads are real
    tokens for the transformer ([blog] §From prompt to tokens; [issue] Text
    encoder, which also caps prompts at 4096 tokens)."""
    assert 0 < n_prompt_tokens <= 4096
    return -(-n_prompt_tokens // TEXT_PAD_MULTIPLE) * TEXT_PAD_MULTIPLE


def build_ids(img_h: int, img_w: int, n_txt: int, refs=()) -> np.ndarray:
    """Position ids (t, h, w, l) per token, in the order image, image_cond,
    text (R1).  [blog] §Positions in four dimensions (the table) and [issue]
    Structure:
      text token i            -> (0, 0, 0, i)
      image token (row, col)  -> (0, row*0.5, col*0.5, 0)
      reference k (row, col)  -> (0, row*0.5, col*0.5, -(k+1))
    Rows/cols are 0-based grid indices, row-major (R4)."""
    rows = []
    for r in range(img_h):
        for c in range(img_w):
            rows.append((0.0, r * IMAGE_ROPE_SCALE, c * IMAGE_ROPE_SCALE, 0.0))
    for k, (rh, rw) in enumerate(refs):
        for r in range(rh):
            for c in range(rw):
                rows.append((0.0, r * IMAGE_ROPE_SCALE, c * IMAGE_ROPE_SCALE, -(k + 1.0)))
    for i in range(n_txt):
        rows.append((0.0, 0.0, 0.0, float(i)))
    return np.array(rows, dtype=np.float64).reshape(-1, 4)


def rope_frequencies() -> np.ndarray:
    """omega[a, j] = theta^(-2j/32) for each axis a and pair j (R5)."""
    out = np.zeros((len(AXES), AXES[0] // 2))
    for a, dim in enumerate(AXES):
        for j in range(dim // 2):
            out[a, j] = THETA ** (-2.0 * j / dim)
    return out


def rope_angles(ids: np.ndarray) -> np.ndarray:
    """Rotation angle per token, axis and pair: ids[n, a] * omega[a, j]."""
    return ids[:, :, None] * rope_frequencies()[None, :, :]


def apply_rope(x: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Rotate x [N, heads, 128] by the 4-axis RoPE.  Axis a owns head dims
    32a .. 32a+31; pair j of axis a is dims (32a+2j, 32a+2j+1), rotated by the
    angle id_a * omega_j (R5).  Same rotation for every head."""
    ang = rope_angles(ids)
    out = x.copy()
    for a, dim in enumerate(AXES):
        for j in range(dim // 2):
            d = a * dim + 2 * j
            c = np.cos(ang[:, a, j])[:, None]
            s = np.sin(ang[:, a, j])[:, None]
            x0 = x[:, :, d]
            x1 = x[:, :, d + 1]
            out[:, :, d] = x0 * c - x1 * s
            out[:, :, d + 1] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------
# Block pieces
# ----------------------------------------------------------------------------

def layer_norm(x: np.ndarray) -> np.ndarray:
    """LayerNorm over the last axis with no learned scale or shift, eps 1e-6
    ([blog] §Inside one block; [issue] Structure).  Biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + EPS)


def modulate(xhat: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """(1 + scale) * xhat + shift ([blog] §Inside one block)."""
    return (1.0 + scale) * xhat + shift


def rms_norm(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Per-head RMSNorm over head_dim 128, eps 1e-6, times the learned scale
    (R7) ([issue] Structure: norm.query_norm.scale / norm.key_norm.scale)."""
    ms = (q * q).mean(axis=-1, keepdims=True)
    return q / np.sqrt(ms + EPS) * scale


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int = 512) -> np.ndarray:
    """Per head: softmax(q k^T / sqrt(128)) v over all keys, no mask
    ([blog] §Two stages: stage 2 has no mask over the joined sequence; the pads
    are attended too, §From prompt to tokens).  q [Nq,H,d], k/v [Nk,H,d].
    Rows are processed in chunks only to bound memory."""
    nq, nh, d = q.shape
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(d)            # R8
    kt = k.transpose(1, 2, 0)             # [H, d, Nk]
    vh = v.transpose(1, 0, 2)             # [H, Nk, d]
    for s in range(0, nq, chunk):
        qh = q[s:s + chunk].transpose(1, 0, 2)          # [H, c, d]
        sc = np.matmul(qh, kt) * scale                  # [H, c, Nk]
        sc -= sc.max(axis=-1, keepdims=True)
        p = np.exp(sc)
        p /= p.sum(axis=-1, keepdims=True)
        out[s:s + chunk] = np.matmul(p, vh).transpose(1, 0, 2)
    return out


def rows_modulation(n: int, segments, mods: np.ndarray):
    """Per-row (shift, scale, gate) [n, 3072] each, from per-segment vectors.
    segments: list of (start, end); mods [n_seg, 3, 3072] = (shift, scale,
    gate) per segment (R10).  Rows outside every segment are an error."""
    shift = np.full((n, HIDDEN), np.nan)
    scale = np.full((n, HIDDEN), np.nan)
    gate = np.full((n, HIDDEN), np.nan)
    for i, (a, b) in enumerate(segments):
        shift[a:b] = mods[i, 0]
        scale[a:b] = mods[i, 1]
        gate[a:b] = mods[i, 2]
    assert not np.isnan(shift).any(), "segments must cover every row"
    return shift, scale, gate


def block_forward(x: np.ndarray, segments, mods: np.ndarray, w: dict, ids: np.ndarray,
                  rows=None) -> np.ndarray:
    """One transformer block ([blog] §Inside one block; [issue] Structure):
        h      = (1 + scale) * LayerNorm(x) + shift
        q,k,v  = h Wq^T, h Wk^T, h Wv^T            (separate projections)
        q, k   = rope(rmsnorm(q)), rope(rmsnorm(k))  per head
        att    = attention(q, k, v) Wo^T            (attn_out, R14)
        a, b   = chunk2(h Win^T)
        mlp    = (silu(a) * b) Wout^T               (SwiGLU, parallel branch)
        return x + gate * (att + mlp)
    shift/scale/gate are taken per row from the row's segment.  All keys are
    attended (a stage-1 call passes one mode's rows only).

    w: float64 arrays under the checkpoint's names (q_proj, k_proj, v_proj,
    attn_out, mlp_in, mlp_out, norm.query_norm.scale, norm.key_norm.scale).
    rows: optional index array; then only those rows of the output are
    computed and returned (keys and values still come from every row)."""
    n = x.shape[0]
    shift, scale, gate = rows_modulation(n, segments, mods)
    h = modulate(layer_norm(x), shift, scale)
    if rows is None:
        rows = np.arange(n)
    hr = h[rows]
    q = (hr @ w["q_proj"].T).reshape(-1, HEADS, HEAD_DIM)
    k = (h @ w["k_proj"].T).reshape(n, HEADS, HEAD_DIM)
    v = (h @ w["v_proj"].T).reshape(n, HEADS, HEAD_DIM)
    q = apply_rope(rms_norm(q, w["norm.query_norm.scale"]), ids[rows])
    k = apply_rope(rms_norm(k, w["norm.key_norm.scale"]), ids)
    att = attention(q, k, v).reshape(-1, HIDDEN) @ w["attn_out"].T
    ab = hr @ w["mlp_in"].T
    a, b = ab[:, :MLP_HIDDEN], ab[:, MLP_HIDDEN:]
    mlp = (silu(a) * b) @ w["mlp_out"].T
    return x[rows] + gate[rows] * (att + mlp)


# ----------------------------------------------------------------------------
# fp8r: rowwise FP8 projections ([blog] §Base model and quantized variants:
# the transformer also ships as "fp8r (rowwise FP8)"), in the OCP E4M3 format
# of CDNA4's FP8 units (R17)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0   # largest finite E4M3 value: 1.75 * 2^8


def e4m3_round(x):
    """Nearest OCP E4M3 value of float32 input: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; normals 2^-6 .. 448, subnormals k * 2^-9; no
    infinities.  Ties go to the even mantissa; magnitudes past 448 saturate.
    Returns (codes uint8, values float64)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))      # a = m 2^ex, m in [0.5, 1)
    e = np.minimum(ex - 1, 8)                        # binade 2^e (subnormals: e = -6)
    q = np.ldexp(1.0, e - 3)                         # value spacing in that binade
    v = np.minimum(np.rint(a / q) * q, E4M3_MAX)     # rint: ties to even
    # encode: normals E = e' + 7, M = v / 2^(e'-3) - 8; subnormals E = 0, M = v / 2^-9
    _, ev = np.frexp(np.where(v > 0, v, 1.0))
    ev = ev - 1
    normal = v >= 2.0 ** -6
    big_e = np.where(normal, ev + 7, 0)
    man = np.where(normal, v / np.ldexp(1.0, ev - 3) - 8, v / 2.0 ** -9)
    codes = (np.signbit(x).astype(np.uint16) << 7) | (big_e.astype(np.uint16) << 3) | man.astype(np.uint16)
    return codes.astype(np.uint8), np.where(np.signbit(x), -v, v)


def e4m3_value(codes):
    """Value of E4M3 codes (inverse of the encoding above; 0x7F/0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    big_e, man = (c >> 3) & 15, c & 7
    mag = np.where(big_e > 0, np.ldexp(1.0 + man / 8.0, big_e - 7), man * 2.0 ** -9)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def quantize_rows_fp8(x):
    """Rowwise FP8 (R17): per row, scale = max|x| / 448 and codes of
    x * (448 / max|x|), the scale, its reciprocal and the product each taken
    in float32 (the precision in which the codes are decided); a row of zeros
    gets scale 1.  Returns (codes uint8, scale float32 per row, dequantized
    float64 = value * scale)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    inv = np.where(nz, np.float32(E4M3_MAX) / safe, np.float32(1)).astype(np.float32)
    scale = np.where(nz, safe / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    codes, vals = e4m3_round((x32 * inv[:, None]).astype(np.float32))
    return codes, scale, vals * scale.astype(np.float64)[:, None]


def fp8r_linear(a: np.ndarray, w: np.ndarray, quant=quantize_rows_fp8) -> np.ndarray:
    """One Linear of the fp8r transformer, a w^T, with its input quantized per
    row (per token) and its weight per output row, the dot products exact and
    scaled afterwards (R17)."""
    return quant(a)[2] @ quant(w)[2].T


def block_forward_fp8r(x: np.ndarray, segments, mods: np.ndarray, w: dict, ids: np.ndarray,
                       rows=None, quant=quantize_rows_fp8) -> np.ndarray:
    """block_forward with each of the block's six Linears (q_proj, k_proj,
    v_proj, mlp_in, attn_out, mlp_out) as a rowwise-FP8 product of its own
    (R17).  Everything else as in block_forward."""
    n = x.shape[0]
    shift, scale, gate = rows_modulation(n, segments, mods)
    h = modulate(layer_norm(x), shift, scale)
    if rows is None:
        rows = np.arange(n)
    hr = h[rows]
    q = fp8r_linear(hr, w["q_proj"], quant).reshape(-1, HEADS, HEAD_DIM)
    k = fp8r_linear(h, w["k_proj"], quant).reshape(n, HEADS, HEAD_DIM)
    v = fp8r_linear(h, w["v_proj"], quant).reshape(n, HEADS, HEAD_DIM)
    q = apply_rope(rms_norm(q, w["norm.query_norm.scale"]), ids[rows])
    k = apply_rope(rms_norm(k, w["norm.key_norm.scale"]), ids)
    o = attention(q, k, v).reshape(-1, HIDDEN)
    att = fp8r_linear(o, w["attn_out"], quant)
    ab = fp8r_linear(hr, w["mlp_in"], quant)
    a, b = ab[:, :MLP_HIDDEN], ab[:, MLP_HIDDEN:]
    mlp = fp8r_linear(silu(a) * b, w["mlp_out"], quant)
    return x[rows] + gate[rows] * (att + mlp)


# ----------------------------------------------------------------------------
# Conditioning: timestep embeddings, per-mode vectors, modulation
# ----------------------------------------------------------------------------

def timestep_embedding(t: float) -> np.ndarray:
    """[cos, sin] of 1000 * t * f_j, f_j = exp(-ln(10000) * j / 128),
    j = 0..127; width 256 ([issue] Structure, "Time")."""
    half = TIME_DIM // 2
    f = np.exp(-math.log(MAX_PERIOD) * np.arange(half, dtype=np.float64) / half)
    arg = TIME_FACTOR * float(t) * f
    return np.concatenate([np.cos(arg), np.sin(arg)])


def mlp_embedder(e: np.ndarray, w_in: np.ndarray, w_out: np.ndarray) -> np.ndarray:
    """Linear, SiLU, Linear, no biases ([issue] Structure; tensor names
    time_in.{in_layer,out_layer})."""
    return w_out @ silu(w_in @ e)


def mode_vectors(W, sigma: float, sigma_next, modes) -> dict:
    """Conditioning vector per mode ([blog] §Every token gets its own
    timestep; [issue] Structure): image tokens carry t = sigma, the other modes
    t = 0.  For the flow-map checkpoint (sigma_next not None) every mode also
    gets ref_time_in(emb(sigma_next)) added.  W: name -> float64 array."""
    out = {}
    for m in modes:
        t = sigma if m == "image" else 0.0
        vec = mlp_embedder(timestep_embedding(t), W("time_in.in_layer.weight"),
                           W("time_in.out_layer.weight"))
        if sigma_next is not None:
            vec = vec + mlp_embedder(timestep_embedding(sigma_next),
                                     W("ref_time_in.in_layer.weight"),
                                     W("ref_time_in.out_layer.weight"))
        out[m] = vec
    return out


def modulation(vec: np.ndarray, lin: np.ndarray) -> np.ndarray:
    """(shift, scale, gate) = chunk3(lin silu(vec)) -> [3, 3072]
    (R9, R10; [issue] Tensor names: lin.weight [9216, 3072] = 3 x 3072)."""
    return (lin @ silu(vec)).reshape(3, HIDDEN)


def final_layer(x_img: np.ndarray, vec_img: np.ndarray, w_ada: np.ndarray,
                w_lin: np.ndarray) -> np.ndarray:
    """Image tokens only: LayerNorm, shift/scale from adaLN_modulation (SiLU
    then Linear to 2 x 3072), then the linear to 128 channels ([issue]
    Structure, "Output"; [blog] §Two stages)."""
    ss = w_ada @ silu(vec_img)
    shift, scale = ss[:HIDDEN], ss[HIDDEN:]
    return modulate(layer_norm(x_img), shift, scale) @ w_lin.T


# ----------------------------------------------------------------------------
# The whole transformer and the sampler
# ----------------------------------------------------------------------------

def _early_prefix(mode: str, i: int) -> str:
    return f"txt_mode_blocks.{i}" if mode == "txt" else f"content_mode_blocks.{mode}.{i}"


def stack_forward(W, B, img: np.ndarray, cond, txt: np.ndarray, img_h: int, img_w: int,
                  refs, sigma: float, sigma_next, n_early: int = 5, n_single: int = 28,
                  block=None) -> np.ndarray:
    """Velocity for the image tokens ([blog] §Two stages, §Every token gets its
    own timestep; [issue] Structure):
      1. embed: img emb_in.image, references emb_in.image_cond, text txt_in;
      2. stage 1: each mode through its own n_early blocks with its
         early_stream_modulations, attending only within the mode (R12);
      3. concatenate in the order image, image_cond, text (R1);
      4. stage 2: n_single shared blocks, each token modulated by its mode's
         single_stream_modulations;
      5. final layer on the image tokens -> v [N_img, 128].
    W(name) -> float64 global tensor; B(prefix) -> dict of one block's float64
    tensors.  cond may be None (no references).  block: the block function
    (block_forward, or block_forward_fp8r for the fp8r transformer)."""
    block = block_forward if block is None else block
    ids = build_ids(img_h, img_w, txt.shape[0], refs)
    modes, streams, vecs = stage1(W, B, img, cond, txt, ids, refs, sigma, sigma_next, n_early, block)

    # stage 2: the streams concatenated, one unmasked attention over all rows
    seg = []
    start = 0
    for xs in streams:
        seg.append((start, start + xs.shape[0]))
        start += xs.shape[0]
    x = np.concatenate(streams, axis=0)
    mods = np.stack([modulation(vecs[m], W(f"single_stream_modulations.{m}.lin.weight"))
                     for m in modes])
    for i in range(n_single):
        x = block(x, seg, mods, B(f"single_blocks.{i}"), ids)

    n_img = img.shape[0]
    return final_layer(x[:n_img], vecs["image"], W("final_layer.image.adaLN_modulation.1.weight"),
                       W("final_layer.image.linear.weight"))


def stage1(W, B, img, cond, txt, ids, refs, sigma, sigma_next, n_early: int = 5, block=None):
    """Embedding and stage 1 ([blog] §Two stages; [issue] Structure): each
    mode is embedded by its own input linear, then runs through its own
    n_early blocks with its early_stream_modulations, attending only to its
    own tokens (one image_cond stream holds every reference, R12).
    Returns (modes, streams, vecs)."""
    embedded = [("image", img @ W("emb_in.image.weight").T)]
    if cond is not None and len(refs) > 0:
        embedded.append(("image_cond", cond @ W("emb_in.image_cond.weight").T))
    embedded.append(("txt", txt @ W("txt_in.weight").T))
    modes = [m for m, _ in embedded]
    vecs = mode_vectors(W, sigma, sigma_next, modes)
    start = 0
    streams = []
    for m, xs in embedded:
        n = xs.shape[0]
        ids_m = ids[start:start + n]
        mod = modulation(vecs[m], W(f"early_stream_modulations.{m}.lin.weight"))[None]
        for i in range(n_early):
            xs = (block or block_forward)(xs, [(0, n)], mod, B(_early_prefix(m, i)), ids_m)
        streams.append(xs)
        start += n
    return modes, streams, vecs


def sigmas(steps: int, alpha: float = SHIFT_ALPHA) -> np.ndarray:
    """t = linspace(1, 0, steps+1); sigma = alpha t / (1 + (alpha - 1) t)
    ([issue] Sampling; shift 6.93 from [blog] §The denoising loop)."""
    t = np.linspace(1.0, 0.0, steps + 1)
    return alpha * t / (1.0 + (alpha - 1.0) * t)


def sample_flow_map(velocity, x: np.ndarray, steps: int = 16) -> np.ndarray:
    """Distilled flow-map sampler ([issue] Sampling): at step k call the model
    with (sigma_k, sigma_{k+1}) and update x += (sigma_{k+1} - sigma_k) v.
    velocity(x, sigma, sigma_next) -> v."""
    s = sigmas(steps)
    for k in range(steps):
        v = velocity(x, s[k], s[k + 1])
        x = x + (s[k + 1] - s[k]) * v
    return x


BASE_STEPS = 50       # base checkpoint ([issue] Sampling)
CFG_GUIDANCE = 3.5    # base checkpoint's guidance scale ([issue] Sampling)


def cfg_velocity(v_uncond: np.ndarray, v_cond: np.ndarray, guidance: float) -> np.ndarray:
    """Classifier-free guidance of the base checkpoint's two-sample pack
    [empty prompt, prompt] ([issue] Sampling, "CFG 3.5"): the unconditional
    velocity moved `guidance` times along the difference to the conditional
    one (R13: the usual guidance formula; the pages give only the scale)."""
    return v_uncond + guidance * (v_cond - v_uncond)


def sample_base_cfg(velocity, x: np.ndarray, steps: int = BASE_STEPS,
                    guidance: float = CFG_GUIDANCE) -> np.ndarray:
    """Base-checkpoint sampler ([issue] Sampling): the same shifted schedule and
    Euler update as the flow map, but each step evaluates the model (timestep
    sigma_k, no ref_time_in) on both samples of the pack and guides.
    velocity(x, sigma, sample) -> v, sample 0 = empty prompt, 1 = prompt."""
    s = sigmas(steps)
    for k in range(steps):
        v = cfg_velocity(velocity(x, s[k], 0), velocity(x, s[k], 1), guidance)
        x = x + (s[k + 1] - s[k]) * v
    return x


def euler_update(x: np.ndarray, v: np.ndarray, sigma: float, sigma_next: float) -> np.ndarray:
    """One sampler update x + (sigma_next - sigma) v ([issue] Sampling)."""
    return x + (sigma_next - sigma) * v


# ----------------------------------------------------------------------------
# Work counts (algorithmic, for rooflines and baselines)
# ----------------------------------------------------------------------------

def block_flops(n: int) -> float:
    """2 N (4 H^2 + 3 H F) for the six projections plus 4 N^2 H for QK^T and
    PV (H = 3072, F = 9216)."""
    return 2.0 * n * (4 * HIDDEN * HIDDEN + 3 * HIDDEN * MLP_HIDDEN) + 4.0 * n * n * HIDDEN
