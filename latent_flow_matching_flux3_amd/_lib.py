"""ctypes binding of libflux3_dit.so.

Argument marshalling only: every function forwards to the C entry point of the
same name (declared in include/flux3_dit.h) with raw device pointers taken
from torch tensors and the current HIP stream.  No arithmetic of the model
happens here.  A missing library is an error; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflux3_dit.so")

HIDDEN = 3072
HEADS = 24
HEAD_DIM = 128
MLP_HIDDEN = 9216
W_IN_ROWS = 27648
W_OUT_COLS = 12288
MAX_SEG = 8

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4


class Flux3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"flux3 error {code}: {msg}")
        self.code = code


_lib = None

P = C.c_void_p
I = C.c_int
F = C.c_float
S = C.c_size_t


class BlockWeightsC(C.Structure):
    _fields_ = [("w_in", P), ("w_out", P), ("q_scale", P), ("k_scale", P),
                ("w_in_fp8", P), ("w_in_scale", P), ("w_out_fp8", P), ("w_out_scale", P)]


class ModelWeightsC(C.Structure):
    _fields_ = [
        ("emb_in_image", P), ("emb_in_image_cond", P), ("txt_in", P),
        ("time_in_w1", P), ("time_in_w2", P), ("ref_time_in_w1", P), ("ref_time_in_w2", P),
        ("early_mod", P * 3), ("single_mod", P * 3),
        ("early", C.POINTER(BlockWeightsC) * 3), ("single", C.POINTER(BlockWeightsC)),
        ("n_early", I), ("n_single", I),
        ("final_ada", P), ("final_linear", P),
    ]


_SIGS = {
    "flux3_last_error": (C.c_char_p, []),
    "flux3_version": (I, []),
    "flux3_build_ids": (I, [I, I, I, P, I, P, C.POINTER(I)]),
    "flux3_rope_table": (I, [P, I, P, P]),
    "flux3_modulate": (I, [P, P, I, P, P]),
    "flux3_ln_modulate": (I, [P, I, P, I, I, P, I, P, I, P]),
    "flux3_qk_norm_rope": (I, [P, I, P, I, I, P, P, P, P]),
    "flux3_attention": (I, [P, I, P, I, P, I, P, I, I, P]),
    "flux3_attention_workspace_size": (S, [I]),
    "flux3_attention_ws": (I, [P, I, P, I, P, I, P, I, I, P, S, P]),
    "flux3_attention_noalloc": (I, [P, I, P, I, P, I, P, I, I, P]),
    "flux3_linear": (I, [P, I, P, I, P, I, P, I, I, I, P]),
    "flux3_pack_block": (I, [P, P, P, P, P, P, P, P, P]),
    "flux3_block_in_proj": (I, [P, I, P, P, P, I, P]),
    "flux3_block_out_proj": (I, [P, I, P, P, P, I, P, P]),
    "flux3_block_workspace_size": (S, [I]),
    "flux3_block_forward": (I, [P, I, P, I, P, C.POINTER(BlockWeightsC), P, P, S, P]),
    "flux3_time_vectors": (I, [P, P, P, P, F, F, P, I, P, P, S, P]),
    "flux3_stack_workspace_size": (S, [I, I, I]),
    "flux3_stack_forward": (I, [C.POINTER(ModelWeightsC), P, I, P, I, P, I, P, F, F, P, P, S, P]),
    "flux3_sample_workspace_size": (S, [I, I, I]),
    "flux3_sample": (I, [C.POINTER(ModelWeightsC), P, I, P, I, P, I, P, P, I, P, S, P]),
    "flux3_build_ids_cfg": (I, [I, I, I, P, I, I, P, C.POINTER(I)]),
    "flux3_stack_cfg_workspace_size": (S, [I, I, I, I]),
    "flux3_stack_forward_cfg": (I, [C.POINTER(ModelWeightsC), P, I, P, I, P, I, P, I, P, F, F, F, P, P, S, P]),
    "flux3_sample_cfg_workspace_size": (S, [I, I, I, I]),
    "flux3_sample_cfg": (I, [C.POINTER(ModelWeightsC), P, I, P, I, P, I, P, I, P, P, I, F, P, S, P]),
    "flux3_quantize_rows_fp8": (I, [P, I, I, I, P, I, P, P]),
    "flux3_pack_block_fp8": (I, [P, P, P, P, P, P, P]),
    "flux3_linear_fp8": (I, [P, I, P, P, I, P, P, P, I, I, I, I, P]),
    "flux3_euler_step": (I, [P, P, P, I, F, F, P]),
    "flux3_sigmas": (I, [I, C.c_double, P]),
    "flux3_timer_start": (I, [C.c_uint, I]),
    "flux3_timer_stop": (I, [P, P, P, I, C.POINTER(I)]),
}

EXPORTS = tuple(_SIGS)


def lib():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m latent_flow_matching_flux3_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise Flux3Error(rc, lib().flux3_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require_dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() >= 2 else t.shape[-1]


def _segs(seg_off):
    arr = (I * len(seg_off))(*[int(s) for s in seg_off])
    return arr, len(seg_off) - 1


# ---- entry points (same names as the C ABI) ------------------------------------

def flux3_version() -> int:
    return lib().flux3_version()


def flux3_build_ids(img_h: int, img_w: int, n_txt: int, refs=()) -> torch.Tensor:
    """Host ids [N, 4] fp32 (token order image, references, text)."""
    refs = list(refs)
    hw = (I * max(1, 2 * len(refs)))(*[int(v) for r in refs for v in r])
    n = I(0)
    _check(lib().flux3_build_ids(img_h, img_w, len(refs), hw, n_txt, None, C.byref(n)))
    out = torch.empty((n.value, 4), dtype=torch.float32)
    _check(lib().flux3_build_ids(img_h, img_w, len(refs), hw, n_txt, out.data_ptr(), C.byref(n)))
    return out


def flux3_rope_table(ids: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _require_dev(ids, torch.float32, "ids")
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, 64, 2), dtype=torch.float32, device=ids.device)
    _check(lib().flux3_rope_table(_ptr(ids.contiguous()), n, _ptr(out), _stream(stream)))
    return out


def flux3_modulate(vec: torch.Tensor, w_lin: list, out: torch.Tensor | None = None, stream=None):
    _require_dev(vec, torch.float32, "vec")
    n_seg = vec.shape[0]
    if out is None:
        out = torch.empty((n_seg, 3, HIDDEN), dtype=torch.float32, device=vec.device)
    ptrs = (P * n_seg)(*[_ptr(w) for w in w_lin])
    _check(lib().flux3_modulate(_ptr(vec), ptrs, n_seg, _ptr(out), _stream(stream)))
    return out


def flux3_ln_modulate(x, out, seg_off, mod, mod_stride=3 * HIDDEN, stream=None):
    arr, n_seg = _segs(seg_off)
    _check(lib().flux3_ln_modulate(_ptr(x), _ld(x), _ptr(out), _ld(out), x.shape[0], arr, n_seg,
                                   _ptr(mod), mod_stride, _stream(stream)))
    return out


def flux3_qk_norm_rope(q, k, q_scale, k_scale, table, stream=None):
    _check(lib().flux3_qk_norm_rope(_ptr(q), _ld(q), _ptr(k), _ld(k), q.shape[0], _ptr(q_scale),
                                    _ptr(k_scale), _ptr(table), _stream(stream)))


def flux3_attention(q, k, v, o, stream=None):
    _check(lib().flux3_attention(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o),
                                 q.shape[0], _stream(stream)))
    return o


def flux3_attention_workspace_size(n: int) -> int:
    return lib().flux3_attention_workspace_size(n)


def flux3_attention_ws(q, k, v, o, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().flux3_attention_ws(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o),
                                    q.shape[0], _ptr(workspace) if workspace is not None else None,
                                    ws_bytes, _stream(stream)))
    return o


def flux3_attention_noalloc(q, k, v, o, stream=None):
    _check(lib().flux3_attention_noalloc(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o),
                                         _ld(o), q.shape[0], _stream(stream)))
    return o


def flux3_linear(x, w, y=None, y_f32=None, stream=None):
    m, k = x.shape
    n = w.shape[0]
    _check(lib().flux3_linear(_ptr(x), _ld(x), _ptr(w), _ld(w), _ptr(y),
                              _ld(y) if y is not None else _ld(y_f32), _ptr(y_f32), m, n, k,
                              _stream(stream)))
    return y if y is not None else y_f32


def flux3_pack_block(w: dict, device=None, stream=None):
    """Pack one block's checkpoint tensors (device bf16, checkpoint names)
    into (w_in, w_out) device tensors."""
    dev = w["q_proj"].device if device is None else device
    w_in = torch.empty((W_IN_ROWS, HIDDEN), dtype=torch.bfloat16, device=dev)
    w_out = torch.empty((HIDDEN, W_OUT_COLS), dtype=torch.bfloat16, device=dev)
    _check(lib().flux3_pack_block(_ptr(w["q_proj"]), _ptr(w["k_proj"]), _ptr(w["v_proj"]),
                                  _ptr(w["attn_out"]), _ptr(w["mlp_in"]), _ptr(w["mlp_out"]),
                                  _ptr(w_in), _ptr(w_out), _stream(stream)))
    return w_in, w_out


def flux3_quantize_rows_fp8(x, q=None, scale=None, stream=None):
    """Rowwise FP8 of a device bf16 [rows, cols] tensor: (codes uint8 [rows, cols], scale fp32 [rows])."""
    _require_dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty(rows, dtype=torch.float32, device=x.device) if scale is None else scale
    _check(lib().flux3_quantize_rows_fp8(_ptr(x), _ld(x), rows, cols, _ptr(q), _ld(q), _ptr(scale),
                                         _stream(stream)))
    return q, scale


def flux3_linear_fp8(a, a_scale, w, w_scale, y=None, y_f32=None, stream=None):
    m, k = a.shape
    n = w.shape[0]
    _check(lib().flux3_linear_fp8(_ptr(a), _ld(a), _ptr(a_scale), _ptr(w), _ld(w), _ptr(w_scale), _ptr(y),
                                  _ptr(y_f32), _ld(y) if y is not None else _ld(y_f32), m, n, k,
                                  _stream(stream)))
    return y if y is not None else y_f32


class PackedBlock:
    """Device tensors of one packed block; keeps them alive for the C struct.
    fp8=True: the projections are quantized per row (fp8r) and the bf16
    packed weights are dropped."""

    def __init__(self, w: dict, stream=None, fp8: bool = False):
        self.w_in, self.w_out = flux3_pack_block(w, stream=stream)
        self.q_scale = w["norm.query_norm.scale"].contiguous()
        self.k_scale = w["norm.key_norm.scale"].contiguous()
        self.fp8 = None
        if fp8:
            dev = self.w_in.device
            w_in8 = torch.empty((W_IN_ROWS, HIDDEN), dtype=torch.uint8, device=dev)
            w_out8 = torch.empty((HIDDEN, W_OUT_COLS), dtype=torch.uint8, device=dev)
            s_in = torch.empty(W_IN_ROWS, dtype=torch.float32, device=dev)
            s_out = torch.empty(3 * HIDDEN, dtype=torch.float32, device=dev)
            _check(lib().flux3_pack_block_fp8(_ptr(self.w_in), _ptr(self.w_out), _ptr(w_in8), _ptr(s_in),
                                              _ptr(w_out8), _ptr(s_out), _stream(stream)))
            self.fp8 = (w_in8, s_in, w_out8, s_out)
            torch.cuda.synchronize()  # the bf16 packed weights are read until here
            self.w_in = self.w_out = None

    def fp8_copy(self, stream=None) -> "PackedBlock":
        """The same block with fp8r projections (new quantized buffers; this
        block's bf16 weights are kept)."""
        b = PackedBlock.__new__(PackedBlock)
        b.q_scale, b.k_scale = self.q_scale, self.k_scale
        dev = self.w_in.device
        w_in8 = torch.empty((W_IN_ROWS, HIDDEN), dtype=torch.uint8, device=dev)
        w_out8 = torch.empty((HIDDEN, W_OUT_COLS), dtype=torch.uint8, device=dev)
        s_in = torch.empty(W_IN_ROWS, dtype=torch.float32, device=dev)
        s_out = torch.empty(3 * HIDDEN, dtype=torch.float32, device=dev)
        _check(lib().flux3_pack_block_fp8(_ptr(self.w_in), _ptr(self.w_out), _ptr(w_in8), _ptr(s_in),
                                          _ptr(w_out8), _ptr(s_out), _stream(stream)))
        b.fp8 = (w_in8, s_in, w_out8, s_out)
        b.w_in = b.w_out = None
        return b

    def c(self) -> BlockWeightsC:
        f = self.fp8 or (None, None, None, None)
        return BlockWeightsC(_ptr(self.w_in), _ptr(self.w_out), _ptr(self.q_scale), _ptr(self.k_scale),
                             _ptr(f[0]), _ptr(f[1]), _ptr(f[2]), _ptr(f[3]))


def flux3_block_in_proj(xm, w_in, qkv, h, stream=None):
    _check(lib().flux3_block_in_proj(_ptr(xm), xm.shape[0], _ptr(w_in), _ptr(qkv), _ptr(h), _ld(h),
                                     _stream(stream)))


def flux3_block_out_proj(cat, w_out, x, seg_off, mod, stream=None):
    arr, n_seg = _segs(seg_off)
    _check(lib().flux3_block_out_proj(_ptr(cat), cat.shape[0], _ptr(w_out), _ptr(x), arr, n_seg,
                                      _ptr(mod), _stream(stream)))


def flux3_block_workspace_size(n: int) -> int:
    return lib().flux3_block_workspace_size(n)


def flux3_block_forward(x, seg_off, mod, block: PackedBlock, table, workspace, stream=None):
    arr, n_seg = _segs(seg_off)
    cw = block.c()
    _check(lib().flux3_block_forward(_ptr(x), x.shape[0], arr, n_seg, _ptr(mod), C.byref(cw),
                                     _ptr(table), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
    return x


def flux3_time_vectors(w_time_in, w_time_out, w_ref_in, w_ref_out, sigma, sigma_next,
                       mode_is_image, vec, workspace, stream=None):
    arr = (I * len(mode_is_image))(*[int(v) for v in mode_is_image])
    _check(lib().flux3_time_vectors(_ptr(w_time_in), _ptr(w_time_out), _ptr(w_ref_in), _ptr(w_ref_out),
                                    float(sigma), float(sigma_next), arr, len(mode_is_image), _ptr(vec),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return vec


class ModelWeights:
    """All device tensors of the transformer plus the C struct that points at
    them.  glob: name -> device bf16 tensor (checkpoint names); early: mode ->
    list of PackedBlock; single: list of PackedBlock."""

    MODES = ("image", "image_cond", "txt")

    def __init__(self, glob: dict, early: dict, single: list):
        self.glob, self.early, self.single = glob, early, single
        n_early = max((len(v) for v in early.values()), default=0)
        for m, blocks in early.items():
            if blocks and len(blocks) != n_early:
                raise ValueError(f"stream {m} has {len(blocks)} stage-1 blocks, expected {n_early}")
        self._early_arr = {}
        cw = ModelWeightsC()
        g = lambda k: _ptr(glob.get(k))
        cw.emb_in_image = g("emb_in.image.weight")
        cw.emb_in_image_cond = g("emb_in.image_cond.weight")
        cw.txt_in = g("txt_in.weight")
        cw.time_in_w1 = g("time_in.in_layer.weight")
        cw.time_in_w2 = g("time_in.out_layer.weight")
        cw.ref_time_in_w1 = g("ref_time_in.in_layer.weight")
        cw.ref_time_in_w2 = g("ref_time_in.out_layer.weight")
        for i, m in enumerate(self.MODES):
            cw.early_mod[i] = g(f"early_stream_modulations.{m}.lin.weight")
            cw.single_mod[i] = g(f"single_stream_modulations.{m}.lin.weight")
            blocks = early.get(m, [])
            if blocks:
                arr = (BlockWeightsC * len(blocks))(*[b.c() for b in blocks])
                self._early_arr[m] = arr
                cw.early[i] = C.cast(arr, C.POINTER(BlockWeightsC))
        self._single_arr = (BlockWeightsC * max(1, len(single)))(*[b.c() for b in single])
        cw.single = C.cast(self._single_arr, C.POINTER(BlockWeightsC))
        cw.n_early = n_early
        cw.n_single = len(single)
        cw.final_ada = g("final_layer.image.adaLN_modulation.1.weight")
        cw.final_linear = g("final_layer.image.linear.weight")
        self.c = cw


def flux3_stack_workspace_size(n_img: int, n_cond: int, n_txt: int) -> int:
    return lib().flux3_stack_workspace_size(n_img, n_cond, n_txt)


def flux3_stack_forward(weights: ModelWeights, img, cond, txt, table, sigma, sigma_next, v,
                        workspace, stream=None):
    n_cond = 0 if cond is None else cond.shape[0]
    n_txt = 0 if txt is None else txt.shape[0]
    _check(lib().flux3_stack_forward(C.byref(weights.c), _ptr(img), img.shape[0], _ptr(cond), n_cond,
                                     _ptr(txt), n_txt, _ptr(table), float(sigma), float(sigma_next),
                                     _ptr(v), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return v


def flux3_sample_workspace_size(n_img: int, n_cond: int, n_txt: int) -> int:
    return lib().flux3_sample_workspace_size(n_img, n_cond, n_txt)


def flux3_sample(weights: ModelWeights, x, cond, txt, table, sigmas, workspace, stream=None):
    """x: device [n_img, 128] fp32, updated in place; sigmas: [steps + 1] host values."""
    _require_dev(x, torch.float32, "x")
    sig = torch.as_tensor(sigmas, dtype=torch.float32).cpu().contiguous()
    n_cond = 0 if cond is None else cond.shape[0]
    n_txt = 0 if txt is None else txt.shape[0]
    _check(lib().flux3_sample(C.byref(weights.c), _ptr(x), x.shape[0], _ptr(cond), n_cond,
                              _ptr(txt), n_txt, _ptr(table), sig.data_ptr(), sig.numel() - 1,
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)))
    return x


def flux3_build_ids_cfg(img_h: int, img_w: int, n_txt0: int, n_txt1: int, refs=()) -> torch.Tensor:
    """Ids of the guided pack's rows (sample 0: image | refs | text 0, sample 1:
    text 1 | image | refs), host fp32 [n, 4]."""
    hw = (I * (2 * len(refs)))(*[int(v) for r in refs for v in r])
    n = I(0)
    _check(lib().flux3_build_ids_cfg(img_h, img_w, len(refs), hw, n_txt0, n_txt1, None, C.byref(n)))
    out = torch.empty((n.value, 4), dtype=torch.float32)
    _check(lib().flux3_build_ids_cfg(img_h, img_w, len(refs), hw, n_txt0, n_txt1, out.data_ptr(), C.byref(n)))
    return out


def _rows(t):
    return 0 if t is None else t.shape[0]


def flux3_stack_cfg_workspace_size(n_img: int, n_cond: int, n_txt0: int, n_txt1: int) -> int:
    return lib().flux3_stack_cfg_workspace_size(n_img, n_cond, n_txt0, n_txt1)


def flux3_stack_forward_cfg(weights: ModelWeights, img, cond, txt0, txt1, table, sigma, sigma_next,
                            guidance, v, workspace, stream=None):
    _check(lib().flux3_stack_forward_cfg(C.byref(weights.c), _ptr(img), img.shape[0], _ptr(cond), _rows(cond),
                                         _ptr(txt0), _rows(txt0), _ptr(txt1), _rows(txt1), _ptr(table),
                                         float(sigma), float(sigma_next), float(guidance), _ptr(v), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
    return v


def flux3_sample_cfg_workspace_size(n_img: int, n_cond: int, n_txt0: int, n_txt1: int) -> int:
    return lib().flux3_sample_cfg_workspace_size(n_img, n_cond, n_txt0, n_txt1)


def flux3_sample_cfg(weights: ModelWeights, x, cond, txt0, txt1, table, sigmas, guidance, workspace, stream=None):
    """x: device [n_img, 128] fp32, updated in place; sigmas: [steps + 1] host values."""
    _require_dev(x, torch.float32, "x")
    sig = torch.as_tensor(sigmas, dtype=torch.float32).cpu().contiguous()
    _check(lib().flux3_sample_cfg(C.byref(weights.c), _ptr(x), x.shape[0], _ptr(cond), _rows(cond),
                                  _ptr(txt0), _rows(txt0), _ptr(txt1), _rows(txt1), _ptr(table),
                                  sig.data_ptr(), sig.numel() - 1, float(guidance), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return x


def flux3_euler_step(x, x_bf16, v, sigma, sigma_next, stream=None):
    _check(lib().flux3_euler_step(_ptr(x), _ptr(x_bf16), _ptr(v), x.numel(), float(sigma),
                                  float(sigma_next), _stream(stream)))


def flux3_sigmas(steps: int, alpha: float = 6.93) -> torch.Tensor:
    out = torch.empty(steps + 1, dtype=torch.float32)
    _check(lib().flux3_sigmas(steps, float(alpha), out.data_ptr()))
    return out


TIMER_KINDS = {"in_proj": 0, "qk_norm_rope": 1, "attention": 2, "out_proj": 3, "ln_modulate": 4}


def flux3_timer_start(kinds, capacity: int):
    """Arm the launch timer for the named kinds (keys of TIMER_KINDS)."""
    mask = 0
    for k in kinds:
        mask |= 1 << TIMER_KINDS[k]
    _check(lib().flux3_timer_start(mask, int(capacity)))


def flux3_timer_stop(capacity: int):
    """Disarm; returns [(kind name, rows, ms)] per recorded launch, in launch order."""
    ms = (C.c_float * capacity)()
    kind = (I * capacity)()
    rows = (I * capacity)()
    n = I(0)
    _check(lib().flux3_timer_stop(C.addressof(ms), C.addressof(kind), C.addressof(rows), int(capacity),
                                  C.byref(n)))
    names = {v: k for k, v in TIMER_KINDS.items()}
    return [(names[kind[i]], rows[i], ms[i]) for i in range(n.value)]


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer for the *_workspace_size calls (256-byte aligned
    by torch's allocator)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
