"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and arranges them in the shapes of the
FLUX.3 Image Klein transformer; it holds none of the model's arithmetic.  Every
tensor is drawn from its own torch CPU generator whose seed is derived from a
base seed and the tensor's name, so any single tensor can be regenerated on its
own (the oracle streams the 5.5 B-parameter model one block at a time).

Values are drawn in float32 and rounded once to bfloat16 (round-to-nearest-even
by torch), which is the storage format of the checkpoint ("all BF16, no
biases": "[Feature] FLUX.3 Image Klein support #2142", comment listing the
tensor names).  The oracle upcasts those exact bf16 values to float64.

Distributions (the synthetic recipe):
  * weights            ~ N(0, 0.02^2)
  * activations/latents ~ N(0, 1)
  * conditioning vecs  ~ N(0, 1)
  * RMSNorm scales     ~ U(0.5, 1.5) for parity runs, ones for throughput runs
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import torch

HIDDEN = 3072
HEADS = 24
HEAD_DIM = 128
MLP_HIDDEN = 9216
LATENT_CH = 128
TXT_FEAT = 20480
TIME_FEAT = 256
N_EARLY = 5
N_SINGLE = 28
MODES = ("image", "image_cond", "txt")

WEIGHT_STD = 0.02


def _seed(seed: int, name: str) -> int:
    return (int(seed) * 0x9E3779B1 + zlib.crc32(name.encode())) % (2**63 - 1)


def gen(seed: int, name: str) -> torch.Generator:
    return torch.Generator().manual_seed(_seed(seed, name))


def normal_bf16(shape, std: float, seed: int, name: str) -> torch.Tensor:
    """N(0, std^2) draws rounded to bf16 (torch CPU tensor)."""
    x = torch.randn(*shape, generator=gen(seed, name), dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def uniform_bf16(shape, lo: float, hi: float, seed: int, name: str) -> torch.Tensor:
    x = torch.rand(*shape, generator=gen(seed, name), dtype=torch.float32)
    return (x * (hi - lo) + lo).to(torch.bfloat16)


def normal_f32(shape, std: float, seed: int, name: str) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen(seed, name), dtype=torch.float32)
    return x * std if std != 1.0 else x


# ----------------------------------------------------------------------------
# Weights, in the checkpoint's own names and [out, in] shapes.
# ----------------------------------------------------------------------------

BLOCK_SHAPES = {
    "q_proj": (HIDDEN, HIDDEN),
    "k_proj": (HIDDEN, HIDDEN),
    "v_proj": (HIDDEN, HIDDEN),
    "attn_out": (HIDDEN, HIDDEN),
    "mlp_in": (2 * MLP_HIDDEN, HIDDEN),
    "mlp_out": (HIDDEN, MLP_HIDDEN),
    "norm.query_norm.scale": (HEAD_DIM,),
    "norm.key_norm.scale": (HEAD_DIM,),
}


def block_prefixes(n_early: int = N_EARLY, n_single: int = N_SINGLE):
    """Names of every transformer block, stage-1 blocks first."""
    out = []
    for i in range(n_early):
        out.append(f"content_mode_blocks.image.{i}")
    for i in range(n_early):
        out.append(f"content_mode_blocks.image_cond.{i}")
    for i in range(n_early):
        out.append(f"txt_mode_blocks.{i}")
    for i in range(n_single):
        out.append(f"single_blocks.{i}")
    return out


def early_prefix(mode: str, i: int) -> str:
    return f"txt_mode_blocks.{i}" if mode == "txt" else f"content_mode_blocks.{mode}.{i}"


def block_weights(seed: int, prefix: str, norm_scales: str = "uniform") -> dict:
    """One block's weights.  norm_scales: 'uniform' (U(0.5,1.5)) or 'ones'."""
    w = {}
    for k, shp in BLOCK_SHAPES.items():
        name = f"{prefix}.{k}"
        if k.endswith("scale"):
            if norm_scales == "ones":
                w[k] = torch.ones(shp, dtype=torch.bfloat16)
            else:
                w[k] = uniform_bf16(shp, 0.5, 1.5, seed, name)
        else:
            w[k] = normal_bf16(shp, WEIGHT_STD, seed, name)
    return w


GLOBAL_SHAPES = {
    "emb_in.image.weight": (HIDDEN, LATENT_CH),
    "emb_in.image_cond.weight": (HIDDEN, LATENT_CH),
    "txt_in.weight": (HIDDEN, TXT_FEAT),
    "time_in.in_layer.weight": (HIDDEN, TIME_FEAT),
    "time_in.out_layer.weight": (HIDDEN, HIDDEN),
    "ref_time_in.in_layer.weight": (HIDDEN, TIME_FEAT),
    "ref_time_in.out_layer.weight": (HIDDEN, HIDDEN),
    "early_stream_modulations.image.lin.weight": (3 * HIDDEN, HIDDEN),
    "early_stream_modulations.image_cond.lin.weight": (3 * HIDDEN, HIDDEN),
    "early_stream_modulations.txt.lin.weight": (3 * HIDDEN, HIDDEN),
    "single_stream_modulations.image.lin.weight": (3 * HIDDEN, HIDDEN),
    "single_stream_modulations.image_cond.lin.weight": (3 * HIDDEN, HIDDEN),
    "single_stream_modulations.txt.lin.weight": (3 * HIDDEN, HIDDEN),
    "final_layer.image.adaLN_modulation.1.weight": (2 * HIDDEN, HIDDEN),
    "final_layer.image.linear.weight": (LATENT_CH, HIDDEN),
}


def global_weight(seed: int, name: str) -> torch.Tensor:
    return normal_bf16(GLOBAL_SHAPES[name], WEIGHT_STD, seed, name)


def all_tensor_shapes(flow_map: bool = True, n_early: int = N_EARLY, n_single: int = N_SINGLE) -> dict:
    """Name -> shape for every tensor of the transformer checkpoint."""
    shapes = {}
    for k, v in GLOBAL_SHAPES.items():
        if not flow_map and k.startswith("ref_time_in"):
            continue
        shapes[k] = v
    for p in block_prefixes(n_early, n_single):
        for k, v in BLOCK_SHAPES.items():
            shapes[f"{p}.{k}"] = v
    return shapes


# ----------------------------------------------------------------------------
# Workloads: token layouts and activations.
# ----------------------------------------------------------------------------

@dataclass
class Layout:
    """Token layout of one sample: image grid, reference grids, text length."""
    img_h: int
    img_w: int
    n_txt: int
    refs: list = field(default_factory=list)  # list of (h, w) token grids

    @property
    def n_img(self) -> int:
        return self.img_h * self.img_w

    @property
    def n_cond(self) -> int:
        return sum(h * w for h, w in self.refs)

    @property
    def n_total(self) -> int:
        return self.n_img + self.n_cond + self.n_txt

    def segments(self):
        """(mode, start, end) row ranges in the order image, image_cond, txt."""
        out = []
        s = 0
        for mode, n in (("image", self.n_img), ("image_cond", self.n_cond), ("txt", self.n_txt)):
            if n > 0:
                out.append((mode, s, s + n))
                s += n
        return out


# The five workloads: single block at 128x128 px, 1024^2 t2i, 1024^2 i2i with one
# reference; the full stack at 1024^2 t2i; the full stack with 4 references.
WORKLOADS = {
    "block_128px_96tok": Layout(8, 8, 32),
    "block_t2i_1024_4608tok": Layout(64, 64, 512),
    "block_i2i_1024_8704tok": Layout(64, 64, 512, [(64, 64)]),
    "stack_t2i_1024_4608tok": Layout(64, 64, 512),
    "stack_4ref_1024_20992tok": Layout(64, 64, 512, [(64, 64)] * 4),
}

# The token counts of the blog's tokens-per-call chart (What it costs to run):
# image tokens, references at their own size, and text padded to a multiple of
# 80 (the text lengths are what the chart's totals leave; the features are
# random stand-ins for a prompt of that padded length).  1360x768 px is an
# 85-wide, 48-high token grid.
PAGE_WORKLOADS = {
    "block_t2i_1024_page_4256tok": Layout(64, 64, 160),
    "block_i2i_1024_page_8272tok": Layout(64, 64, 80, [(64, 64)]),
    "block_layout_t2i_1024_page_4336tok": Layout(64, 64, 240),
    "block_layout_i2i_1360x768_page_8800tok": Layout(48, 85, 640, [(48, 85)]),
}

# The longest sequence the pages allow: a 1024^2 image, ten 1024^2 references
# and the text at its cap (the largest multiple of 80 not above 4096).
LONG_WORKLOADS = {
    "stack_10ref_1024_49136tok": Layout(64, 64, 4080, [(64, 64)] * 10),
}


def block_activations(seed: int, n: int) -> torch.Tensor:
    """Residual-stream input of one block, N(0,1) bf16 [n, 3072]."""
    return normal_bf16((n, HIDDEN), 1.0, seed, f"x.{n}")


def cond_vectors(seed: int, n_modes: int = 3) -> torch.Tensor:
    """Random conditioning vectors, one per mode, fp32 [n_modes, 3072]."""
    return normal_f32((n_modes, HIDDEN), 1.0, seed, "vec")


def latents(seed: int, n: int, name: str = "img") -> torch.Tensor:
    return normal_bf16((n, LATENT_CH), 1.0, seed, f"latent.{name}.{n}")


def text_features(seed: int, n: int) -> torch.Tensor:
    return normal_bf16((n, TXT_FEAT), 1.0, seed, f"txt.{n}")


def stack_inputs(lay: Layout, seed: int):
    """Inputs of one transformer call on layout `lay`: image latents
    [n_img, 128], reference latents [n_cond, 128] (None without references)
    and text features [n_txt, 20480], all bf16 (torch CPU)."""
    img = latents(seed + 1, lay.n_img)
    cond = latents(seed + 2, lay.n_cond, "cond") if lay.n_cond else None
    txt = text_features(seed + 3, lay.n_txt)
    return img, cond, txt
