"""Helpers shared by the GPU parity tests: device checks, conversions, the
agreement criterion, and uploading seeded weights."""
from __future__ import annotations

import sys

import numpy as np
import torch

import flux3_synth as syn

# Agreement for every bf16-path output: cosine >= 0.9995 and
# max |err| <= 2e-2 * max |ref|.
COS_MIN = 0.9995
REL_MAX = 2e-2
# fp8r outputs (rowwise E4M3 projections): the kernel quantizes activations it
# computed in fp32 (and [o | h] after bf16 rounding), the oracle its float64
# values, so codes near a rounding boundary can land one E4M3 step (2^-3 of
# the element) apart: about 1/64 of a row's inputs at bf16-level input
# differences, moving an output by ~0.75% of its rms; the maximum over ~1e5
# outputs lies a few times above that.  Same cosine bar.
FP8_REL_MAX = 5e-2


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import latent_flow_matching_flux3_amd as L
    L.lib()  # raises if the HIP library is missing
    return L


def say(*a):
    """Print what the next GPU step is (flushed, so a dying box still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


def agreement(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert np.all(np.isfinite(got)), "non-finite output"
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
    rel = float(np.max(np.abs(got - ref)) / (np.max(np.abs(ref)) + 1e-300))
    return cos, rel


def assert_agree(got, ref, what: str, cos_min: float = COS_MIN, rel_max: float = REL_MAX):
    cos, rel = agreement(got, ref)
    say(f"  {what}: cos={cos:.7f} max_err/max_ref={rel:.3e}")
    assert cos >= cos_min and rel <= rel_max, f"{what}: cos={cos} rel={rel}"


def block_weights_cpu(seed: int, prefix: str = "single_blocks.0", scales: str = "uniform") -> dict:
    return syn.block_weights(seed, prefix, scales)


def upload(w: dict) -> dict:
    return {k: dev(v) for k, v in w.items()}


def to_f64(w: dict) -> dict:
    return {k: f64(v) for k, v in w.items()}
