"""flux3_attention_noalloc (the balanced attention schedule with its
workspace in the library's static device memory) against flux3_attention_ws
with a caller workspace: the same kernels, so the outputs must be identical,
on consecutive calls of decreasing size (the static scratch keeps the last
call's contents; its counters must be cleared by each call)."""
import pytest
import torch

import flux3_synth as syn
from gpu_util import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def test_attention_noalloc_matches_workspace_calls():
    L = require_gpu()
    for i, n in enumerate((4608, 2817, 300)):
        qkv = syn.normal_bf16((n, 9216), 1.0, 90 + i, f"att.noalloc.{n}")
        d = dev(qkv)
        q, k, v = d[:, :3072], d[:, 3072:6144], d[:, 6144:]
        say(f"attention_noalloc n={n} (call {i + 1})")
        o_static = torch.full((n, 3072), float("nan"), dtype=torch.bfloat16, device="cuda")
        L.flux3_attention_noalloc(q, k, v, o_static)
        ws_bytes = L.flux3_attention_workspace_size(n)
        ws = L.workspace(ws_bytes) if ws_bytes else None
        o_ws = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
        L.flux3_attention_ws(q, k, v, o_ws, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(o_static.float()).all().item()
        assert torch.equal(o_static, o_ws), f"n={n}: static-scratch attention differs from the workspace call"
