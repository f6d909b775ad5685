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


def test_attention_noalloc_graph_replays():
    """What the entry point is for: captured into a HIP graph (after one
    eager call on the device) and replayed, with other work and fresh inputs
    between replays, each replay equals the workspace call on its inputs (the
    counters are cleared by a captured fill kernel every time)."""
    L = require_gpu()
    n = 4608
    q0 = syn.normal_bf16((n, 9216), 1.0, 95, "att.noalloc.graph")
    d = dev(q0)
    o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    L.flux3_attention_noalloc(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("attention_noalloc graph capture")
    with torch.cuda.graph(g, stream=side):
        L.flux3_attention_noalloc(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o)
    ws = L.workspace(L.flux3_attention_workspace_size(n))
    ref = torch.empty_like(o)
    for rep in range(3):
        d.copy_(dev(syn.normal_bf16((n, 9216), 1.0 + rep, 96 + rep, f"att.noalloc.graph.{rep}")))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        L.flux3_attention_ws(d[:, :3072], d[:, 3072:6144], d[:, 6144:], ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"replay {rep} differs from the workspace call"
    del g
