"""Every kernel twice on the same inputs: the outputs must be equal bit for
bit (no atomics in a reduction order, no dependence on which workgroup
finishes first: the balanced attention schedule merges its parts in a fixed
order; the stack's side stream changes nothing)."""
import numpy as np
import pytest
import torch

import flux3_synth as syn
import oracle as O
from gpu_util import dev, require_gpu, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    return require_gpu()


def _twice(fn):
    a = fn()
    torch.cuda.synchronize()
    b = fn()
    torch.cuda.synchronize()
    return a, b


def _equal(a, b, what):
    assert a.shape == b.shape and torch.equal(a, b), f"{what}: two runs differ"


@pytest.mark.parametrize("n", [300, 2817, 4608])
def test_attention_twice(L, n):
    qkv = dev(syn.normal_bf16((n, 9216), 1.0, 61, f"det.att.{n}"))
    ws_bytes = L.flux3_attention_workspace_size(n)
    ws = L.workspace(ws_bytes) if ws_bytes else None
    say(f"determinism attention n={n}")

    def run():
        o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
        L.flux3_attention_ws(qkv[:, :3072], qkv[:, 3072:6144], qkv[:, 6144:], o, ws)
        return o

    _equal(*_twice(run), f"attention_ws n={n}")


@pytest.mark.parametrize("fp8", [False, True])
def test_block_and_kernels_twice(L, fp8):
    lay = syn.Layout(40, 60, 312)          # 2712 rows: balanced attention, ragged tiles
    n = lay.n_total
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt)
    segs = [0, lay.n_img, n]
    w = upload(syn.block_weights(62, "single_blocks.0"))
    blk = L.PackedBlock(w, fp8=fp8)
    x0 = dev(syn.block_activations(63, n)).float()
    mods = dev(syn.normal_f32((2, 3, 3072), 0.5, 64, "mods"))
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    ws = L.workspace(L.flux3_block_workspace_size(n))
    say(f"determinism block n={n} fp8={fp8}")

    def block():
        x = x0.clone()
        L.flux3_block_forward(x, segs, mods, blk, table, ws)
        return x

    _equal(*_twice(block), f"block fp8={fp8}")
    if fp8:
        return
    xm = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")

    def ln():
        L.flux3_ln_modulate(x0, xm, segs, mods)
        return xm.clone()

    _equal(*_twice(ln), "ln_modulate")
    qkv = torch.empty((n, 9216), dtype=torch.bfloat16, device="cuda")
    # the o part of [o | h] gets seeded values (the in-projection writes h):
    # left uninitialised it may hold NaN patterns, which compare unequal
    cat = torch.empty((n, 12288), dtype=torch.bfloat16, device="cuda")
    cat[:, :3072] = dev(syn.normal_bf16((n, 3072), 1.0, 66, "det.o"))

    def in_proj():
        L.flux3_block_in_proj(xm, blk.w_in, qkv, cat[:, 3072:])
        return torch.cat([qkv, cat[:, 3072:]], 1)

    _equal(*_twice(in_proj), "block_in_proj")
    q0 = qkv.clone()

    def norm_rope():
        t = q0.clone()
        L.flux3_qk_norm_rope(t[:, :3072], t[:, 3072:6144], blk.q_scale, blk.k_scale, table)
        return t

    _equal(*_twice(norm_rope), "qk_norm_rope")

    def out_proj():
        x = x0.clone()
        L.flux3_block_out_proj(cat, blk.w_out, x, segs, mods)
        return x

    _equal(*_twice(out_proj), "block_out_proj")


def test_stack_twice(L):
    """The stack with references and text (stage 1's side stream, split-K
    text embedding), twice."""
    lay = syn.Layout(12, 12, 40, [(12, 12)])
    seed = 65
    glob = {k: dev(syn.global_weight(seed, k)) for k in syn.GLOBAL_SHAPES}
    early = {m: [L.PackedBlock(upload(syn.block_weights(seed, syn.early_prefix(m, 0))))] for m in syn.MODES}
    model = L.ModelWeights(glob, early, [L.PackedBlock(upload(syn.block_weights(seed, "single_blocks.0")))])
    img, cond, txt = (dev(t) for t in syn.stack_inputs(lay, seed))
    table = L.flux3_rope_table(L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs).to("cuda"))
    ws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, lay.n_cond, lay.n_txt))
    say("determinism stack")

    def run():
        v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
        L.flux3_stack_forward(model, img, cond, txt, table, 0.7, 0.6, v, ws)
        return v

    a, b = _twice(run)
    assert np.isfinite(a.cpu().numpy()).all()
    _equal(a, b, "stack_forward")


@pytest.mark.parametrize("fp8", [False, True])
def test_block_dirty_workspace(L, fp8):
    """A block workspace needs no initial contents: its counters (the balanced
    attention's and the stream-K output projection's) are cleared inside the
    block, by the in-projection above 256 rows or by the QK norm kernel where
    that runs on its own (fp8r blocks).  The same block on a workspace of
    0xFF bytes (every counter -1) and on a zeroed one: equal bit for bit."""
    lay = syn.Layout(48, 48, 513)          # 2817 rows: balanced attention and stream-K
    n = lay.n_total
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt)
    segs = [0, lay.n_img, n]
    blk = L.PackedBlock(upload(syn.block_weights(65, "single_blocks.0")), fp8=fp8)
    x0 = dev(syn.block_activations(66, n)).float()
    mods = dev(syn.normal_f32((2, 3, 3072), 0.5, 67, "mods"))
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    ws = L.workspace(L.flux3_block_workspace_size(n))
    say(f"dirty workspace block n={n} fp8={fp8}")
    out = []
    for fill in (0, 255):
        ws.fill_(fill)
        x = x0.clone()
        L.flux3_block_forward(x, segs, mods, blk, table, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(x).all().item()
        out.append(x)
    _equal(out[0], out[1], f"block on a dirty workspace fp8={fp8}")
