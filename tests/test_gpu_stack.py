"""GPU parity of the whole transformer (flux3_stack_forward) and of the
16-step flow-map sampler against the CPU oracle.

Weights and inputs are seeded bf16 from flux3_synth; the GPU gets exactly the
values the oracle reads.  Reduced-depth stacks keep the real widths (hidden
3072, 24 heads, mlp 9216) and only run fewer blocks; one test runs the full
5 + 28 depth with all ~5.5 B parameters."""
import hashlib
import json
import os
import sys

import numpy as np
import pytest
import torch

import flux3_synth as syn
import oracle as O
from gpu_util import FP8_REL_MAX, assert_agree, dev, f64, require_gpu, say

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLD)
import make_stack_golden  # noqa: E402  (fingerprints of the stored cases' inputs)


@pytest.fixture(scope="module")
def L():
    return require_gpu()


class Weights:
    """Seeded weights: device copies for the library, float64 views for the oracle."""

    def __init__(self, L, seed, lay, n_early, n_single, base=False, fp8=False):
        """base: the base checkpoint's tensor set (no ref_time_in); fp8: fp8r blocks."""
        self.seed = seed
        self.fp8 = fp8
        self.glob_cpu = {k: syn.global_weight(seed, k) for k in syn.GLOBAL_SHAPES
                         if not (base and k.startswith("ref_time_in."))}
        glob = {k: dev(v) for k, v in self.glob_cpu.items()}
        modes = ["image"] + (["image_cond"] if lay.n_cond else []) + ["txt"]
        early = {}
        for m in syn.MODES:
            early[m] = [self._packed(L, syn.early_prefix(m, i)) for i in range(n_early)] if m in modes else []
        single = [self._packed(L, f"single_blocks.{i}") for i in range(n_single)]
        self.model = L.ModelWeights(glob, early, single)
        self._w64 = {}

    def _packed(self, L, prefix):
        w = {k: dev(v) for k, v in syn.block_weights(self.seed, prefix).items()}
        b = L.PackedBlock(w, fp8=self.fp8)
        torch.cuda.synchronize()
        return b

    def W(self, name):
        if name not in self._w64:
            self._w64[name] = f64(self.glob_cpu[name])
        return self._w64[name]

    def B(self, prefix):
        return {k: f64(v) for k, v in syn.block_weights(self.seed, prefix).items()}


def _inputs(lay, seed):
    img = syn.latents(seed + 1, lay.n_img)
    cond = syn.latents(seed + 2, lay.n_cond, "cond") if lay.n_cond else None
    txt = syn.text_features(seed + 3, lay.n_txt)
    return img, cond, txt


def _gpu_stack(L, wts, lay, img, cond, txt, sigma, sigma_next):
    ids = L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs).to("cuda")
    table = L.flux3_rope_table(ids)
    ws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, lay.n_cond, lay.n_txt))
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    L.flux3_stack_forward(wts.model, dev(img), None if cond is None else dev(cond), dev(txt), table,
                          sigma, sigma_next, v, ws)
    torch.cuda.synchronize()
    return v


@pytest.mark.parametrize("lay,n_early,n_single", [
    (syn.Layout(4, 4, 8), 1, 2),
    (syn.Layout(3, 5, 11, [(2, 3), (4, 2)]), 2, 1),
    (syn.Layout(12, 12, 40, [(12, 12)]), 1, 1),
    (syn.Layout(3, 4, 80, [(2, 3)] * 10), 1, 1),   # ten references: l = -1 .. -10
])
def test_stack_reduced_depth(L, lay, n_early, n_single):
    seed = 100 + lay.n_total
    say(f"stack n={lay.n_total} depth {n_early}+{n_single}")
    wts = Weights(L, seed, lay, n_early, n_single)
    img, cond, txt = _inputs(lay, seed)
    sig, sig_next = np.float32(0.8739), np.float32(0.6979)
    v = _gpu_stack(L, wts, lay, img, cond, txt, float(sig), float(sig_next))
    ref = O.stack_forward(wts.W, wts.B, f64(img), None if cond is None else f64(cond), f64(txt),
                          lay.img_h, lay.img_w, lay.refs, float(sig), float(sig_next), n_early, n_single)
    assert_agree(f64(v), ref, f"stack n={lay.n_total}")


@pytest.mark.timeout(600)
def test_stack_full_tokens_reduced_depth(L):
    """The benchmarked launch, flux3_stack_forward on the 1024^2 text-to-image
    tokens (64x64 image + 512 text = 4608), at depth 1 + 1: stage 1 on its two
    streams (the 4096-row image block on the balanced attention schedule, the
    text block on the side stream), the joint block at 4608 rows (balanced
    schedule too), the final layer; every output row against the oracle."""
    lay = syn.WORKLOADS["stack_t2i_1024_4608tok"]
    seed = 17
    say(f"stack n={lay.n_total} depth 1+1")
    wts = Weights(L, seed, lay, 1, 1)
    img, cond, txt = _inputs(lay, seed)
    sig, sig_next = np.float32(0.6), np.float32(0.45)
    v = _gpu_stack(L, wts, lay, img, cond, txt, float(sig), float(sig_next))
    say("  oracle")
    ref = O.stack_forward(wts.W, wts.B, f64(img), None, f64(txt), lay.img_h, lay.img_w, [],
                          float(sig), float(sig_next), 1, 1)
    assert_agree(f64(v), ref, f"stack n={lay.n_total} depth 1+1")


@pytest.fixture(scope="module")
def full_model(L):
    """All 5 + 28 blocks of the transformer with every stream's stage-1
    blocks (image, image_cond, text: every checkpoint tensor, ~5.5 B
    parameters) from seed 7."""
    say("generating the 5 + 28 block transformer (5.5B parameters)")
    return Weights(L, 7, syn.WORKLOADS["stack_4ref_1024_20992tok"], 5, 28)


@pytest.mark.timeout(900)
def test_stack_full_depth(L, full_model):
    """All 5 + 28 blocks and every checkpoint tensor, at the smallest
    workload (8x8 image tokens + 32 text tokens)."""
    lay = syn.Layout(8, 8, 32)
    seed = 7
    wts = full_model
    img, cond, txt = _inputs(lay, seed)
    sig, sig_next = np.float32(1.0), np.float32(0.9541)
    say("stack full depth: GPU")
    v = _gpu_stack(L, wts, lay, img, cond, txt, float(sig), float(sig_next))
    say("stack full depth: oracle")
    ref = O.stack_forward(wts.W, wts.B, f64(img), None, f64(txt), lay.img_h, lay.img_w, [],
                          float(sig), float(sig_next), 5, 28)
    assert_agree(f64(v), ref, "stack full depth n=96")


def _golden(name):
    """The oracle's v for a workload too slow to recompute here, written by
    tests/golden/make_stack_golden.py (which calls only the oracle and the
    seeded generators), with the case's description and input fingerprint."""
    with open(os.path.join(GOLD, "stack_golden.json")) as f:
        meta = json.load(f)[name]
    path = os.path.join(GOLD, meta["file"])
    with open(path, "rb") as f:
        assert hashlib.sha256(f.read()).hexdigest() == meta["sha256"], f"{path} changed"
    return meta, np.load(path)


def _check_fingerprint(meta):
    fp = make_stack_golden.fingerprint(meta)
    for k, v in meta["fingerprint"].items():
        assert fp[k] == pytest.approx(v, rel=1e-12, abs=1e-9), f"seeded input {k} differs from the golden's"


@pytest.mark.timeout(900)
def test_stack_full_depth_t2i_1024(L, full_model):
    """The headline workload: flux3_stack_forward with all 5 + 28 blocks on
    the 1024^2 text-to-image tokens (64x64 image + 512 text = 4608) in the
    benchmarked launch (stage 1's side stream, the balanced attention
    schedule), every row of v against the oracle's (stored)."""
    meta, ref = _golden("stack_t2i_1024_4608tok_5+28")
    _check_fingerprint(meta)
    lay = syn.WORKLOADS[meta["layout"]]
    img, cond, txt = syn.stack_inputs(lay, meta["seed"])
    say(f"stack full depth n={lay.n_total}: GPU")
    v = _gpu_stack(L, full_model, lay, img, cond, txt, meta["sigma"], meta["sigma_next"])
    assert_agree(f64(v), ref, f"stack 5+28 n={lay.n_total}")


@pytest.mark.timeout(900)
def test_stack_full_depth_4ref_1024(L, full_model):
    """The longest configuration at full depth: flux3_stack_forward with all
    5 + 28 blocks on four 1024^2 references + a 1024^2 image + 512 text tokens
    (20,992 tokens; the 16,384-row reference stream through its own five
    stage-1 blocks on the side stream), every row of v against the oracle's
    (stored)."""
    meta, ref = _golden("stack_4ref_1024_20992tok_5+28")
    _check_fingerprint(meta)
    lay = syn.WORKLOADS[meta["layout"]]
    img, cond, txt = syn.stack_inputs(lay, meta["seed"])
    say(f"stack full depth n={lay.n_total}: GPU")
    v = _gpu_stack(L, full_model, lay, img, cond, txt, meta["sigma"], meta["sigma_next"])
    assert_agree(f64(v), ref, f"stack 5+28 n={lay.n_total}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["stack_i2i_1024_8704tok_1+1", "stack_4ref_1024_20992tok_1+1"])
def test_stack_references_1024(L, name):
    """flux3_stack_forward with references at their full size, depth 1 + 1,
    every row of v against the oracle's (stored): one 1024^2 reference (8704
    tokens: the image and reference streams' stage-1 attention both on the
    balanced schedule, on two streams with their own workspaces at once) and
    four (20,992 tokens, 16,384 reference rows in one stage-1 stream)."""
    meta, ref = _golden(name)
    _check_fingerprint(meta)
    lay = syn.WORKLOADS[meta["layout"]]
    wts = Weights(L, meta["seed"], lay, meta["n_early"], meta["n_single"])
    img, cond, txt = syn.stack_inputs(lay, meta["seed"])
    say(f"stack n={lay.n_total} depth 1+1: GPU")
    v = _gpu_stack(L, wts, lay, img, cond, txt, meta["sigma"], meta["sigma_next"])
    assert_agree(f64(v), ref, f"stack n={lay.n_total}")


@pytest.mark.timeout(600)
def test_stack_fp8r_t2i_1024(L):
    """The fp8r transformer (every block Linear a rowwise-FP8 product of its
    own) on the 1024^2 text-to-image tokens, depth 1 + 1, every row of v
    against the oracle's fp8r stack (stored), at the fp8r block bar."""
    meta, ref = _golden("stack_t2i_1024_4608tok_fp8r_1+1")
    _check_fingerprint(meta)
    lay = syn.WORKLOADS[meta["layout"]]
    wts = Weights(L, meta["seed"], lay, meta["n_early"], meta["n_single"], fp8=True)
    img, cond, txt = syn.stack_inputs(lay, meta["seed"])
    say(f"stack fp8r n={lay.n_total} depth 1+1: GPU")
    v = _gpu_stack(L, wts, lay, img, cond, txt, meta["sigma"], meta["sigma_next"])
    assert_agree(f64(v), ref, f"stack fp8r n={lay.n_total}", rel_max=FP8_REL_MAX)


def test_flow_map_sampler(L):
    """Four sampler steps through a reduced-depth stack: the GPU loop of
    stack_forward + euler_step against the oracle's sample_flow_map."""
    lay = syn.Layout(4, 4, 8)
    seed = 300
    wts = Weights(L, seed, lay, 1, 1)
    img, _, txt = _inputs(lay, seed)
    steps = 4
    sig = L.flux3_sigmas(steps).tolist()
    ids = L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt).to("cuda")
    table = L.flux3_rope_table(ids)
    ws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, 0, lay.n_txt))
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    x = dev(img).float()
    xb = dev(img)
    txt_d = dev(txt)
    say("sampler 4 steps")
    for k in range(steps):
        L.flux3_stack_forward(wts.model, xb, None, txt_d, table, sig[k], sig[k + 1], v, ws)
        L.flux3_euler_step(x, xb, v, sig[k], sig[k + 1])
    torch.cuda.synchronize()

    def velocity(xx, s, sn):
        return O.stack_forward(wts.W, wts.B, xx, None, f64(txt), lay.img_h, lay.img_w, [], s, sn, 1, 1)

    xr = O.sample_flow_map(velocity, f64(img), steps)
    assert_agree(f64(x), xr, "sampler 4 steps")


def _sample_setup(L, lay, seed, n_early, n_single):
    wts = Weights(L, seed, lay, n_early, n_single)
    img, cond, txt = _inputs(lay, seed)
    ids = L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs).to("cuda")
    table = L.flux3_rope_table(ids)
    return wts, img, cond, txt, table


def test_sample_one_call(L):
    """flux3_sample (the whole loop in one call) on a non-square grid with a
    reference and an 80-token text: bit-identical to the step-by-step calls,
    and within tolerance of the oracle's sampler."""
    lay = syn.Layout(6, 11, 80, [(6, 11)])
    seed = 310
    steps = 3
    wts, img, cond, txt, table = _sample_setup(L, lay, seed, 1, 1)
    sig = L.flux3_sigmas(steps)
    cond_d, txt_d = dev(cond), dev(txt)
    say(f"sample one call n={lay.n_total} steps={steps}")
    x = dev(img).float()
    ws = L.workspace(L.flux3_sample_workspace_size(lay.n_img, lay.n_cond, lay.n_txt))
    L.flux3_sample(wts.model, x, cond_d, txt_d, table, sig, ws)
    # the same loop through the per-step entry points
    xs, xb = dev(img).float(), dev(img)
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    sws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, lay.n_cond, lay.n_txt))
    s = sig.tolist()
    for k in range(steps):
        L.flux3_stack_forward(wts.model, xb, cond_d, txt_d, table, s[k], s[k + 1], v, sws)
        L.flux3_euler_step(xs, xb, v, s[k], s[k + 1])
    torch.cuda.synchronize()
    assert torch.equal(x, xs), "flux3_sample differs from the step-by-step loop"

    def velocity(xx, a, b):
        return O.stack_forward(wts.W, wts.B, xx, f64(cond), f64(txt), lay.img_h, lay.img_w, lay.refs,
                               a, b, 1, 1)

    xr = O.sample_flow_map(velocity, f64(img), steps)
    assert_agree(f64(x), xr, f"sample {steps} steps")
    # zero steps leave x alone
    x0 = x.clone()
    L.flux3_sample(wts.model, x, cond_d, txt_d, table, sig[:1], ws)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)


@pytest.mark.parametrize("base", [False, True])
def test_sample_conditioning_chunks(L, base):
    """flux3_sample computes the conditioning of up to eight steps at a time:
    10 steps (a chunk of eight, then two) equal the step-by-step calls bit for
    bit, with the flow-map checkpoint's ref_time_in and without it."""
    lay = syn.Layout(4, 4, 8)
    seed = 330 + int(base)
    steps = 10
    wts = Weights(L, seed, lay, 1, 1, base=base)
    img, _, txt = _inputs(lay, seed)
    table = L.flux3_rope_table(L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt).to("cuda"))
    sig = L.flux3_sigmas(steps)
    txt_d = dev(txt)
    say(f"sample conditioning chunks: {steps} steps, base={base}")
    x = dev(img).float()
    ws = L.workspace(L.flux3_sample_workspace_size(lay.n_img, 0, lay.n_txt))
    L.flux3_sample(wts.model, x, None, txt_d, table, sig, ws)
    xs, xb = dev(img).float(), dev(img)
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    sws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, 0, lay.n_txt))
    s = sig.tolist()
    for k in range(steps):
        L.flux3_stack_forward(wts.model, xb, None, txt_d, table, s[k], s[k + 1], v, sws)
        L.flux3_euler_step(xs, xb, v, s[k], s[k + 1])
    torch.cuda.synchronize()
    assert torch.isfinite(x).all()
    assert torch.equal(x, xs), "flux3_sample differs from the step-by-step loop"


def test_sample_graph_replays(L):
    """flux3_sample captured into one HIP graph: every replay (with eager
    library work and synchronisations between replays, sharing the
    workspace) equals the eager call bit for bit."""
    lay = syn.Layout(4, 4, 8)
    seed = 320
    wts, img, _, txt, table = _sample_setup(L, lay, seed, 1, 1)
    sig = L.flux3_sigmas(4)
    txt_d = dev(txt)
    ws = L.workspace(L.flux3_sample_workspace_size(lay.n_img, 0, lay.n_txt))
    x0 = dev(img).float()
    xe = x0.clone()
    say("sample graph: eager")
    L.flux3_sample(wts.model, xe, None, txt_d, table, sig, ws)
    torch.cuda.synchronize()
    xg = x0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.flux3_sample(wts.model, xg, None, txt_d, table, sig, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(xg, xe)
    say("sample graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.flux3_sample(wts.model, xg, None, txt_d, table, sig, ws)
    for r in range(3):
        say(f"sample graph: replay {r}")
        xo = x0.clone()
        L.flux3_sample(wts.model, xo, None, txt_d, table, sig[:3], ws)  # eager work in between
        xg.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, xe), f"replay {r} differs from the eager call"


def _cfg_case(L, seed, lay, n_txt1, n_early=1, n_single=1):
    wts = Weights(L, seed, lay, n_early, n_single, base=True)
    img, cond, txt0 = _inputs(lay, seed)          # txt0: the empty prompt (lay.n_txt rows)
    txt1 = syn.text_features(seed + 4, n_txt1)    # the prompt
    ids = L.flux3_build_ids_cfg(lay.img_h, lay.img_w, lay.n_txt, n_txt1, lay.refs).to("cuda")
    table = L.flux3_rope_table(ids)
    return wts, img, cond, txt0, txt1, table


def _oracle_velocity(wts, lay, cond, txts, n_early, n_single):
    def velocity(x, sigma, i):
        return O.stack_forward(wts.W, wts.B, x, None if cond is None else f64(cond), f64(txts[i]),
                               lay.img_h, lay.img_w, lay.refs, sigma, None, n_early, n_single)
    return velocity


def test_stack_cfg_pack(L):
    """The base checkpoint's guided pack (image and references shared through
    stage 1, texts side by side, both samples in one stage-2 pass) against
    the oracle's two separate stacks and guidance; also against two separate
    GPU stack calls."""
    lay = syn.Layout(3, 5, 80, [(2, 3), (3, 2)])
    n_txt1 = 160
    seed = 330
    g = 3.5
    wts, img, cond, txt0, txt1, table = _cfg_case(L, seed, lay, n_txt1)
    say(f"stack cfg pack n_img={lay.n_img} n_cond={lay.n_cond} texts {lay.n_txt}/{n_txt1}")
    ws = L.workspace(L.flux3_stack_cfg_workspace_size(lay.n_img, lay.n_cond, lay.n_txt, n_txt1))
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    sig = 0.8739
    L.flux3_stack_forward_cfg(wts.model, dev(img), dev(cond), dev(txt0), dev(txt1), table, sig, 0.0, g, v, ws)
    torch.cuda.synchronize()
    vel = _oracle_velocity(wts, lay, cond, [txt0, txt1], 1, 1)
    v0, v1 = vel(f64(img), sig, 0), vel(f64(img), sig, 1)
    assert_agree(f64(v), O.cfg_velocity(v0, v1, g), "cfg pack vs oracle")
    # the same two samples through flux3_stack_forward one at a time
    outs = []
    for t in (txt0, txt1):
        ids = L.flux3_build_ids(lay.img_h, lay.img_w, t.shape[0], lay.refs).to("cuda")
        sws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, lay.n_cond, t.shape[0]))
        vi = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
        L.flux3_stack_forward(wts.model, dev(img), dev(cond), dev(t), L.flux3_rope_table(ids), sig, 0.0, vi, sws)
        outs.append(f64(vi))
    torch.cuda.synchronize()
    # (rounding differs only through accumulation order, e.g. split-K choices
    # that depend on the row count; guidance amplifies it 3.5 times)
    assert_agree(f64(v), outs[0] + g * (outs[1] - outs[0]), "cfg pack vs two separate calls")
    # guidance 1: the prompt's velocity alone
    L.flux3_stack_forward_cfg(wts.model, dev(img), dev(cond), dev(txt0), dev(txt1), table, sig, 0.0, 1.0, v, ws)
    torch.cuda.synchronize()
    assert_agree(f64(v), v1, "cfg pack guidance 1 vs oracle prompt velocity")


def test_sample_cfg(L):
    """The guided sampler in one call: bit-identical to step-by-step guided
    stack calls + Euler updates, and within tolerance of the oracle's
    base-checkpoint sampler (3 steps of the shifted schedule)."""
    lay = syn.Layout(4, 4, 80)
    n_txt1 = 240
    seed = 340
    steps, g = 3, 3.5
    wts, img, cond, txt0, txt1, table = _cfg_case(L, seed, lay, n_txt1)
    sig = L.flux3_sigmas(steps)
    say(f"sample cfg n_img={lay.n_img} texts {lay.n_txt}/{n_txt1} steps={steps}")
    ws = L.workspace(L.flux3_sample_cfg_workspace_size(lay.n_img, 0, lay.n_txt, n_txt1))
    x = dev(img).float()
    L.flux3_sample_cfg(wts.model, x, None, dev(txt0), dev(txt1), table, sig, g, ws)
    xs, xb = dev(img).float(), dev(img)
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    cws = L.workspace(L.flux3_stack_cfg_workspace_size(lay.n_img, 0, lay.n_txt, n_txt1))
    sl = sig.tolist()
    for k in range(steps):
        L.flux3_stack_forward_cfg(wts.model, xb, None, dev(txt0), dev(txt1), table, sl[k], sl[k + 1], g, v, cws)
        L.flux3_euler_step(xs, xb, v, sl[k], sl[k + 1])
    torch.cuda.synchronize()
    assert torch.equal(x, xs), "flux3_sample_cfg differs from the step-by-step loop"
    xr = O.sample_base_cfg(_oracle_velocity(wts, lay, None, [txt0, txt1], 1, 1), f64(img), steps, g)
    assert_agree(f64(x), xr, f"cfg sampler {steps} steps")


def test_stack_fp8r(L):
    """The whole transformer (reduced depth, real widths, references) with
    fp8r blocks against the oracle's stack with fp8r blocks."""
    from gpu_util import FP8_REL_MAX
    lay = syn.Layout(6, 6, 40, [(4, 5)])
    seed = 350
    say(f"stack fp8r n={lay.n_total} depth 1+2")
    wts = Weights(L, seed, lay, 1, 2, fp8=True)
    img, cond, txt = _inputs(lay, seed)
    sig, sig_next = np.float32(0.8739), np.float32(0.6979)
    v = _gpu_stack(L, wts, lay, img, cond, txt, float(sig), float(sig_next))
    args = (wts.W, wts.B, f64(img), f64(cond), f64(txt), lay.img_h, lay.img_w, lay.refs,
            float(sig), float(sig_next), 1, 2)
    ref = O.stack_forward(*args, block=O.block_forward_fp8r)
    plain = O.stack_forward(*args)
    from gpu_util import agreement
    c_gpu, r_gpu = agreement(f64(v), ref)
    c_q, r_q = agreement(ref, plain)
    say(f"  stack fp8r: gpu vs oracle fp8r cos={c_gpu:.7f} rel={r_gpu:.3e}; "
        f"oracle fp8r vs oracle unquantized cos={c_q:.7f} rel={r_q:.3e}")
    # The kernel and the oracle quantize activations computed in different
    # precision, so their FP8 codes differ at rounding boundaries and the
    # differences compound through the blocks: the GPU result must be closer
    # to the oracle's fp8r result than FP8 quantization itself moves it.
    assert 1 - c_gpu <= 1 - c_q and r_gpu <= r_q, (c_gpu, r_gpu, c_q, r_q)
    assert_agree(f64(v), ref, "stack fp8r", cos_min=0.999, rel_max=FP8_REL_MAX)


@pytest.mark.parametrize("n,qk_kernel", [(200, True), (300, False)])
def test_launch_timer_block_kinds(L, n, qk_kernel):
    """Which kernels a bf16 block launches, as the launch timer sees them: at
    129..256 rows the QK norm + RoPE is a kernel of its own; above 256 rows
    the in-projection applies it in its epilogue, so the block records
    LayerNorm, in-projection, attention and output projection only."""
    from gpu_util import upload
    lay = syn.Layout(10, 10, n - 100)
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt)
    segs = [0, lay.n_img, n]
    blk = L.PackedBlock(upload(syn.block_weights(72, "single_blocks.0")))
    x = dev(syn.block_activations(73, n)).float()
    mods = dev(syn.normal_f32((2, 3, 3072), 0.5, 74, "mods"))
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    ws = L.workspace(L.flux3_block_workspace_size(n))
    say(f"launch timer: block n={n}")
    L.flux3_timer_start(list(L.TIMER_KINDS), 16)
    L.flux3_block_forward(x, segs, mods, blk, table, ws)
    recs = L.flux3_timer_stop(16)
    expect = ["ln_modulate", "in_proj"] + (["qk_norm_rope"] if qk_kernel else []) + ["attention", "out_proj"]
    assert [k for k, _, _ in recs] == expect
    assert all(r == n and ms > 0 for _, r, ms in recs)


def test_launch_timer(L):
    """The launch timer records the block's five kernels in every block call of
    a stack step, with the call's rows, on the stream each runs on (the text
    stream's stage-1 block on the side stream), and leaves the results
    unchanged; it stops at its capacity and records nothing under graph
    capture."""
    lay = syn.Layout(8, 12, 40)  # 96 image + 40 text rows
    seed = 71
    say("launch timer: stack 96 + 40 rows, depth 1+2")
    wts = Weights(L, seed, lay, 1, 2)
    img, _, txt = _inputs(lay, seed)
    img_d, txt_d = dev(img), dev(txt)
    table = L.flux3_rope_table(L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt).to("cuda"))
    ws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, 0, lay.n_txt))
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")

    def run():
        L.flux3_stack_forward(wts.model, img_d, None, txt_d, table, 0.7, 0.5, v, ws)

    run()
    torch.cuda.synchronize()
    plain = v.clone()
    kinds = list(L.TIMER_KINDS)
    L.flux3_timer_start(kinds, 64)
    run()
    recs = L.flux3_timer_stop(64)
    assert torch.equal(v, plain), "the timer changed the result"
    order = ["ln_modulate", "in_proj", "qk_norm_rope", "attention", "out_proj"]
    # at most 128 rows the in-projection applies the QK norm itself
    fused = [k for k in order if k != "qk_norm_rope"]
    # stage 1: the image block (96 rows) and the text block (40 rows, side
    # stream); stage 2: two joint blocks (136 rows)
    expect = [(k, r) for r in (96, 40) for k in fused] + [(k, 136) for _ in range(2) for k in order]
    assert sorted((k, r) for k, r, _ in recs) == sorted(expect)
    assert [k for k, r, _ in recs if r != 40] == fused + order * 2
    assert [k for k, r, _ in recs if r == 40] == fused
    assert all(ms > 0 for _, _, ms in recs)
    say("launch timer: capacity")
    L.flux3_timer_start(["in_proj", "attention"], 3)
    run()
    recs = L.flux3_timer_stop(3)
    assert [(k, r) for k, r, _ in recs] == [("in_proj", 96), ("attention", 96), ("in_proj", 40)]
    say("launch timer: graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    L.flux3_timer_start(kinds, 64)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    assert L.flux3_timer_stop(64) == []
    v.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(v, plain), "the captured step differs from the eager one"
