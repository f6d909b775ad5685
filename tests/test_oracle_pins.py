"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden/page_facts.json), closed forms at chosen points
(tests/golden/closed_forms.json), invariants, special cases, and library
routines (torch CPU, float64) that define the same operation independently.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import flux3_synth as syn
import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# Page facts
# ----------------------------------------------------------------------------

def test_token_grid_1024():
    g = _load("page_facts.json")["tokens_1024px_image"]
    h, w = O.token_grid(1024, 1024)
    assert [h, w] == g["grid"] and h * w == g["value"]
    assert len(O.build_ids(h, w, 0)) == g["value"]


def test_reference_adds_4096_tokens():
    g = _load("page_facts.json")["reference_adds_tokens"]
    h, w = O.token_grid(1024, 1024)
    base = len(O.build_ids(h, w, 80))
    with_ref = len(O.build_ids(h, w, 80, [(h, w)]))
    assert with_ref - base == g["value"]


def test_tokens_per_call_chart():
    """Every bar of the chart is image tokens (16x16 px each) plus references
    at their own size plus a text length that is a multiple of 80."""
    g = _load("page_facts.json")["tokens_per_call"]
    m = g["text_pad_multiple"]
    for case in g["cases"]:
        h, w = O.token_grid(*case["output_px"])
        refs = [O.token_grid(*r) for r in case["refs_px"]]
        n_img = len(O.build_ids(h, w, 0, refs))
        n_txt = case["total"] - n_img
        assert n_txt > 0 and n_txt % m == 0, case
        assert O.padded_text_len(n_txt) == n_txt
        assert len(O.build_ids(h, w, n_txt, refs)) == case["total"]
    assert O.padded_text_len(1) == 80 and O.padded_text_len(81) == 160


def test_page_workloads_match_the_chart():
    """The seeded page workloads reproduce the chart's four bars exactly."""
    g = _load("page_facts.json")["tokens_per_call"]
    lays = list(syn.PAGE_WORKLOADS.values())
    assert len(lays) == len(g["cases"])
    for lay, case in zip(lays, g["cases"]):
        assert (lay.img_h, lay.img_w) == O.token_grid(*case["output_px"])
        assert lay.refs == [O.token_grid(*r) for r in case["refs_px"]]
        assert lay.n_total == case["total"] and lay.n_txt % g["text_pad_multiple"] == 0


def test_schedule_facts():
    g = _load("page_facts.json")["schedule"]
    s = O.sigmas(g["steps"], g["alpha"])
    assert s[0] == 1.0 and s[-1] == 0.0
    assert np.all(np.diff(s) < 0)
    assert int((s[:-1] > 0.5).sum()) == g["steps_above_half"]
    assert round(float(s[g["step"]]), 2) == g["sigma_at_step_rounded_2dp"]
    # closed form of the threshold: sigma > 1/2  <=>  t > 1/(alpha + 1)
    t = np.linspace(1, 0, g["steps"] + 1)[:-1]
    assert int((t > 1.0 / (g["alpha"] + 1.0)).sum()) == g["steps_above_half"]


def test_checkpoint_parameter_count():
    """The tensor table (names and shapes) reproduces the printed counts.
    Dropping ref_time_in (base checkpoint) or making modulation per block
    would break it."""
    g = _load("page_facts.json")["checkpoint"]
    shapes = syn.all_tensor_shapes(flow_map=True)
    assert len(shapes) == g["n_tensors"]
    n = sum(int(np.prod(s)) for s in shapes.values())
    assert round(n / 1e9, 3) == g["n_params_billions_3dp"]
    base = sum(int(np.prod(s)) for s in syn.all_tensor_shapes(flow_map=False).values())
    assert round(base / 1e9, 3) != g["n_params_billions_3dp"]


# ----------------------------------------------------------------------------
# Positions and RoPE
# ----------------------------------------------------------------------------

def test_ids_table():
    ids = O.build_ids(3, 4, 5, [(2, 2), (1, 3)])
    assert ids.shape == (12 + 4 + 3 + 5, 4)
    assert (ids[:, 0] == 0).all()                        # t axis is 0 everywhere
    assert tuple(ids[4 * 2 + 3]) == (0, 1.0, 1.5, 0)     # image row 2, col 3
    assert tuple(ids[12 + 3]) == (0, 0.5, 0.5, -1)       # ref 0, row 1, col 1
    assert tuple(ids[16 + 2]) == (0, 0.0, 1.0, -2)       # ref 1, row 0, col 2
    assert tuple(ids[19 + 4]) == (0, 0, 0, 4)            # text 4
    # every id is an exact multiple of 1/2
    assert np.all(ids * 2 == np.round(ids * 2))


def _ids_for(entry):
    if entry["token"] == "text":
        ids = O.build_ids(0, 0, entry["index"] + 1)
        return ids[-1:]
    if entry["token"] == "image":
        ids = O.build_ids(entry["row"] + 1, entry["col"] + 1, 0)
        return ids[entry["row"] * (entry["col"] + 1) + entry["col"]][None]
    if entry["token"] == "ref1":
        ids = O.build_ids(1, 1, 0, [(1, 1), (1, 1)])
        return ids[2][None]
    raise AssertionError(entry)


def test_rope_closed_forms():
    for e in _load("closed_forms.json")["rope"]:
        ids = _ids_for(e)
        d0, d1 = e["dims"]
        for vec, expect in (((1.0, 0.0), (math.cos(e["angle_rad"]), math.sin(e["angle_rad"]))),
                            ((0.0, 1.0), (-math.sin(e["angle_rad"]), math.cos(e["angle_rad"])))):
            x = np.zeros((1, 2, 128))
            x[0, :, d0], x[0, :, d1] = vec
            y = O.apply_rope(x, ids)
            np.testing.assert_allclose(y[0, :, d0], expect[0], atol=1e-12)
            np.testing.assert_allclose(y[0, :, d1], expect[1], atol=1e-12)


def test_rope_against_complex_multiplication():
    """Independent formulation: adjacent pairs as complex numbers multiplied
    by exp(i * id * omega), built with torch.polar."""
    rng = np.random.default_rng(0)
    ids = O.build_ids(3, 5, 7, [(2, 3)])
    x = rng.standard_normal((len(ids), 3, 128))
    om = torch.tensor([10000.0 ** (-2.0 * j / 32) for j in range(16)], dtype=torch.float64)
    ang = torch.cat([torch.tensor(ids[:, a:a + 1]) * om[None] for a in range(4)], dim=1)  # [N,64]
    rot = torch.polar(torch.ones_like(ang), ang)
    xc = torch.view_as_complex(torch.tensor(x).reshape(len(ids), 3, 64, 2))
    ref = torch.view_as_real(xc * rot[:, None, :]).reshape(len(ids), 3, 128).numpy()
    np.testing.assert_allclose(O.apply_rope(x, ids), ref, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(1)
    ids = O.build_ids(4, 4, 6, [(4, 4)])
    n = len(ids)
    q = rng.standard_normal((n, 2, 128))
    k = rng.standard_normal((n, 2, 128))
    rq, rk = O.apply_rope(q, ids), O.apply_rope(k, ids)
    # norm preserved
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-12)
    # t axis dims untouched (t = 0); text rotates only l dims; image only h,w dims
    np.testing.assert_array_equal(rq[:, :, :32], q[:, :, :32])
    n_img = 16
    txt = slice(n - 6, n)
    np.testing.assert_array_equal(rq[txt, :, :96], q[txt, :, :96])
    np.testing.assert_array_equal(rq[:n_img, :, 96:], q[:n_img, :, 96:])
    # scores depend only on relative position: shift every id by an integer vector
    shift = np.array([0.0, 3.0, -2.0, 5.0])
    rq2, rk2 = O.apply_rope(q, ids + shift), O.apply_rope(k, ids + shift)
    s1 = np.einsum("nhd,mhd->hnm", rq, rk)
    s2 = np.einsum("nhd,mhd->hnm", rq2, rk2)
    np.testing.assert_allclose(s1, s2, atol=1e-9)


# ----------------------------------------------------------------------------
# Norms, attention
# ----------------------------------------------------------------------------

def test_layer_norm_library_and_properties():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 3072)) * 3 + 1.5
    y = O.layer_norm(x)
    ref = F.layer_norm(torch.tensor(x), (3072,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, atol=1e-10)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(-1), 1, atol=1e-5)
    shift = rng.standard_normal(3072)
    np.testing.assert_array_equal(O.modulate(y, shift, -np.ones(3072)), np.broadcast_to(shift, y.shape))


def test_rms_norm_library():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 24, 128)) * 2
    s = rng.uniform(0.5, 1.5, 128)
    ref = F.rms_norm(torch.tensor(q), (128,), weight=torch.tensor(s), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(q, s), ref, atol=1e-10)


def test_attention_library_and_special_cases():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((37, 3, 128)) for _ in range(3))
    ref = F.scaled_dot_product_attention(*(torch.tensor(t).transpose(0, 1) for t in (q, k, v)))
    np.testing.assert_allclose(O.attention(q, k, v, chunk=8), ref.transpose(0, 1).numpy(), atol=1e-10)
    # V = ones -> ones (softmax rows sum to 1)
    np.testing.assert_allclose(O.attention(q, k, np.ones_like(v)), 1.0, atol=1e-12)
    # one key -> output is that value
    np.testing.assert_allclose(O.attention(q, k[:1], v[:1]), np.broadcast_to(v[:1], q.shape), atol=1e-12)
    # equal keys -> mean of V
    ke = np.broadcast_to(k[:1], k.shape).copy()
    np.testing.assert_allclose(O.attention(q, ke, v), np.broadcast_to(v.mean(0), q.shape), atol=1e-12)


# ----------------------------------------------------------------------------
# Block
# ----------------------------------------------------------------------------

SMALL = dict(n_img_h=4, n_img_w=4, n_txt=8)


def _block_case(seed=0, refs=()):
    lay = syn.Layout(SMALL["n_img_h"], SMALL["n_img_w"], SMALL["n_txt"], list(refs))
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    w = {k: f64(v) for k, v in syn.block_weights(seed, "single_blocks.0").items()}
    x = f64(syn.block_activations(seed + 1, lay.n_total))
    segs = [(a, b) for _, a, b in lay.segments()]
    rng = np.random.default_rng(seed)
    mods = rng.standard_normal((len(segs), 3, 3072)) * 0.5
    return lay, ids, w, x, segs, mods


def _torch_block(x, segs, mods, w, ids):
    """The block written with torch library layers (F.linear is x W^T by
    definition), RoPE as complex multiplication."""
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    x = T(x)
    n = x.shape[0]
    shift = torch.zeros(n, 3072, dtype=torch.float64)
    scale, gate = shift.clone(), shift.clone()
    for i, (a, b) in enumerate(segs):
        shift[a:b], scale[a:b], gate[a:b] = T(mods[i, 0]), T(mods[i, 1]), T(mods[i, 2])
    h = (1 + scale) * F.layer_norm(x, (3072,), eps=1e-6) + shift
    q = F.linear(h, T(w["q_proj"])).view(n, 24, 128)
    k = F.linear(h, T(w["k_proj"])).view(n, 24, 128)
    v = F.linear(h, T(w["v_proj"])).view(n, 24, 128)
    q = F.rms_norm(q, (128,), weight=T(w["norm.query_norm.scale"]), eps=1e-6)
    k = F.rms_norm(k, (128,), weight=T(w["norm.key_norm.scale"]), eps=1e-6)
    om = torch.tensor([10000.0 ** (-2.0 * j / 32) for j in range(16)], dtype=torch.float64)
    ang = torch.cat([T(ids[:, a:a + 1]) * om[None] for a in range(4)], dim=1)
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    q = torch.view_as_real(torch.view_as_complex(q.reshape(n, 24, 64, 2)) * rot).reshape(n, 24, 128)
    k = torch.view_as_real(torch.view_as_complex(k.reshape(n, 24, 64, 2)) * rot).reshape(n, 24, 128)
    att = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
    att = F.linear(att.transpose(0, 1).reshape(n, 3072), T(w["attn_out"]))
    a, b = F.linear(h, T(w["mlp_in"])).chunk(2, dim=-1)
    mlp = F.linear(F.silu(a) * b, T(w["mlp_out"]))
    return (x + gate * (att + mlp)).numpy()


def test_block_against_torch_layers():
    lay, ids, w, x, segs, mods = _block_case(0, refs=[(2, 3)])
    y = O.block_forward(x, segs, mods, w, ids)
    np.testing.assert_allclose(y, _torch_block(x, segs, mods, w, ids), atol=1e-9)


def test_block_rows_subset_matches_full():
    lay, ids, w, x, segs, mods = _block_case(1)
    full = O.block_forward(x, segs, mods, w, ids)
    rows = np.array([0, 5, 17, 23])
    np.testing.assert_allclose(O.block_forward(x, segs, mods, w, ids, rows=rows), full[rows], atol=1e-12)


def test_block_zero_gate_is_identity():
    lay, ids, w, x, segs, mods = _block_case(2)
    mods[:, 2] = 0.0
    np.testing.assert_array_equal(O.block_forward(x, segs, mods, w, ids), x)


def test_block_scale_minus_one_is_identity():
    """scale = -1, shift = 0 -> h = 0 -> q = k = v = 0 and mlp(0) = 0."""
    lay, ids, w, x, segs, mods = _block_case(3)
    mods[:, 0] = 0.0
    mods[:, 1] = -1.0
    np.testing.assert_array_equal(O.block_forward(x, segs, mods, w, ids), x)


def test_block_permutation_equivariance():
    """Permuting tokens together with their ids and modes permutes outputs
    (so the concatenation order of the streams does not matter)."""
    lay, ids, w, x, segs, mods = _block_case(4, refs=[(2, 2)])
    y = O.block_forward(x, segs, mods, w, ids)
    # give every row its own 'segment' so a permutation can carry modulation
    n = len(x)
    row_seg = np.zeros(n, dtype=int)
    for i, (a, b) in enumerate(segs):
        row_seg[a:b] = i
    perm = np.random.default_rng(0).permutation(n)
    mods_rows = mods[row_seg[perm]]
    yp = O.block_forward(x[perm], [(i, i + 1) for i in range(n)], mods_rows, w, ids[perm])
    np.testing.assert_allclose(yp, y[perm], atol=1e-10)


# ----------------------------------------------------------------------------
# Conditioning, final layer, stack, sampler
# ----------------------------------------------------------------------------

def test_timestep_embedding_closed_forms():
    for e in _load("closed_forms.json")["timestep_embedding"]:
        emb = O.timestep_embedding(e["t"])
        assert emb.shape == (256,)
        if e["index"] == "all cos":
            np.testing.assert_array_equal(emb[:128], 1.0)
        elif e["index"] == "all sin":
            np.testing.assert_array_equal(emb[128:], 0.0)
        else:
            fn = math.cos if e["value_fn"] == "cos" else math.sin
            assert abs(emb[e["index"]] - fn(e["arg_rad"])) < 1e-12
    assert np.all(np.abs(O.timestep_embedding(0.37)) <= 1.0)


def _global_W(seed):
    cache = {}

    def W(name):
        if name not in cache:
            cache[name] = f64(syn.global_weight(seed, name))
        return cache[name]
    return W


def test_modulation_and_mode_vectors_against_torch():
    W = _global_W(5)
    vecs = O.mode_vectors(W, 0.7, 0.4, ["image", "txt"])
    T = lambda a: torch.tensor(a, dtype=torch.float64)

    def emb(t):
        f = torch.exp(-math.log(10000) * torch.arange(128, dtype=torch.float64) / 128)
        a = 1000 * t * f
        return torch.cat([torch.cos(a), torch.sin(a)])

    def mlp(e, p):
        return F.linear(F.silu(F.linear(e, T(W(p + ".in_layer.weight")))), T(W(p + ".out_layer.weight")))
    img = mlp(emb(0.7), "time_in") + mlp(emb(0.4), "ref_time_in")
    txt = mlp(emb(0.0), "time_in") + mlp(emb(0.4), "ref_time_in")
    np.testing.assert_allclose(vecs["image"], img.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(vecs["txt"], txt.numpy(), rtol=1e-10, atol=1e-12)
    lin = W("single_stream_modulations.txt.lin.weight")
    shift, scale, gate = F.linear(F.silu(T(vecs["txt"])), T(lin)).chunk(3)
    m = O.modulation(vecs["txt"], lin)
    np.testing.assert_allclose(m, torch.stack([shift, scale, gate]).numpy(), rtol=1e-10, atol=1e-12)
    # base model (no flow map): no ref_time_in term
    base = O.mode_vectors(W, 0.7, None, ["image"])["image"]
    np.testing.assert_allclose(base, mlp(emb(0.7), "time_in").numpy(), rtol=1e-10, atol=1e-12)


def test_final_layer_against_torch():
    W = _global_W(6)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((10, 3072))
    vec = rng.standard_normal(3072)
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    shift, scale = F.linear(F.silu(T(vec)), T(W("final_layer.image.adaLN_modulation.1.weight"))).chunk(2)
    ref = F.linear((1 + scale) * F.layer_norm(T(x), (3072,), eps=1e-6) + shift,
                   T(W("final_layer.image.linear.weight")))
    out = O.final_layer(x, vec, W("final_layer.image.adaLN_modulation.1.weight"),
                        W("final_layer.image.linear.weight"))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-10)


def test_sampler_closed_forms():
    x0 = np.array([2.0, -1.0])
    # constant velocity c: x_S = x_0 + (sigma_S - sigma_0) c = x_0 - c
    c = np.array([0.25, 4.0])
    np.testing.assert_allclose(O.sample_flow_map(lambda x, s, sn: c, x0, 16), x0 - c, atol=1e-12)
    # v = x: product of (1 + dsigma_k)
    s = O.sigmas(16)
    expect = x0 * np.prod(1.0 + np.diff(s))
    np.testing.assert_allclose(O.sample_flow_map(lambda x, a, b: x, x0, 16), expect, rtol=1e-12)
    # the model is called with (sigma_k, sigma_{k+1})
    calls = []
    O.sample_flow_map(lambda x, a, b: calls.append((a, b)) or 0 * x, x0, 4)
    assert calls == [(s4, s5) for s4, s5 in zip(O.sigmas(4)[:-1], O.sigmas(4)[1:])]


def test_base_cfg_sampler_special_cases():
    """Guidance 1 is the conditional sampler alone, guidance 0 the
    unconditional one, equal samples make guidance irrelevant, and linear
    velocities have a product closed form; the model sees sigma_k only."""
    x0 = np.array([1.5, -0.5, 2.0])
    vu = lambda x, s: -x
    vc = lambda x, s: 0.5 * x + 1.0

    def vel(x, s, i):
        return vu(x, s) if i == 0 else vc(x, s)

    def plain(v, steps):  # Euler with one velocity
        sg = O.sigmas(steps)
        x = x0
        for k in range(steps):
            x = x + (sg[k + 1] - sg[k]) * v(x, sg[k])
        return x

    np.testing.assert_allclose(O.sample_base_cfg(vel, x0, 7, 1.0), plain(vc, 7), rtol=1e-12)
    np.testing.assert_allclose(O.sample_base_cfg(vel, x0, 7, 0.0), plain(vu, 7), rtol=1e-12)
    same = lambda x, s, i: vc(x, s)
    np.testing.assert_allclose(O.sample_base_cfg(same, x0, 5, 3.5), O.sample_base_cfg(same, x0, 5, -2.0),
                               rtol=1e-12)
    # guided velocity g*vc + (1-g)*vu = (0.5 g - (1 - g)) x + g: affine steps
    g, steps = 3.5, 50
    sg = O.sigmas(steps)
    a, b = 0.5 * g - (1.0 - g), g
    x = x0.copy()
    for k in range(steps):
        d = sg[k + 1] - sg[k]
        x = (1.0 + d * a) * x + d * b
    np.testing.assert_allclose(O.sample_base_cfg(vel, x0), x, rtol=1e-12)
    calls = []
    O.sample_base_cfg(lambda x, s, i: calls.append((s, i)) or 0 * x, x0, 3)
    assert calls == [(s3, i) for s3 in O.sigmas(3)[:-1] for i in (0, 1)]
    assert O.BASE_STEPS == 50 and O.CFG_GUIDANCE == 3.5


def _stack_case(seed, refs, n_early, n_single):
    lay = syn.Layout(2, 3, 5, list(refs))
    W = _global_W(seed)
    bcache = {}

    def B(prefix):
        if prefix not in bcache:
            bcache[prefix] = {k: f64(v) for k, v in syn.block_weights(seed, prefix).items()}
        return bcache[prefix]
    img = f64(syn.latents(seed, lay.n_img))
    cond = f64(syn.latents(seed, lay.n_cond, "cond")) if lay.n_cond else None
    txt = f64(syn.text_features(seed, lay.n_txt))
    return lay, W, B, img, cond, txt


def test_stage1_streams_are_isolated():
    """Stage 1 attends within a mode only: changing the text leaves the image
    and reference streams unchanged."""
    lay, W, B, img, cond, txt = _stack_case(7, [(1, 2)], 1, 0)
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    _, s1, _ = O.stage1(W, B, img, cond, txt, ids, lay.refs, 0.8, 0.6, 1)
    _, s2, _ = O.stage1(W, B, img, cond, txt + 1.0, ids, lay.refs, 0.8, 0.6, 1)
    np.testing.assert_array_equal(s1[0], s2[0])
    np.testing.assert_array_equal(s1[1], s2[1])
    assert not np.allclose(s1[2], s2[2])


def test_stack_stream_order_does_not_matter():
    """Stage 2 run in the blog's [text | image | reference] order gives the
    same image rows as the order image, image_cond, text."""
    lay, W, B, img, cond, txt = _stack_case(8, [(1, 2)], 1, 1)
    v = O.stack_forward(W, B, img, cond, txt, lay.img_h, lay.img_w, lay.refs, 0.8, 0.6, 1, 1)
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    modes, streams, vecs = O.stage1(W, B, img, cond, txt, ids, lay.refs, 0.8, 0.6, 1)
    order = [2, 0, 1]     # text, image, reference
    segs, start = [], 0
    for i in order:
        segs.append((start, start + len(streams[i])))
        start += len(streams[i])
    x = np.concatenate([streams[i] for i in order])
    starts = np.cumsum([0] + [len(s) for s in streams])
    idp = np.concatenate([ids[starts[i]:starts[i + 1]] for i in order])
    mods = np.stack([O.modulation(vecs[modes[i]], W(f"single_stream_modulations.{modes[i]}.lin.weight"))
                     for i in order])
    x = O.block_forward(x, segs, mods, B("single_blocks.0"), idp)
    x_img = x[segs[1][0]:segs[1][1]]
    v2 = O.final_layer(x_img, vecs["image"], W("final_layer.image.adaLN_modulation.1.weight"),
                       W("final_layer.image.linear.weight"))
    np.testing.assert_allclose(v, v2, atol=1e-10)
    assert v.shape == (lay.n_img, 128)


def test_block_flops_formula():
    # 4 square projections + mlp_in (2F x H) + mlp_out (H x F), plus QK^T and PV
    n = 96
    gemm = 2 * n * (4 * 3072 * 3072 + 2 * 9216 * 3072 + 3072 * 9216)
    att = 2 * 2 * n * n * 3072
    assert O.block_flops(n) == gemm + att


def test_stack_uses_each_modulation_where_the_pages_say():
    """gate = 0 makes a block the identity.  Zeroing the gate third of one
    named modulation must switch off exactly the blocks that the pages tie to
    it: early_stream_modulations.<mode> for that mode's stage-1 blocks,
    single_stream_modulations.* for the joint blocks."""
    lay, W0, B, img, cond, txt = _stack_case(9, [(1, 2)], 1, 1)

    def zero_gate(names):
        def W(name):
            w = W0(name)
            if name in names:
                w = w.copy()
                w[2 * 3072:] = 0.0
            return w
        return W
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    W = zero_gate({"early_stream_modulations.txt.lin.weight"})
    _, s, _ = O.stage1(W, B, img, cond, txt, ids, lay.refs, 0.8, 0.6, 2)
    np.testing.assert_array_equal(s[2], txt @ W0("txt_in.weight").T)
    assert not np.array_equal(s[0], img @ W0("emb_in.image.weight").T)
    names = {f"single_stream_modulations.{m}.lin.weight" for m in ("image", "image_cond", "txt")}
    W = zero_gate(names)
    v = O.stack_forward(W, B, img, cond, txt, lay.img_h, lay.img_w, lay.refs, 0.8, 0.6, 1, 2)
    _, s, vecs = O.stage1(W, B, img, cond, txt, ids, lay.refs, 0.8, 0.6, 1)
    v2 = O.final_layer(s[0], vecs["image"], W("final_layer.image.adaLN_modulation.1.weight"),
                       W("final_layer.image.linear.weight"))
    np.testing.assert_array_equal(v, v2)


def test_longest_sequence():
    """Ten 1024^2 references and the longest padded text: 49,136 tokens; the
    references take l = -1 .. -10."""
    g = _load("page_facts.json")["longest_sequence"]
    lay = syn.LONG_WORKLOADS["stack_10ref_1024_49136tok"]
    h, w = O.token_grid(1024, 1024)
    assert lay.refs == [(h, w)] * g["max_refs"] and (lay.img_h, lay.img_w) == (h, w)
    cap = g["text_max_tokens"] // g["text_pad_multiple"] * g["text_pad_multiple"]
    assert lay.n_txt == cap == O.padded_text_len(cap) and O.padded_text_len(cap + 1) > g["text_max_tokens"]
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    assert len(ids) == lay.n_total == 49136
    l_axis = ids[lay.n_img:lay.n_img + lay.n_cond, 3]
    assert sorted(set(l_axis.tolist())) == [-float(k) for k in range(10, 0, -1)]
    assert (ids[lay.n_img + lay.n_cond:, 3] == range(lay.n_txt)).all()


# ---- fp8r (rowwise FP8, R17) --------------------------------------------------

def test_e4m3_rounding_against_torch():
    """OCP E4M3 rounding (ties to even) agrees code for code with torch's
    float8_e4m3fn conversion over the finite range, including exact ties
    and subnormals."""
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    grid = O.e4m3_value(np.arange(0, 0x7F))                 # every finite non-negative value
    ties = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)  # midpoints (exact in float32)
    x = np.concatenate([x, ties, -ties, grid.astype(np.float32), np.float32([448.0, -448.0, 0.0])])
    codes, vals = O.e4m3_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(codes, ref.view(torch.uint8).numpy())
    np.testing.assert_array_equal(vals, ref.to(torch.float64).numpy())


def test_e4m3_closed_forms():
    cases = {448.0: 0x7E, 2.0 ** -9: 0x01, -1.0: 0xB8, 1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A,
             3 * 2.0 ** -10: 0x02, 2.0 ** -10: 0x00, 240.0: 0x77, 2.0 ** -6: 0x08, 0.875 * 2.0 ** -6: 0x07}
    codes, _ = O.e4m3_round(np.array(list(cases), np.float32))
    assert [int(c) for c in codes] == list(cases.values())
    # every finite code decodes and re-encodes to itself; 0x7F is NaN
    all_codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    back, _ = O.e4m3_round(O.e4m3_value(all_codes).astype(np.float32))
    assert np.array_equal(back[all_codes != 0x80], all_codes[all_codes != 0x80])
    assert np.isnan(O.e4m3_value([0x7F, 0xFF])).all()
    assert O.e4m3_round(np.float32([1e6, -1e6]))[1].tolist() == [448.0, -448.0]   # saturates


def test_rowwise_fp8_quantization_properties():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 300)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32)
    x[5] = 0.0
    codes, scale, deq = O.quantize_rows_fp8(x)
    amax = np.abs(x).max(axis=1)
    hit = np.abs(x) == amax[:, None]
    assert set(codes[hit & (amax[:, None] > 0)].tolist()) <= {0x7E, 0xFE}   # the row max lands on 448
    assert (codes[5] == 0).all() and scale[5] == 1.0 and (deq[5] == 0).all()
    # half a spacing: 2^-4 relative for normals, 2^-10 * scale below 2^-6 * scale
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None].astype(np.float64))
    assert (err <= bound * (1 + 1e-9)).all()


def test_fp8r_linear_exact_on_representable_rows():
    """Rows made of E4M3 values times a power of two, with the row max at
    448 times that power, quantize exactly: the FP8 product equals the exact
    product (catches a misplaced or transposed scale)."""
    rng = np.random.default_rng(2)
    grid = O.e4m3_value(np.arange(1, 0x7F))
    def rows(n, k):
        v = rng.choice(grid, (n, k)) * rng.choice([-1.0, 1.0], (n, k))
        v[:, 0] = 448.0
        return v * np.exp2(rng.integers(-20, 5, (n, 1)))
    a, w = rows(9, 64), rows(13, 64)
    np.testing.assert_allclose(O.fp8r_linear(a, w), a @ w.T, rtol=1e-13)


def test_fp8r_block_structure_matches_block_forward():
    """With the quantizer replaced by the identity, the fp8r block (six
    Linears, each a product of its own) is the plain block, which is pinned to
    torch's layers; with FP8 it stays close."""
    rng = np.random.default_rng(3)
    n = 12
    w = {k: f64(v) for k, v in syn.block_weights(5, "single_blocks.0").items()}
    x = rng.standard_normal((n, O.HIDDEN))
    mods = rng.standard_normal((1, 3, O.HIDDEN)) * 0.3
    ids = O.build_ids(2, 3, 6)
    ident = lambda a: (None, None, np.asarray(a, np.float64))
    ref = O.block_forward(x, [(0, n)], mods, w, ids)
    np.testing.assert_allclose(O.block_forward_fp8r(x, [(0, n)], mods, w, ids, quant=ident), ref,
                               rtol=1e-10, atol=1e-10)
    got = O.block_forward_fp8r(x, [(0, n)], mods, w, ids)
    d, r = got - x, ref - x
    assert float((d * r).sum() / np.linalg.norm(d) / np.linalg.norm(r)) > 0.99


def test_fp8r_block_quantizes_each_linear_on_its_own():
    """A per-tensor rowwise checkpoint holds one scale per row of each of the
    block's tensors ("[Feature] FLUX.3 Image Klein support #2142", Tensor
    names: q_proj, k_proj, v_proj, attn_out [3072, 3072], mlp_in
    [18432, 3072], mlp_out [3072, 9216]): the quantizer must see each weight
    as that tensor and each Linear's own input (h four times, o, swiglu),
    never a concatenation of two of them."""
    rng = np.random.default_rng(4)
    n = 5
    w = {k: f64(v) for k, v in syn.block_weights(6, "single_blocks.0").items()}
    x = rng.standard_normal((n, O.HIDDEN))
    mods = rng.standard_normal((1, 3, O.HIDDEN)) * 0.3
    seen = []

    def spy(a):
        a = np.asarray(a, np.float64)
        seen.append(a)
        return O.quantize_rows_fp8(a)

    O.block_forward_fp8r(x, [(0, n)], mods, w, O.build_ids(1, 2, 3), quant=spy)
    shapes = sorted(a.shape for a in seen)
    want = sorted([(n, O.HIDDEN)] * 5 + [(n, O.MLP_HIDDEN)] +
                  [w[k].shape for k in ("q_proj", "k_proj", "v_proj", "attn_out", "mlp_in", "mlp_out")])
    assert shapes == want
    for k in ("q_proj", "k_proj", "v_proj", "attn_out", "mlp_in", "mlp_out"):
        assert any(a.shape == w[k].shape and np.array_equal(a, w[k]) for a in seen), k


def test_fp8r_output_parts_keep_their_own_scales():
    """attn_out(o) + mlp_out(swiglu) with o and swiglu at very different
    magnitudes: per-Linear rowwise scales keep both products exact on
    E4M3-representable rows, where one scale across [o | swiglu] would round
    the small part away."""
    rng = np.random.default_rng(5)
    grid = O.e4m3_value(np.arange(1, 0x7F))

    def rows(nr, k, lo, hi):
        v = rng.choice(grid, (nr, k)) * rng.choice([-1.0, 1.0], (nr, k))
        v[:, 0] = 448.0
        return v * np.exp2(rng.integers(lo, hi, (nr, 1)))

    o, sw = rows(6, 128, -24, -18), rows(6, 384, 0, 4)
    wo, wm = rows(8, 128, -10, -6), rows(8, 384, -3, 1)
    exact = o @ wo.T + sw @ wm.T
    np.testing.assert_allclose(O.fp8r_linear(o, wo) + O.fp8r_linear(sw, wm), exact, rtol=1e-13)
    fused = O.fp8r_linear(np.concatenate([o, sw], 1), np.concatenate([wo, wm], 1))
    assert np.abs(fused - exact).max() > 1e-3 * np.abs(o @ wo.T).max()


# ---- sampler update ([issue] Sampling: x += (sigma_{k+1} - sigma_k) v) --------

def test_euler_update_closed_forms():
    """On the straight path x(s) = (1 - s) x0 + s x1, whose velocity
    dx/ds = x1 - x0 is constant, the update from sigma to sigma_next lands on
    x(sigma_next) exactly, step after step, and ends on x0 at sigma = 0; a
    zero-length step leaves x unchanged; two steps add up to one."""
    rng = np.random.default_rng(6)
    x0, x1 = rng.standard_normal((2, 7, 128))
    v = x1 - x0
    s = O.sigmas(16)
    x = x1.copy()
    for k in range(16):
        x = O.euler_update(x, v, s[k], s[k + 1])
        np.testing.assert_allclose(x, (1 - s[k + 1]) * x0 + s[k + 1] * x1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(x, x0, rtol=0, atol=1e-12)
    assert np.array_equal(O.euler_update(x1, v, 0.37, 0.37), x1)
    two = O.euler_update(O.euler_update(x1, v, 0.9, 0.6), v, 0.6, 0.2)
    np.testing.assert_allclose(two, O.euler_update(x1, v, 0.9, 0.2), rtol=0, atol=1e-12)
