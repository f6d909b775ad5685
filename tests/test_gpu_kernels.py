"""GPU parity of each entry point against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and a ragged tail.

Inputs come from flux3_synth (seeded, bf16); both sides read the same values.
All calls go through the C ABI (latent_flow_matching_flux3_amd)."""
import math

import numpy as np
import pytest
import torch

import flux3_synth as syn
import oracle as O
from gpu_util import assert_agree, dev, f64, require_gpu, say, to_f64, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    return require_gpu()


# ---- a1: ids and rope table ------------------------------------------------------

@pytest.mark.parametrize("lay", [(8, 8, 32, []), (64, 64, 512, [(64, 64)]), (3, 5, 7, [(2, 2), (4, 1)]),
                                 (48, 85, 640, [(48, 85)])])
def test_ids_bit_exact_and_rope_table(L, lay):
    h, w, nt, refs = lay
    ids = L.flux3_build_ids(h, w, nt, refs)
    ref = O.build_ids(h, w, nt, refs)
    np.testing.assert_array_equal(ids.numpy().astype(np.float64), ref)   # bit-exact
    say(f"rope_table n={len(ids)}")
    tab = L.flux3_rope_table(dev(ids))
    torch.cuda.synchronize()
    ang = O.rope_angles(ref).reshape(len(ref), 64)
    expect = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    got = tab.cpu().numpy()
    # <= 2 ulp of fp32 (values are in [-1, 1])
    assert np.max(np.abs(got - expect)) <= 2 * 2.0 ** -24 * 1.0 + 1e-12


# ---- GEMMs -------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (37, 128, 192), (300, 256, 320), (130, 3072, 128),
                                   (1030, 13312, 128), (513, 27648, 64), (96, 3072, 12288),
                                   (128, 27648, 3072), (65, 384, 4096)])
def test_linear(L, m, n, k):
    x = syn.normal_bf16((m, k), 1.0, 11, f"lin.x.{m}.{k}")
    w = syn.normal_bf16((n, k), 0.02, 12, f"lin.w.{n}.{k}")
    say(f"linear m={m} n={n} k={k}")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    L.flux3_linear(dev(x), dev(w), y=y)
    yf = torch.empty((m, n), dtype=torch.float32, device="cuda")
    L.flux3_linear(dev(x), dev(w), y_f32=yf)
    torch.cuda.synchronize()
    ref = f64(x) @ f64(w).T
    assert_agree(f64(y), ref, "linear bf16")
    # fp32 output: only fp32 accumulation-order error
    np.testing.assert_allclose(f64(yf), ref, rtol=1e-4, atol=1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("m,n,k", [(520, 22528, 8192)])
def test_linear_long_k_sampled_columns(L, m, n, k):
    # The persistent ring kernel with the deep (5-slice) ring used for long
    # products: 264 tiles (more than one per CU), a ragged last tile row.
    # Reference on 192 sampled output columns.
    x = syn.normal_bf16((m, k), 1.0, 13, f"lin.x.{m}.{k}")
    w = syn.normal_bf16((n, k), 0.02, 14, f"lin.w.{n}.{k}")
    say(f"linear long-k m={m} n={n} k={k}")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    L.flux3_linear(dev(x), dev(w), y=y)
    yf = torch.empty((m, n), dtype=torch.float32, device="cuda")
    L.flux3_linear(dev(x), dev(w), y_f32=yf)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(5).choice(n, 192, replace=False))
    ref = f64(x) @ f64(w[cols]).T
    assert_agree(f64(y)[:, cols], ref, "linear long-k bf16")
    np.testing.assert_allclose(f64(yf)[:, cols], ref, rtol=1e-4, atol=1e-4 * np.abs(ref).max())


# ---- a2: modulation ----------------------------------------------------------------

def test_modulate(L):
    vec = syn.cond_vectors(21, 3)
    lins = [syn.global_weight(22, f"single_stream_modulations.{m}.lin.weight") for m in syn.MODES]
    say("modulate")
    mod = L.flux3_modulate(dev(vec), [dev(w) for w in lins])
    torch.cuda.synchronize()
    for i in range(3):
        ref = O.modulation(f64(vec[i]), f64(lins[i]))
        assert_agree(f64(mod[i]), ref, f"modulate seg {i}", cos_min=0.99999, rel_max=1e-4)


# ---- a3: LayerNorm + modulation --------------------------------------------------------

@pytest.mark.parametrize("n,segs", [(1, [0, 1]), (7, [0, 3, 7]), (300, [0, 128, 200, 300])])
def test_ln_modulate(L, n, segs):
    x = syn.normal_f32((n, 3072), 2.0, 31, f"ln.x.{n}") + 0.5     # fp32 residual stream
    nseg = len(segs) - 1
    mod = syn.normal_f32((nseg, 3, 3072), 0.5, 32, "ln.mod")
    out = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    say(f"ln_modulate n={n}")
    L.flux3_ln_modulate(dev(x), out, segs, dev(mod))
    torch.cuda.synchronize()
    xm = O.layer_norm(f64(x))
    ref = np.empty_like(xm)
    for s in range(nseg):
        a, b = segs[s], segs[s + 1]
        ref[a:b] = O.modulate(xm[a:b], f64(mod[s, 0]), f64(mod[s, 1]))
    assert_agree(f64(out), ref, "ln_modulate")
    # per element: bf16 rounding of the output plus fp32 statistics
    np.testing.assert_allclose(f64(out), ref, rtol=2 ** -7, atol=1e-2)


def test_ln_modulate_scale_minus_one_gives_shift(L):
    n = 5
    x = syn.normal_f32((n, 3072), 1.0, 33, "ln.x2")
    mod = torch.zeros((1, 3, 3072))
    mod[0, 0] = syn.normal_f32((3072,), 1.0, 34, "ln.shift")
    mod[0, 1] = -1.0
    out = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    L.flux3_ln_modulate(dev(x), out, [0, n], dev(mod))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(out), np.broadcast_to(f64(mod[0, 0].to(torch.bfloat16)), (n, 3072)))


# ---- a6: QK RMSNorm + RoPE ---------------------------------------------------------------

@pytest.mark.parametrize("lay", [(2, 3, 5, []), (8, 8, 32, [(4, 4)])])
def test_qk_norm_rope(L, lay):
    h, w, nt, refs = lay
    ids = O.build_ids(h, w, nt, refs)
    n = len(ids)
    qkv = syn.normal_bf16((n, 9216), 1.5, 41, f"qkv.{n}")
    sq = syn.uniform_bf16((128,), 0.5, 1.5, 42, "sq")
    sk = syn.uniform_bf16((128,), 0.5, 1.5, 43, "sk")
    d = dev(qkv)
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    say(f"qk_norm_rope n={n}")
    L.flux3_qk_norm_rope(d[:, :3072], d[:, 3072:6144], dev(sq), dev(sk), table)
    torch.cuda.synchronize()
    q = f64(qkv[:, :3072]).reshape(n, 24, 128)
    k = f64(qkv[:, 3072:6144]).reshape(n, 24, 128)
    rq = O.apply_rope(O.rms_norm(q, f64(sq)), ids).reshape(n, 3072)
    rk = O.apply_rope(O.rms_norm(k, f64(sk)), ids).reshape(n, 3072)
    out = f64(d)
    assert_agree(out[:, :3072], rq, "q")
    assert_agree(out[:, 3072:6144], rk, "k")
    np.testing.assert_allclose(out[:, :6144], np.concatenate([rq, rk], 1), rtol=2 ** -7, atol=2e-2)
    np.testing.assert_array_equal(out[:, 6144:], f64(qkv[:, 6144:]))   # v untouched


# ---- a7: attention -------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 64, 130, 300, 513])
def test_attention(L, n):
    qkv = syn.normal_bf16((n, 9216), 1.0, 51, f"att.{n}")
    d = dev(qkv)
    o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    say(f"attention n={n}")
    L.flux3_attention(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o)
    torch.cuda.synchronize()
    q, k, v = (f64(qkv[:, i * 3072:(i + 1) * 3072]).reshape(n, 24, 128) for i in range(3))
    # scale q so the softmax is peaked enough to matter
    ref = O.attention(q, k, v).reshape(n, 3072)
    assert_agree(f64(o), ref, f"attention n={n}")


def test_attention_special_cases(L):
    n = 200
    qkv = syn.normal_bf16((n, 9216), 2.0, 52, "att.sp")
    qkv[:, 6144:] = 1.0                      # V = ones -> O = ones
    d = dev(qkv)
    o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    L.flux3_attention(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(o), 1.0, atol=2 ** -7)
    # one key: O = V of that key
    o1 = torch.empty((1, 3072), dtype=torch.bfloat16, device="cuda")
    d1 = dev(syn.normal_bf16((1, 9216), 1.0, 53, "att.one"))
    L.flux3_attention(d1[:, :3072], d1[:, 3072:6144], d1[:, 6144:], o1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(o1), f64(d1[:, 6144:]))


@pytest.mark.parametrize("n", [2817, 4608, 8272])
def test_attention_balanced_schedule(L, n):
    """flux3_attention_ws: whole rounds of 512 (head, query block) items, then
    the leftover items' key tiles shared out over the workgroups, the parts of
    a cut item merged by the one that finishes last.  2817 rows: 552 items, 40
    leftover in parts of 23 tiles (up to five parts an item; 23 query blocks,
    a ragged one; 89 key tiles, the last one 1 key); 4608 rows: 352 leftover,
    two or three parts; 8272 rows: three whole rounds, then 24 items in up to
    five parts.  Two calls in a row on one workspace (its counters must come
    back to zero), the second with other data; every row against the oracle
    at 2817 rows, three rows of every query block (so every item, cut or not)
    above."""
    ws_bytes = L.flux3_attention_workspace_size(n)
    assert ws_bytes > 0
    ws = L.workspace(ws_bytes)
    if n < 3000:
        rows = np.arange(n)
    else:
        rows = np.array(sorted({min(b + r, n - 1) for b in range(0, n, 128) for r in (0, 77, 127)}))
    for call in range(2):
        qkv = syn.normal_bf16((n, 9216), 1.0 + call, 54 + call, f"att.ws.{n}.{call}")
        d = dev(qkv)
        o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
        say(f"attention_ws n={n} call={call}")
        L.flux3_attention_ws(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o, ws)
        torch.cuda.synchronize()
        q, k, v = (f64(qkv[:, i * 3072:(i + 1) * 3072]).reshape(n, 24, 128) for i in range(3))
        ref = O.attention(q[rows], k, v).reshape(len(rows), 3072)
        assert_agree(f64(o)[rows], ref, f"attention_ws n={n} call={call}")
        # The workspace ends with one int counter per item (256-byte aligned
        # block); the workgroup that merges an item resets its counter, so a
        # launch leaves them all zero: a block's later attention groups (the
        # guided pack's two samples) start from zero without a clearing kernel.
        items = 24 * ((n + 127) // 128)
        cnt = ws[ws_bytes - (items * 4 + 255) // 256 * 256:][:items * 4].view(torch.int32)
        assert int(cnt.abs().sum().item()) == 0, "split counters not reset"


def test_attention_ws_plain_sizes(L):
    """Item counts at or below one round of 512 workgroups, or a whole number
    of rounds, need no workspace: flux3_attention_ws runs the plain schedule."""
    assert L.flux3_attention_workspace_size(2688) == 0      # 21 blocks x 24 heads = 504 items
    assert L.flux3_attention_workspace_size(65536) == 0     # 512 x 24 items: 24 whole rounds
    assert L.flux3_attention_workspace_size(20992) == 0     # 3936 items: 7 whole rounds
    assert L.flux3_attention_workspace_size(2689) > 0
    n = 300
    qkv = syn.normal_bf16((n, 9216), 1.0, 56, "att.ws.plain")
    d = dev(qkv)
    o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    L.flux3_attention_ws(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o, None)
    torch.cuda.synchronize()
    q, k, v = (f64(qkv[:, i * 3072:(i + 1) * 3072]).reshape(n, 24, 128) for i in range(3))
    assert_agree(f64(o), O.attention(q, k, v).reshape(n, 3072), "attention_ws plain")


@pytest.mark.parametrize("n,balanced", [(1030, False), (2817, True)])
def test_attention_rising_scores(L, n, balanced):
    """Scores that rise from key tile to key tile by more than the online
    softmax lets its reference max lag (8 in log2 units), up to |s| ~ 1e3:
    q = a_row e_0 + noise, k = b_key e_0 + noise with b rising along the
    keys, so rows with a = 8 see their max jump past the reference on every
    32-key tile (the output accumulator must be rescaled each time, and a
    missed or inverted rescale overflows or mis-weights), rows with a = -8
    keep their max in the first tile, a = 0.5 rises slowly, a = 0 is flat.
    At 2817 rows the balanced schedule merges parts whose reference maxima
    are hundreds apart."""
    rise = 30.0 if n < 2000 else 11.0          # log2 units per 32-key tile at a = 8
    beta = rise / (32 * 8 * math.log2(math.e) / math.sqrt(128))
    g = torch.Generator().manual_seed(n)
    a = torch.tensor([8.0, -8.0, 0.5, 0.0]).repeat((n + 3) // 4)[:n]
    b = 8.0 + beta * torch.arange(n, dtype=torch.float32)
    q = torch.randn(n, 24, 128, generator=g)
    k = torch.randn(n, 24, 128, generator=g)
    q[:, :, 0] = a[:, None]
    k[:, :, 0] = b[:, None]
    v = torch.randn(n, 24, 128, generator=g)
    qkv = torch.cat([q.reshape(n, 3072), k.reshape(n, 3072), v.reshape(n, 3072)], 1).to(torch.bfloat16)
    qf, kf, vf = (f64(qkv[:, i * 3072:(i + 1) * 3072]).reshape(n, 24, 128) for i in range(3))
    s_max = np.abs(np.einsum("nhd,nhd->nh", qf, kf)).max() / math.sqrt(128) * math.log2(math.e)
    say(f"attention rising scores n={n} balanced={balanced} (|s| up to {s_max:.0f} log2 units)")
    d = dev(qkv)
    o = torch.empty((n, 3072), dtype=torch.bfloat16, device="cuda")
    if balanced:
        ws = L.workspace(L.flux3_attention_workspace_size(n))
        L.flux3_attention_ws(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o, ws)
    else:
        L.flux3_attention(d[:, :3072], d[:, 3072:6144], d[:, 6144:], o)
    torch.cuda.synchronize()
    ref = O.attention(qf, kf, vf).reshape(n, 3072)
    got = f64(o)
    for r0, what in ((0, "a=8"), (1, "a=-8"), (2, "a=0.5"), (3, "a=0")):
        assert_agree(got[r0::4], ref[r0::4], f"attention rising n={n} rows {what}")


# ---- a3..a8: one block ------------------------------------------------------------------------

def _block_inputs(seed, lay, mod_scale=0.5):
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    n = len(ids)
    segs = [0] + [b for _, _, b in lay.segments()]
    w = syn.block_weights(seed, "single_blocks.0")
    x = syn.block_activations(seed + 1, n)
    mods = syn.normal_f32((len(segs) - 1, 3, 3072), mod_scale, seed + 2, "mods")
    return ids, segs, w, x, mods


def _run_block(L, ids, segs, w, x, mods):
    blk = L.PackedBlock(upload(w))
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    xd = dev(x).float()     # the residual stream is fp32 (values from the bf16 draw)
    ws = L.workspace(L.flux3_block_workspace_size(len(ids)))
    L.flux3_block_forward(xd, segs, dev(mods), blk, table, ws)
    torch.cuda.synchronize()
    return xd


# 1, 33, 55, 96 and 128 rows run the skinny in-projection with the QK norm
# in its epilogue (one to four 32-row fragments, ragged), 600 rows the ring
# kernel and the norm kernel.
@pytest.mark.parametrize("lay", [syn.Layout(8, 8, 32), syn.Layout(5, 6, 13, [(3, 4)]),
                                 syn.Layout(16, 20, 88, [(8, 24)]), syn.Layout(1, 1, 0),
                                 syn.Layout(4, 4, 17), syn.Layout(8, 12, 32)])
def test_block_forward(L, lay):
    ids, segs, w, x, mods = _block_inputs(61, lay)
    say(f"block_forward n={len(ids)}")
    got = _run_block(L, ids, segs, w, x, mods)
    segs_t = list(zip(segs[:-1], segs[1:]))
    ref = O.block_forward(f64(x), segs_t, f64(mods), to_f64(w), ids)
    assert_agree(f64(got), ref, f"block n={len(ids)}")
    # the update x_out - x must agree too (it is small next to x)
    assert_agree(f64(got) - f64(x), ref - f64(x), "block update", cos_min=0.999, rel_max=5e-2)


def test_block_zero_gate_is_identity(L):
    lay = syn.Layout(8, 8, 32)
    ids, segs, w, x, mods = _block_inputs(62, lay)
    mods[:, 2] = 0.0
    got = _run_block(L, ids, segs, w, x, mods)
    np.testing.assert_array_equal(f64(got), f64(x))


def test_block_scale_minus_one_is_identity(L):
    lay = syn.Layout(8, 8, 32)
    ids, segs, w, x, mods = _block_inputs(63, lay)
    mods[:, 0] = 0.0
    mods[:, 1] = -1.0
    got = _run_block(L, ids, segs, w, x, mods)
    np.testing.assert_array_equal(f64(got), f64(x))


# ---- a4..a5, a12: the block's two projections through their own entry points -----------------
# Row counts that take each GEMM path: at most 128 rows (the weight-streaming
# kernel), up to a few hundred (register-staged tiles), 1030 (the persistent
# ring kernel, ragged last tile row; checked on sampled columns).

def test_pack_block_layout(L):
    """flux3_pack_block bit for bit: w_in rows q | k | v, then mlp_in with its
    a (first 9216 rows) and b (last 9216) halves interleaved in groups of 32
    rows; w_out = [attn_out | mlp_out] along the input dimension."""
    w = syn.block_weights(77, "single_blocks.0")
    w_in, w_out = L.flux3_pack_block(upload(w))
    torch.cuda.synchronize()
    wi, wo = w_in.cpu(), w_out.cpu()
    assert torch.equal(wi[:9216], torch.cat([w["q_proj"], w["k_proj"], w["v_proj"]]))
    a, b = w["mlp_in"][:9216], w["mlp_in"][9216:]
    inter = torch.stack([a.reshape(288, 32, 3072), b.reshape(288, 32, 3072)], dim=1).reshape(18432, 3072)
    assert torch.equal(wi[9216:], inter)
    assert torch.equal(wo, torch.cat([w["attn_out"], w["mlp_out"]], dim=1))


@pytest.mark.parametrize("m", [1, 33, 96, 128, 129, 300, 1030])
def test_block_in_proj(L, m):
    """q|k|v = xm [Wq; Wk; Wv]^T and h = silu(a) * b with a, b the two halves
    of xm Win^T ([blog] "Inside one block": the projections and the SwiGLU
    MLP all read the modulated row; [issue] "Structure")."""
    w = syn.block_weights(71, "single_blocks.0")
    blk = L.PackedBlock(upload(w))
    xm = syn.normal_bf16((m, 3072), 1.0, 72, f"inproj.x.{m}")
    qkv = torch.empty((m, 3 * 3072), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((m, 9216), dtype=torch.bfloat16, device="cuda")
    say(f"block_in_proj m={m}")
    L.flux3_block_in_proj(dev(xm), blk.w_in, qkv, h)
    torch.cuda.synchronize()
    wf = to_f64(w)
    x = f64(xm)
    if m > 300:  # sampled columns of each output
        cq = np.sort(np.random.default_rng(7).choice(9216, 256, replace=False))
        ch = np.sort(np.random.default_rng(8).choice(9216, 256, replace=False))
    else:
        cq = ch = np.arange(9216)
    wqkv = np.concatenate([wf["q_proj"], wf["k_proj"], wf["v_proj"]])
    assert_agree(f64(qkv)[:, cq], x @ wqkv[cq].T, f"in_proj q|k|v m={m}")
    a = x @ wf["mlp_in"][:9216][ch].T
    b = x @ wf["mlp_in"][9216:][ch].T
    assert_agree(f64(h)[:, ch], O.silu(a) * b, f"in_proj h m={m}")


@pytest.mark.parametrize("m", [1, 96, 128, 300, 1030])
def test_block_out_proj(L, m):
    """x += gate[seg(row)] (o Wo^T + h Wout^T), [o | h] one product with
    K = 12288 ([blog] "Inside one block"; [issue] "Structure": the gated
    residual), with two row segments of different gates."""
    w = syn.block_weights(73, "single_blocks.0")
    blk = L.PackedBlock(upload(w))
    cat = syn.normal_bf16((m, 12288), 1.0, 74, f"outproj.cat.{m}")
    x0 = syn.normal_f32((m, 3072), 1.0, 75, f"outproj.x.{m}")
    mods = syn.normal_f32((2, 3, 3072), 0.5, 76, "outproj.mods")
    segs = [0, m // 3, m] if m > 1 else [0, 1]
    x = dev(x0)
    say(f"block_out_proj m={m}")
    L.flux3_block_out_proj(dev(cat), blk.w_out, x, segs, dev(mods))
    torch.cuda.synchronize()
    wf = to_f64(w)
    c = f64(cat)
    upd = c[:, :3072] @ wf["attn_out"].T + c[:, 3072:] @ wf["mlp_out"].T
    gate = np.empty((m, 3072))
    for si, (lo, hi) in enumerate(zip(segs[:-1], segs[1:])):
        gate[lo:hi] = f64(mods)[si, 2]
    ref = f64(x0) + gate * upd
    # fp32 accumulation of exact bf16 products: only summation-order error
    np.testing.assert_allclose(f64(x), ref, rtol=1e-4, atol=1e-4 * np.abs(gate * upd).max())


# ---- conditioning -------------------------------------------------------------------------------

def test_time_vectors(L):
    W = {k: syn.global_weight(71, k) for k in ("time_in.in_layer.weight", "time_in.out_layer.weight",
                                               "ref_time_in.in_layer.weight", "ref_time_in.out_layer.weight")}
    Wd = {k: dev(v) for k, v in W.items()}
    vec = torch.empty((3, 3072), dtype=torch.float32, device="cuda")
    ws = L.workspace(1 << 20)
    say("time_vectors")
    for sig, sig_next in ((0.9652, 0.93), (1.0, 0.5), (0.1, 0.0)):
        L.flux3_time_vectors(Wd["time_in.in_layer.weight"], Wd["time_in.out_layer.weight"],
                             Wd["ref_time_in.in_layer.weight"], Wd["ref_time_in.out_layer.weight"],
                             sig, sig_next, [1, 0, 0], vec, ws)
        torch.cuda.synchronize()
        ref = O.mode_vectors(lambda k: f64(W[k]), np.float32(sig), np.float32(sig_next),
                             ["image", "image_cond", "txt"])
        for i, m in enumerate(["image", "image_cond", "txt"]):
            assert_agree(f64(vec[i]), ref[m], f"vec {m} sigma={sig}", cos_min=0.99999, rel_max=1e-3)
    # base checkpoint: no ref_time_in
    L.flux3_time_vectors(Wd["time_in.in_layer.weight"], Wd["time_in.out_layer.weight"], None, None,
                         0.5, 0.0, [1], vec, ws)
    torch.cuda.synchronize()
    ref = O.mode_vectors(lambda k: f64(W[k]), 0.5, None, ["image"])["image"]
    assert_agree(f64(vec[0]), ref, "vec base", cos_min=0.99999, rel_max=1e-3)


def test_euler_step(L):
    x = torch.randn(1000, generator=torch.Generator().manual_seed(0))
    v = torch.randn(1000, generator=torch.Generator().manual_seed(1))
    xd, vd = dev(x), dev(v)
    xb = torch.empty(1000, dtype=torch.bfloat16, device="cuda")
    L.flux3_euler_step(xd, xb, vd, 0.9, 0.7)
    torch.cuda.synchronize()
    ref = O.euler_update(f64(x), f64(v), np.float32(0.9), np.float32(0.7))
    np.testing.assert_allclose(f64(xd), ref, rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(f64(xb), f64(xd.cpu().to(torch.bfloat16)))
