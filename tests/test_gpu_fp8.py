"""GPU parity of the fp8r path (rowwise FP8, OCP E4M3) against the oracle:
row quantization bit for bit, fp8 products, and the block with fp8
projections ("Welcome FLUX.3 Image Klein in Diffusers", §Base model and
quantized variants: fp8r)."""
import numpy as np
import pytest
import torch

import flux3_synth as syn
import oracle as O
from gpu_util import FP8_REL_MAX, assert_agree, dev, f64, require_gpu, say, to_f64, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    return require_gpu()


@pytest.mark.parametrize("rows,cols", [(7, 264), (33, 3072), (5, 12288), (9, 2048), (3, 16384)])
def test_quantize_rows_bit_exact(L, rows, cols):
    """Codes and scales equal the oracle's (both decide in fp32), incl. a
    zero row and rows of very different magnitudes; widths of both the
    register (multiples of 2048) and the two-pass kernel."""
    g = torch.Generator().manual_seed(rows * cols)
    x = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-10, 10, (rows, 1), generator=g).float())
    x[min(3, rows - 1)] = 0
    xb = x.to(torch.bfloat16)
    say(f"quantize rows {rows}x{cols}")
    q, s = L.flux3_quantize_rows_fp8(dev(xb))
    torch.cuda.synchronize()
    codes, scale, _ = O.quantize_rows_fp8(xb.float().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), codes)
    np.testing.assert_array_equal(s.cpu().numpy(), scale)


def test_pack_block_fp8_bit_exact(L):
    """flux3_pack_block_fp8 (through PackedBlock(fp8=True)): the codes and
    row scales of the packed w_in equal the oracle's rowwise quantization of
    its bf16 rows, and those of w_out equal the quantization of attn_out and
    mlp_out as two tensors ("[Feature] FLUX.3 Image Klein support #2142",
    Tensor names), with the ratio of their row scales (sampled rows)."""
    w = syn.block_weights(78, "single_blocks.0")
    wd = {k: dev(v) for k, v in w.items()}
    w_in, w_out = L.flux3_pack_block(wd)
    blk = L.PackedBlock(wd, fp8=True)
    torch.cuda.synchronize()
    w_in8, s_in, w_out8, s_out = (t.cpu() for t in blk.fp8)
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(w_in.shape[0], 48, replace=False))
    codes, scale, _ = O.quantize_rows_fp8(w_in[rows].float().cpu().numpy())
    np.testing.assert_array_equal(w_in8[rows].numpy(), codes, err_msg="w_in")
    np.testing.assert_array_equal(s_in[rows].numpy(), scale, err_msg="w_in")
    rows = np.sort(rng.choice(w_out.shape[0], 48, replace=False))
    s_out = s_out.view(3, -1).numpy()
    scales = []
    for part, (c0, c1), name in [(0, (0, 3072), "attn_out"), (1, (3072, 12288), "mlp_out")]:
        src = w[name][rows].float().numpy()
        np.testing.assert_array_equal(w_out[rows, c0:c1].float().cpu().numpy(), src, err_msg=name)
        codes, scale, _ = O.quantize_rows_fp8(src)
        np.testing.assert_array_equal(w_out8[rows, c0:c1].numpy(), codes, err_msg=name)
        np.testing.assert_array_equal(s_out[part, rows], scale, err_msg=name)
        scales.append(scale)
    np.testing.assert_array_equal(s_out[2, rows], scales[0] / scales[1])


@pytest.mark.parametrize("m,n,k", [(300, 512, 3072), (513, 256, 256), (64, 27648, 3072), (130, 3072, 12288),
                                   (600, 27648, 3072)])
def test_linear_fp8(L, m, n, k):
    """fp8 products of quantized operands against the exact product of the
    oracle's dequantized operands (fp32 accumulation: tight bound), fp32 and
    bf16 outputs; several tiles, a ragged last tile row, and (600 x 27648)
    more tiles than workgroups, so workgroups move between full and ragged
    tiles."""
    g = torch.Generator().manual_seed(m + n + k)
    a = (torch.randn(m, k, generator=g)).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    say(f"linear fp8 m={m} n={n} k={k}")
    qa, sa = L.flux3_quantize_rows_fp8(dev(a))
    qw, sw = L.flux3_quantize_rows_fp8(dev(w))
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    L.flux3_linear_fp8(qa, sa, qw, sw, y_f32=y)
    yb = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    L.flux3_linear_fp8(qa, sa, qw, sw, y=yb)
    torch.cuda.synchronize()
    ref = O.fp8r_linear(a.float().numpy(), w.float().numpy())
    assert_agree(f64(y), ref, "linear fp8 f32", cos_min=0.999999, rel_max=1e-4)
    assert_agree(f64(yb), ref, "linear fp8 bf16", cos_min=0.99999, rel_max=1e-2)


def _fp8_block_case(L, n, seed, segs):
    w = syn.block_weights(seed, "single_blocks.0")
    x = syn.block_activations(seed + 1, n)
    mods = syn.normal_f32((len(segs) - 1, 3, 3072), 0.5, seed + 2, "mods")
    blk = L.PackedBlock(upload(w), fp8=True)
    return w, x, mods, blk


@pytest.mark.parametrize("n,cuts", [(96, [64]), (300, [200, 260]), (600, []), (1300, [1000])])
def test_block_fp8(L, n, cuts):
    """The block with fp8r projections against the oracle's fp8r block
    (its activation codes come from float64 LayerNorm values, so a few codes
    may differ by one step from the kernel's fp32 ones).  The output
    projection's two Linears: 96 and 300 rows split K into ranges that each
    lie in one Linear; 1300 rows into three ranges, the first spanning both
    (rescaled at column 3072); 600 rows unsplit (rescaled at 3072)."""
    segs = [0] + cuts + [n]
    seed = 700 + n
    w, x, mods, blk = _fp8_block_case(L, n, seed, segs)
    ids = O.build_ids(1, n - 40, 40) if n > 40 else O.build_ids(1, n, 0)
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    xd = dev(x).float()
    ws = L.workspace(L.flux3_block_workspace_size(n))
    say(f"block fp8 n={n} segments {segs}")
    L.flux3_block_forward(xd, segs, dev(mods), blk, table, ws)
    torch.cuda.synchronize()
    ref = O.block_forward_fp8r(f64(x), list(zip(segs[:-1], segs[1:])), f64(mods), to_f64(w), ids)
    got = f64(xd)
    assert_agree(got, ref, f"block fp8 n={n}", rel_max=FP8_REL_MAX)
    assert_agree(got - f64(x), ref - f64(x), f"block fp8 n={n} update", cos_min=0.999, rel_max=5e-2)


@pytest.mark.timeout(600)
def test_block_fp8_full_size_sampled(L):
    """The fp8 block at 4608 tokens (1024^2 t2i, the bench's launch
    configuration) on sampled rows."""
    lay = syn.WORKLOADS["block_t2i_1024_4608tok"]
    n = lay.n_total
    segs = [0] + [b for _, _, b in lay.segments()]
    seed = 760
    w, x, mods, blk = _fp8_block_case(L, n, seed, segs)
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    xd = dev(x).float()
    ws = L.workspace(L.flux3_block_workspace_size(n))
    say(f"block fp8 full size n={n}")
    L.flux3_block_forward(xd, segs, dev(mods), blk, table, ws)
    torch.cuda.synchronize()
    rows = np.array(sorted(set([0, 1, 4095, 4096, 4607] + np.random.default_rng(0).choice(n, 40, replace=False).tolist())))
    ref = O.block_forward_fp8r(f64(x), list(zip(segs[:-1], segs[1:])), f64(mods), to_f64(w), ids, rows=rows)
    got = f64(xd)[rows]
    assert_agree(got, ref, "block fp8 4608 sampled rows", rel_max=FP8_REL_MAX)
    assert_agree(got - f64(x)[rows], ref - f64(x)[rows], "block fp8 4608 update", cos_min=0.999, rel_max=5e-2)
