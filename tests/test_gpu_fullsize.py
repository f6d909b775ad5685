"""Block parity at the workloads' full sizes, in the launch configuration the
bench times (flux3_block_forward on all rows), checked on sampled output rows
that the oracle computes one by one (keys and values from every row).

Workloads: 1024^2 text-to-image (64x64 image + 512 text = 4608 tokens),
1024^2 image-to-image with one reference (8704 tokens), four references
(20992 tokens), and the four bars of the blog's tokens-per-call chart
(4256, 8272, 4336 tokens, and 8800 with the non-square 85x48 grid): text
lengths that are multiples of 80 and row counts with ragged tiles; and the
longest sequence the pages allow (ten references, 4080 text tokens: 49,136)."""
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


def _sample_rows(lay, k=40, seed=0):
    rng = np.random.default_rng(seed)
    edges = []
    for _, a, b in lay.segments():
        edges += [a, a + 1, b - 2, b - 1]
    rows = set(edges) | set(rng.choice(lay.n_total, size=k, replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["block_t2i_1024_4608tok", "block_i2i_1024_8704tok", "stack_4ref_1024_20992tok"]
                         + list(syn.PAGE_WORKLOADS) + list(syn.LONG_WORKLOADS))
def test_block_full_size_sampled(L, name):
    lay = syn.WORKLOADS.get(name) or syn.PAGE_WORKLOADS.get(name) or syn.LONG_WORKLOADS[name]
    n = lay.n_total
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    segs = [0] + [b for _, _, b in lay.segments()]
    seed = 500 + len(segs)
    w = syn.block_weights(seed, "single_blocks.0")
    x = syn.block_activations(seed + 1, n)
    mods = syn.normal_f32((len(segs) - 1, 3, 3072), 0.5, seed + 2, "mods")
    say(f"block full size {name} n={n}")
    blk = L.PackedBlock(upload(w))
    table = L.flux3_rope_table(dev(torch.tensor(ids, dtype=torch.float32)))
    xd = dev(x).float()     # fp32 residual stream holding the bf16 draw
    ws = L.workspace(L.flux3_block_workspace_size(n))
    L.flux3_block_forward(xd, segs, dev(mods), blk, table, ws)
    torch.cuda.synchronize()
    got = f64(xd)
    del ws, xd
    rows = _sample_rows(lay)
    say(f"  oracle on {len(rows)} rows")
    ref = O.block_forward(f64(x), list(zip(segs[:-1], segs[1:])), f64(mods), to_f64(w), ids, rows=rows)
    assert_agree(got[rows], ref, f"{name} sampled rows")
    assert_agree(got[rows] - f64(x)[rows], ref - f64(x)[rows], f"{name} update", cos_min=0.999, rel_max=5e-2)
    # every row is finite and the rows not sampled changed too (the block ran on all rows)
    assert np.isfinite(got).all()
    assert (np.abs(got - f64(x)).max(axis=1) > 0).mean() > 0.99
