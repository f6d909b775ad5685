"""Write the oracle's velocity for the transformer workloads that are too slow
to recompute inside a GPU test.

    python tests/golden/make_stack_golden.py [case ...]

Calls only the oracle (oracle/) and the seeded input generators
(flux3_synth/).  For each case it draws the weights and inputs from their
seeds, runs oracle.stack_forward (float64 throughout) and stores v
[n_img, 128] as float32 in tests/golden/<case>.npy, plus the case's
description, a fingerprint of its inputs and the file's SHA-256 in
tests/golden/stack_golden.json.  The GPU tests regenerate the same inputs
from the same seeds, check the fingerprint, run the library and compare
every row of v with the stored one.

Cases (layouts from flux3_synth.WORKLOADS):
  stack_t2i_1024_4608tok_5+28   1024^2 text-to-image, all 5 + 28 blocks
  stack_4ref_1024_20992tok_5+28 four 1024^2 references (20,992 tokens), all 5 + 28 blocks
  stack_i2i_1024_8704tok_1+1    1024^2 image-to-image, one 1024^2 reference
  stack_4ref_1024_20992tok_1+1  four 1024^2 references (20,992 tokens)
  stack_t2i_1024_4608tok_fp8r_1+1  the rowwise-FP8 transformer at 1024^2
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import flux3_synth as syn  # noqa: E402
import oracle as O  # noqa: E402

META = os.path.join(HERE, "stack_golden.json")

# sigma pairs are float32 values of the 16-step shifted schedule, as the
# library receives them
_S16 = O.sigmas(16)


def _f32(x: float) -> float:
    return float(np.float32(x))


CASES = {
    "stack_t2i_1024_4608tok_5+28": dict(layout="stack_t2i_1024_4608tok", seed=7, n_early=5,
                                        n_single=28, sigma=_f32(_S16[3]), sigma_next=_f32(_S16[4]),
                                        block="bf16"),
    "stack_4ref_1024_20992tok_5+28": dict(layout="stack_4ref_1024_20992tok", seed=7, n_early=5,
                                          n_single=28, sigma=_f32(_S16[2]), sigma_next=_f32(_S16[3]),
                                          block="bf16"),
    "stack_i2i_1024_8704tok_1+1": dict(layout="block_i2i_1024_8704tok", seed=23, n_early=1,
                                       n_single=1, sigma=_f32(_S16[8]), sigma_next=_f32(_S16[9]),
                                       block="bf16"),
    "stack_4ref_1024_20992tok_1+1": dict(layout="stack_4ref_1024_20992tok", seed=29, n_early=1,
                                         n_single=1, sigma=_f32(_S16[0]), sigma_next=_f32(_S16[1]),
                                         block="bf16"),
    "stack_t2i_1024_4608tok_fp8r_1+1": dict(layout="stack_t2i_1024_4608tok", seed=31, n_early=1,
                                            n_single=1, sigma=_f32(_S16[5]), sigma_next=_f32(_S16[6]),
                                            block="fp8r"),
}


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def fingerprint(case: dict) -> dict:
    """Sums of the case's inputs and of its last block's mlp_out, to catch a
    change in the seeded generators."""
    lay = syn.WORKLOADS[case["layout"]]
    img, cond, txt = syn.stack_inputs(lay, case["seed"])
    last = f"single_blocks.{case['n_single'] - 1}"
    fp = {"img": float(_f64(img).sum()), "txt": float(_f64(txt).sum()),
          last + ".mlp_out": float(_f64(syn.block_weights(case["seed"], last)["mlp_out"]).sum())}
    if cond is not None:
        fp["cond"] = float(_f64(cond).sum())
    return fp


def run_case(name: str) -> np.ndarray:
    case = CASES[name]
    lay = syn.WORKLOADS[case["layout"]]
    seed = case["seed"]
    cache = {}

    def W(k):
        if k not in cache:
            cache[k] = _f64(syn.global_weight(seed, k))
        return cache[k]

    def B(prefix):
        return {k: _f64(v) for k, v in syn.block_weights(seed, prefix).items()}

    img, cond, txt = syn.stack_inputs(lay, seed)
    block = O.block_forward_fp8r if case["block"] == "fp8r" else O.block_forward
    return O.stack_forward(W, B, _f64(img), None if cond is None else _f64(cond), _f64(txt),
                           lay.img_h, lay.img_w, lay.refs, case["sigma"], case["sigma_next"],
                           case["n_early"], case["n_single"], block=block)


def main(argv):
    names = argv or list(CASES)
    meta = json.load(open(META)) if os.path.exists(META) else {}
    for name in names:
        t0 = time.time()
        print(f"{name}: oracle ...", flush=True)
        v = run_case(name).astype(np.float32)
        fname = name + ".npy"
        path = os.path.join(HERE, fname)
        np.save(path, v)
        meta[name] = dict(CASES[name], file=fname, shape=list(v.shape),
                          sha256=hashlib.sha256(open(path, "rb").read()).hexdigest(),
                          fingerprint=fingerprint(CASES[name]),
                          command=f"python tests/golden/make_stack_golden.py {name}")
        with open(META, "w") as f:
            json.dump(meta, f, indent=1, sort_keys=True)
            f.write("\n")
        print(f"{name}: done in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
