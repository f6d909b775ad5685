#!/usr/bin/env python3
"""Throughput of the FLUX.3 Image Klein denoiser on one MI355X.

One step = one flow-map sampling step of the whole transformer at the 1024x1024
text-to-image shape: 4096 image tokens + 512 text tokens = 4608 tokens through
embeddings, 5 per-stream blocks, 28 joint blocks, the final layer, then the
sampler update x += (sigma_{k+1} - sigma_k) v.  Weights are seeded random init
(N(0, 0.02) bf16, ~5.5 B parameters), inputs seeded N(0, 1) bf16.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --only KERNEL [--steps K]     # one kernel, for counter runs

Prints one JSON line.  `value` is TFLOP/s of algorithmic work per step; the
dominant kernel's roofline is measured live with HIP events on the stream the
kernels run on.  --only runs a single kernel of the joint block at 4608 tokens
(or the copy used to calibrate the HBM byte counters) K times and prints its
average time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HIDDEN, MLP = 3072, 9216
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "DiT step latency (ms) & TFLOP/s at 1024² (4608 tok); % of MI355X bf16 peak"
COPY_BYTES = 1 << 30           # calibration copy: 1 GiB read + 1 GiB written

# HBM bytes per launch at 4608 rows from rocprofv3 FETCH_SIZE + WRITE_SIZE
# (calibrated against the 1 GiB copy: factors 2.0 and 1.0), with the code
# digests (code_digest) of the sources they were measured on; reported only
# while that code is unchanged.  The in-projection's figure is the mean over
# its 4608-row launches inside stack steps (as its roofline is timed); the
# others are of their kernel alone (--only).
TRAFFIC = {
    "gemm_in_proj_swiglu": (1491.8e6 + 170.2e6, {"gemm_kernels.hpp": "c6587cfc6a48c98d", "gemm.hip": "f10221f408a8d22b",
                                                 "kernels.hpp": "30f6016329aff61f", "common.hpp": "a628a66ce9fdd5dc"}),
    "gemm_out_proj_gated": (751.6e6 + 59.3e6, {"gemm_kernels.hpp": "c6587cfc6a48c98d", "gemm.hip": "f10221f408a8d22b",
                                               "kernels.hpp": "30f6016329aff61f", "common.hpp": "a628a66ce9fdd5dc"}),
    "attention": (357.5e6 + 90.0e6, {"attention.hip": "bbd9a581ae964ab5", "kernels.hpp": "30f6016329aff61f", "common.hpp": "a628a66ce9fdd5dc"}),
}


def code_digest(path: str) -> str:
    """Digest of a source file's code: comments and whitespace removed, so an
    edit of a comment keeps it and any change of the code changes it."""
    import hashlib
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return hashlib.sha256(re.sub(r"\s+", "", text).encode()).hexdigest()[:16]


def measured_traffic(kernel: str):
    """The rocprofv3 bytes of `kernel`, if its sources' code is the code they
    were measured on, else None."""
    if kernel not in TRAFFIC:
        return None
    nbytes, sources = TRAFFIC[kernel]
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "latent_flow_matching_flux3_amd", "csrc")
    for name, digest in sources.items():
        if code_digest(os.path.join(csrc, name)) != digest:
            return None
    return nbytes


def block_flops(n: int) -> float:
    """Six projections (2 N (4 H^2 + 3 H F)) plus QK^T and PV (4 N^2 H)."""
    return 2.0 * n * (4 * HIDDEN * HIDDEN + 3 * HIDDEN * MLP) + 4.0 * n * n * HIDDEN


def stack_flops(n_img: int, n_cond: int, n_txt: int, n_early: int = 5, n_single: int = 28) -> float:
    n_modes = 1 + (n_cond > 0) + (n_txt > 0)
    f = 2.0 * (n_img + n_cond) * 128 * HIDDEN + 2.0 * n_txt * 20480 * HIDDEN       # embeddings
    f += n_early * sum(block_flops(n) for n in (n_img, n_cond, n_txt) if n > 0)   # stage 1
    f += n_single * block_flops(n_img + n_cond + n_txt)                           # stage 2
    f += 2.0 * n_img * HIDDEN * 128                                               # final linear
    f += 2.0 * (HIDDEN * 256 + HIDDEN * HIDDEN) * (n_modes + 1)                   # time MLPs
    f += 2.0 * 3 * HIDDEN * HIDDEN * 2 * n_modes + 2.0 * 2 * HIDDEN * HIDDEN      # modulations
    return f


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the fp8r (rowwise FP8 projections) stack step")
    ap.add_argument("--no-cfg", action="store_true",
                    help="skip the base checkpoint's guided 50-step sampling")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the stack step at the longest sequence (10 references, 49,136 tokens)")
    ap.add_argument("--no-sampler-loop", action="store_true",
                    help="skip the timing of the 16-step loop as one call (eager and graph)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (one block at 96 / 4608 / 8704 tokens, "
                         "the stack step with four references at 20,992 tokens)")
    ap.add_argument("--no-fixtures", action="store_true",
                    help="skip the per-kernel fixture timing (each kernel alone, back to back)")
    ap.add_argument("--no-kernel-timer", action="store_true",
                    help="time the steps without the library's launch timer (the roofline then "
                         "comes from the back-to-back fixtures)")
    ap.add_argument("--probe", action="store_true",
                    help="only the peak probes (register-only bf16 MFMA, HBM copy)")
    ap.add_argument("--only", default=None,
                    help="in_proj | out_proj | attention | ln_modulate | qk_norm_rope | copy | loop_96tok")
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


def make_block(L, torch, rnd):
    import flux3_synth as syn
    w = {k: rnd(shp) for k, shp in syn.BLOCK_SHAPES.items() if not k.endswith("scale")}
    w["norm.query_norm.scale"] = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    w["norm.key_norm.scale"] = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    b = L.PackedBlock(w)
    torch.cuda.synchronize()
    return b


def device_rnd(torch, seed: int):
    import flux3_synth as syn
    g = torch.Generator(device="cuda").manual_seed(seed)

    def rnd(shape):
        t = torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).mul_(syn.WEIGHT_STD)
        return t.to(torch.bfloat16)
    return rnd


def build_model(L, torch, seed: int, n_early: int = 5, n_single: int = 28):
    """Seeded random-init weights generated on the device, blocks packed."""
    import flux3_synth as syn
    rnd = device_rnd(torch, seed)
    glob = {k: rnd(shp) for k, shp in syn.GLOBAL_SHAPES.items()}
    early = {m: [make_block(L, torch, rnd) for _ in range(n_early)] for m in syn.MODES}
    single = [make_block(L, torch, rnd) for _ in range(n_single)]
    return L.ModelWeights(glob, early, single)


# The launch timer's kinds, the name of the kernel each one times, and its
# algorithmic work per launch of r rows (unit as in kernel_fixtures).
TIMED = {
    "in_proj": ("gemm_in_proj_swiglu", lambda r: 2.0 * r * HIDDEN * (3 * HIDDEN + 2 * MLP), "flop"),
    "qk_norm_rope": ("qk_norm_rope", lambda r: 8.0 * r * HIDDEN + 512.0 * r, "byte"),
    "attention": ("attention", lambda r: 4.0 * r * r * HIDDEN, "flop"),
    "out_proj": ("gemm_out_proj_gated", lambda r: 2.0 * r * (HIDDEN + MLP) * HIDDEN, "flop"),
    "ln_modulate": ("ln_modulate", lambda r: 6.0 * r * HIDDEN, "byte"),
}


def in_stack_kernels(records, steps: int):
    """Launch-timer records [(kind, rows, ms)] of the timed steps, summarised
    per kernel and row count: launches, average ms, rate."""
    out = {}
    for kind, rows, ms in records:
        name, work, unit = TIMED[kind]
        k = out.setdefault(name, {"ms_per_step": 0.0, "rows": {}})
        k["ms_per_step"] += ms / steps
        r = k["rows"].setdefault(str(rows), {"launches": 0, "ms": 0.0})
        r["launches"] += 1
        r["ms"] += ms
    for name, k in out.items():
        _, work, unit = next(v for v in TIMED.values() if v[0] == name)
        k["ms_per_step"] = round(k["ms_per_step"], 3)
        for rows, r in k["rows"].items():
            avg = r.pop("ms") / r["launches"]
            r["avg_ms"] = round(avg, 4)
            rate = work(int(rows)) / (avg * 1e-3)
            if unit == "flop":
                r["tflops"] = round(rate / 1e12, 1)
            else:
                r["gbs"] = round(rate / 1e9, 1)
    return out


def kernel_fixtures(L, torch, blk, table, n_img: int, n: int):
    """The joint block's kernels at n rows, each as (call, work, unit):
    work is algorithmic FLOP (unit 'flop') or HBM bytes (unit 'byte') per call."""
    g = torch.Generator(device="cuda").manual_seed(1)
    xm = torch.empty((n, HIDDEN), dtype=torch.bfloat16, device="cuda")
    qkv = torch.randn((n, 3 * HIDDEN), device="cuda", generator=g).to(torch.bfloat16)
    cat = torch.randn((n, HIDDEN + MLP), device="cuda", generator=g).to(torch.bfloat16)
    xs = torch.randn((n, HIDDEN), device="cuda", generator=g)
    mod = torch.randn((2, 3, HIDDEN), device="cuda", generator=g) * 0.1
    segs = [0, n_img, n]
    L.flux3_ln_modulate(xs, xm, segs, mod)
    qn = qkv.clone()
    attn_ws_bytes = L.flux3_attention_workspace_size(n)
    attn_ws = L.workspace(attn_ws_bytes) if attn_ws_bytes else None
    return {
        "ln_modulate": (lambda: L.flux3_ln_modulate(xs, xm, segs, mod),
                        6.0 * n * HIDDEN, "byte"),        # fp32 x in, bf16 out
        "gemm_in_proj_swiglu": (lambda: L.flux3_block_in_proj(xm, blk.w_in, qkv, cat[:, HIDDEN:]),
                                2.0 * n * HIDDEN * (3 * HIDDEN + 2 * MLP), "flop"),
        "qk_norm_rope": (lambda: L.flux3_qk_norm_rope(qn[:, :HIDDEN], qn[:, HIDDEN:2 * HIDDEN],
                                                      blk.q_scale, blk.k_scale, table),
                         8.0 * n * HIDDEN + 512.0 * n, "byte"),  # q, k in and out + rope table
        # the block's schedule (balanced over the last round; the call also
        # clears the workspace's counters with a small fill kernel)
        "attention": (lambda: L.flux3_attention_ws(qkv[:, :HIDDEN], qkv[:, HIDDEN:2 * HIDDEN],
                                                   qkv[:, 2 * HIDDEN:], cat[:, :HIDDEN], attn_ws),
                      4.0 * n * n * HIDDEN, "flop"),
        "gemm_out_proj_gated": (lambda: L.flux3_block_out_proj(cat, blk.w_out, xs, segs, mod),
                                2.0 * n * (HIDDEN + MLP) * HIDDEN, "flop"),
    }


def cold_fixtures(L, torch, blk, table, n_img: int, n: int, sets: int = 6):
    """The memory-bound kernels of kernel_fixtures, each call on the next of
    `sets` copies of its buffers (together well past the 256 MB Infinity
    Cache), so back-to-back calls find their inputs in HBM, not in a cache."""
    g = torch.Generator(device="cuda").manual_seed(2)
    xs = [torch.randn((n, HIDDEN), device="cuda", generator=g) for _ in range(sets)]
    xm = [torch.empty((n, HIDDEN), dtype=torch.bfloat16, device="cuda") for _ in range(sets)]
    qk = [torch.randn((n, 2 * HIDDEN), device="cuda", generator=g).to(torch.bfloat16) for _ in range(sets)]
    tables = [table.clone() for _ in range(sets)]
    mod = torch.randn((2, 3, HIDDEN), device="cuda", generator=g) * 0.1
    segs = [0, n_img, n]
    state = {"ln": 0, "qk": 0}

    def ln():
        i = state["ln"] = (state["ln"] + 1) % sets
        L.flux3_ln_modulate(xs[i], xm[i], segs, mod)

    def qk_norm():
        i = state["qk"] = (state["qk"] + 1) % sets
        L.flux3_qk_norm_rope(qk[i][:, :HIDDEN], qk[i][:, HIDDEN:], blk.q_scale, blk.k_scale, tables[i])

    return {"ln_modulate": ln, "qk_norm_rope": qk_norm}


def event_time_ms(torch, fn, reps: int) -> float:
    """Average duration of fn() over reps launches, HIP events on the current stream."""
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    b.synchronize()
    return a.elapsed_time(b) / reps


def sampler_loop(L, torch, model, img, txt, table, n_img: int, n_txt: int, steps: int):
    """The whole sampling loop (steps flow-map steps) as one flux3_sample call,
    timed eagerly and as one captured HIP graph (3 timed runs each)."""
    ws = L.workspace(L.flux3_sample_workspace_size(n_img, 0, n_txt))
    x0 = img.float().contiguous()
    x = x0.clone()
    sig = L.flux3_sigmas(steps)

    def run():
        L.flux3_sample(model, x, None, txt, table, sig, ws)

    eager = event_time_ms(torch, run, 3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    graph_ms = event_time_ms(torch, graph.replay, 3)
    x.copy_(x0)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.isfinite(x).all().item(), "non-finite sample"
    del graph
    n = n_img + n_txt
    return {"tokens": n, "steps": steps, "eager_ms_per_image": round(eager, 3),
            "graph_ms_per_image": round(graph_ms, 3), "graph_steps_per_s": round(steps * 1e3 / graph_ms, 2),
            "graph_tflops": round(steps * stack_flops(n_img, 0, n_txt) / (graph_ms * 1e-3) / 1e12, 1)}


def fp8r(L, torch, syn, model, img, txt, table, n_img: int, n_txt: int, seed: int):
    """The same transformer with fp8r blocks (rowwise E4M3 projections, from
    the same weights): one stack step at 4608 tokens (3 timed after a
    warm-up), and one joint block at 4608 rows in bf16 and fp8 (5 each)."""
    q = L.ModelWeights(model.glob, {m: [b.fp8_copy() for b in bl] for m, bl in model.early.items()},
                       [b.fp8_copy() for b in model.single])
    ws = L.workspace(L.flux3_stack_workspace_size(n_img, 0, n_txt))
    v = torch.empty((n_img, 128), dtype=torch.float32, device="cuda")
    sig = L.flux3_sigmas(16).tolist()
    ms = event_time_ms(torch, lambda: L.flux3_stack_forward(q, img, None, txt, table, sig[0], sig[1], v, ws), 3)
    assert torch.isfinite(v).all().item(), "non-finite velocity"
    n = n_img + n_txt
    x = torch.randn((n, HIDDEN), device="cuda", generator=torch.Generator(device="cuda").manual_seed(seed))
    mod = torch.randn((2, 3, HIDDEN), device="cuda", generator=torch.Generator(device="cuda").manual_seed(seed + 1)) * 0.1
    bws = L.workspace(L.flux3_block_workspace_size(n))
    segs = [0, n_img, n]
    blk = {"bf16": model.single[0], "fp8": q.single[0]}
    block_ms = {k: round(event_time_ms(torch, lambda b=b: L.flux3_block_forward(x, segs, mod, b, table, bws), 5), 4)
                for k, b in blk.items()}
    f = stack_flops(n_img, 0, n_txt)
    del q, ws, bws
    return {"workload": "stack_t2i_1024_4608tok", "ms_per_step": round(ms, 3), "tflops": round(f / (ms * 1e-3) / 1e12, 1),
            "joint_block_ms": block_ms, "mfma_dtype": "fp8 e4m3 (block projections), bf16 elsewhere"}


def cfg_flops(n_img: int, n_t0: int, n_t1: int, n_early: int = 5, n_single: int = 28) -> float:
    """Algorithmic work of one guided step on the pack (no references): the
    image stream's embedding and stage 1 once, both texts, stage 2 on both
    samples (GEMMs on all rows, attention within each sample), final layer on
    both image blocks, conditioning once."""
    gemm_row = 2.0 * (4 * HIDDEN * HIDDEN + 3 * HIDDEN * MLP)   # per row per block
    att = lambda n: 4.0 * n * n * HIDDEN
    n0, n1 = n_img + n_t0, n_img + n_t1
    f = 2.0 * n_img * 128 * HIDDEN + 2.0 * (n_t0 + n_t1) * 20480 * HIDDEN
    f += n_early * (gemm_row * (n_img + n_t0 + n_t1) + att(n_img) + att(n_t0) + att(n_t1))
    f += n_single * (gemm_row * (n0 + n1) + att(n0) + att(n1))
    f += 2.0 * 2 * n_img * HIDDEN * 128
    f += 2.0 * (HIDDEN * 256 + HIDDEN * HIDDEN) * 2 + 2.0 * 3 * HIDDEN * HIDDEN * 2 * 2 + 2.0 * 2 * HIDDEN * HIDDEN
    return f


def cfg_base(L, torch, syn, model, seed: int):
    """The base checkpoint's guided sampling: pack [empty prompt (80 tokens),
    prompt (512 tokens)] on a 1024^2 image, guidance 3.5, 50 steps, the same
    weights without ref_time_in.  One guided step timed with HIP events (3
    after a warm-up), then the 50-step loop as one flux3_sample_cfg call."""
    base = L.ModelWeights({k: t for k, t in model.glob.items() if not k.startswith("ref_time_in.")},
                          model.early, model.single)
    n_img, n_t0, n_t1, g, steps = 4096, 80, 512, 3.5, 50
    img = syn.latents(seed + 8, n_img).to("cuda")
    txt0 = syn.text_features(seed + 9, n_t0).to("cuda")
    txt1 = syn.text_features(seed + 10, n_t1).to("cuda")
    table = L.flux3_rope_table(L.flux3_build_ids_cfg(64, 64, n_t0, n_t1).to("cuda"))
    ws = L.workspace(L.flux3_sample_cfg_workspace_size(n_img, 0, n_t0, n_t1))
    v = torch.empty((n_img, 128), dtype=torch.float32, device="cuda")
    sig = L.flux3_sigmas(steps)
    s0 = float(sig[0])
    ms = event_time_ms(torch, lambda: L.flux3_stack_forward_cfg(base, img, None, txt0, txt1, table, s0, 0.0,
                                                                g, v, ws), 3)
    x = img.float().contiguous()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    L.flux3_sample_cfg(base, x, None, txt0, txt1, table, sig, g, ws)
    e1.record(st)
    e1.synchronize()
    loop_ms = e0.elapsed_time(e1)
    assert torch.isfinite(x).all().item(), "non-finite sample"
    f = cfg_flops(n_img, n_t0, n_t1)
    return {"workload": "cfg_base_t2i_1024_pack_80_512tok", "rows": 2 * n_img + n_t0 + n_t1, "guidance": g,
            "ms_per_step": round(ms, 2), "tflop_per_step": round(f / 1e12, 2),
            "tflops": round(f / (ms * 1e-3) / 1e12, 1), "steps": steps, "image_s": round(loop_ms / 1e3, 3)}


def long_step(L, torch, syn, model, seed: int, steps: int = 2):
    """One flow-map step of the whole stack at the longest sequence the pages
    allow (1024^2 image, ten 1024^2 references, 4080 text tokens), timed with
    HIP events over `steps` steps after one warm-up."""
    name = "stack_10ref_1024_49136tok"
    lay = syn.LONG_WORKLOADS[name]
    img = syn.latents(seed + 5, lay.n_img).to("cuda")
    cond = syn.latents(seed + 6, lay.n_cond, "cond").to("cuda")
    txt = syn.text_features(seed + 7, lay.n_txt).to("cuda")
    table = L.flux3_rope_table(L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs).to("cuda"))
    ws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, lay.n_cond, lay.n_txt))
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    sig = L.flux3_sigmas(16).tolist()

    def run():
        L.flux3_stack_forward(model, img, cond, txt, table, sig[0], sig[1], v, ws)

    ms = event_time_ms(torch, run, steps)
    assert torch.isfinite(v).all().item(), "non-finite velocity"
    flops = stack_flops(lay.n_img, lay.n_cond, lay.n_txt)
    del ws
    return {"workload": name, "tokens": lay.n_total, "steps": steps, "ms_per_step": round(ms, 2),
            "tflop_per_step": round(flops / 1e12, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}


def probe_peaks(torch):
    """What this GPU sustains: register-only bf16 MFMA (one wave per SIMD,
    8 independent accumulator chains, random operands) and streaming copies
    of 2 GiB (HBM read + write: the probe copy on 512, 768 and 1024
    workgroups, and torch's elementwise multiply, the best of them), each the
    median of 5 timed launches after a warm-up (libflux3_probe.so)."""
    import ctypes as C
    lib = C.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "latent_flow_matching_flux3_amd",
                              "libflux3_probe.so"))
    lib.flux3_probe_mfma_bf16.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    lib.flux3_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 40000
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()

    def mfma():
        assert lib.flux3_probe_mfma_bf16(cus, iters, out.data_ptr(), st.cuda_stream) == 0

    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_mfma = median_event_ms(torch, mfma, 5)
    copies = {}
    for blocks in (512, 768, 1024):
        def copy(b=blocks):
            assert lib.flux3_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, b, st.cuda_stream) == 0
        copies[f"probe_copy_{blocks}wg"] = round(2.0 * nbytes / (median_event_ms(torch, copy, 5) * 1e-3) / 1e9, 1)
    assert torch.equal(src[:1 << 20], dst[:1 << 20])
    copies["torch_mul"] = round(2.0 * nbytes / (median_event_ms(torch, lambda: torch.mul(src, 1.0, out=dst), 5)
                                                 * 1e-3) / 1e9, 1)
    flop = cus * 4 * iters * 8 * 32768.0
    del src, dst
    return {"mfma_bf16_tflops": round(flop / (t_mfma * 1e-3) / 1e12, 1),
            "hbm_copy_gbs": max(copies.values()), "copies_gbs": copies,
            "vendor": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS},
            "how": f"register-only v_mfma_f32_32x32x16_bf16, {cus} workgroups x 4 waves x {iters} x 8; "
                   f"copies of {nbytes >> 30} GiB; median of 5"}


def median_event_ms(torch, fn, reps: int, flush=None) -> float:
    """Median duration of fn() over reps launches, each between its own HIP
    events on the current stream; flush() (untimed) runs before each."""
    import statistics
    st = torch.cuda.current_stream()
    fn()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        fn()
        b.record(st)
        b.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times)


def config_lines(L, torch, syn, model, seed: int):
    """The other workloads: one joint block at 96 (128^2 px), 4608 (1024^2
    t2i) and 8704 tokens (1024^2 with one 1024^2 reference), each the median
    of 20 launches, and one stack step with four 1024^2 references (20,992
    tokens), the median of 3."""
    out = {}
    blk = model.single[0]
    for name in ("block_128px_96tok", "block_t2i_1024_4608tok", "block_i2i_1024_8704tok"):
        lay = syn.WORKLOADS[name]
        n = lay.n_total
        segs = [0] + [b for _, _, b in lay.segments()]
        table = L.flux3_rope_table(L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs).to("cuda"))
        x = torch.randn((n, HIDDEN), device="cuda", generator=torch.Generator(device="cuda").manual_seed(seed))
        mod = torch.randn((len(segs) - 1, 3, HIDDEN), device="cuda",
                          generator=torch.Generator(device="cuda").manual_seed(seed + 1)) * 0.1
        ws = L.workspace(L.flux3_block_workspace_size(n))
        ms = median_event_ms(torch, lambda: L.flux3_block_forward(x, segs, mod, blk, table, ws), 20)
        assert torch.isfinite(x).all().item(), "non-finite block output"
        f = block_flops(n)
        out[name] = {"tokens": n, "ms": round(ms, 4), "gflop": round(f / 1e9, 1),
                     "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
        del ws
    name = "stack_4ref_1024_20992tok"
    lay = syn.WORKLOADS[name]
    img, cond, txt = (t.to("cuda") for t in syn.stack_inputs(lay, seed + 12))
    table = L.flux3_rope_table(L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs).to("cuda"))
    ws = L.workspace(L.flux3_stack_workspace_size(lay.n_img, lay.n_cond, lay.n_txt))
    v = torch.empty((lay.n_img, 128), dtype=torch.float32, device="cuda")
    sig = L.flux3_sigmas(16).tolist()
    ms = median_event_ms(torch, lambda: L.flux3_stack_forward(model, img, cond, txt, table, sig[0], sig[1], v, ws), 3)
    assert torch.isfinite(v).all().item(), "non-finite velocity"
    f = stack_flops(lay.n_img, lay.n_cond, lay.n_txt)
    out[name] = {"tokens": lay.n_total, "ms_per_step": round(ms, 2), "tflop_per_step": round(f / 1e12, 1),
                 "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
    del ws
    return out


def cpu_baseline(seed: int):
    """The CPU oracle (float64 NumPy), untuned, on a bounded sample: one joint
    block at 4608 tokens (image 64x64 + 512 text), two modulation segments."""
    import torch
    import flux3_synth as syn
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    lay = syn.WORKLOADS["block_t2i_1024_4608tok"]
    ids = O.build_ids(lay.img_h, lay.img_w, lay.n_txt, lay.refs)
    w = {k: v.to(torch.float64).numpy() for k, v in syn.block_weights(seed, "single_blocks.0").items()}
    x = syn.block_activations(seed + 1, lay.n_total).to(torch.float64).numpy()
    mods = syn.normal_f32((2, 3, HIDDEN), 0.5, seed + 2, "mods").to(torch.float64).numpy()
    segs = [(a, b) for _, a, b in lay.segments()]
    t0 = time.perf_counter()
    O.block_forward(x, segs, mods, w, ids)
    dt = time.perf_counter() - t0
    fl = block_flops(lay.n_total)
    # the 128^2 px block (96 tokens) on all cores and on one thread
    small = syn.WORKLOADS["block_128px_96tok"]
    ids_s = O.build_ids(small.img_h, small.img_w, small.n_txt)
    xs = syn.block_activations(seed + 1, small.n_total).to(torch.float64).numpy()
    segs_s = [(a, b) for _, a, b in small.segments()]
    t0 = time.perf_counter()
    O.block_forward(xs, segs_s, mods, w, ids_s)
    dt_s = time.perf_counter() - t0
    dt_s1 = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.block_forward(xs, segs_s, mods, w, ids_s)
            dt_s1 = time.perf_counter() - t0
    except ImportError:
        pass
    fl_s = block_flops(small.n_total)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one joint block at {lay.n_total} tokens ({fl / 1e12:.2f} TFLOP), float64 NumPy, "
                      f"{dt:.2f} s; the full step is {stack_flops(4096, 0, 512) / 1e12:.1f} TFLOP",
            "block_96tok_ms": {"all_cores": round(dt_s * 1e3, 1),
                               "one_thread": None if dt_s1 is None else round(dt_s1 * 1e3, 1),
                               "gflop": round(fl_s / 1e9, 1)}}


def run_only(args, L, torch, syn):
    """One kernel, args.steps times, for counter collection."""
    lay = syn.WORKLOADS["stack_t2i_1024_4608tok"]
    n = lay.n_total
    if args.only == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        fn, work, unit = (lambda: torch.mul(src, 1.0, out=dst)), 2.0 * COPY_BYTES, "byte"
    elif args.only == "loop_96tok":
        # the 128^2 px workload's 16 flow-map steps in one flux3_sample call
        model = build_model(L, torch, args.seed)
        small = syn.WORKLOADS["block_128px_96tok"]
        img = syn.latents(args.seed + 3, small.n_img).to("cuda")
        txt = syn.text_features(args.seed + 4, small.n_txt).to("cuda")
        table = L.flux3_rope_table(L.flux3_build_ids(small.img_h, small.img_w, small.n_txt).to("cuda"))
        ws = L.workspace(L.flux3_sample_workspace_size(small.n_img, 0, small.n_txt))
        sig = L.flux3_sigmas(16)
        x = img.float().contiguous()
        fn = lambda: L.flux3_sample(model, x, None, txt, table, sig, ws)
        work, unit = 16 * stack_flops(small.n_img, 0, small.n_txt), "flop"
    else:
        blk = make_block(L, torch, device_rnd(torch, args.seed))
        ids = L.flux3_build_ids(lay.img_h, lay.img_w, lay.n_txt).to("cuda")
        table = L.flux3_rope_table(ids)
        names = {"in_proj": "gemm_in_proj_swiglu", "out_proj": "gemm_out_proj_gated"}
        fx = kernel_fixtures(L, torch, blk, table, lay.n_img, n)
        fn, work, unit = fx[names.get(args.only, args.only)]
    ms = event_time_ms(torch, fn, args.steps)
    rate = work / (ms * 1e-3) / (1e12 if unit == "flop" else 1e9)
    print(json.dumps({"kernel": args.only, "calls": args.steps + 1, "ms": round(ms, 4),
                      "work_per_call": work, "rate": round(rate, 1),
                      "rate_unit": "TFLOP/s" if unit == "flop" else "GB/s"}), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        return 2
    import torch
    import latent_flow_matching_flux3_amd as L
    import flux3_synth as syn

    assert torch.cuda.is_available(), "no GPU visible"
    L.lib()
    if args.only:
        return run_only(args, L, torch, syn)
    if args.probe:
        print(json.dumps({"peaks": probe_peaks(torch)}), flush=True)
        return 0
    lay = syn.WORKLOADS["stack_t2i_1024_4608tok"]
    n_img, n_txt = lay.n_img, lay.n_txt
    n = n_img + n_txt

    print("[bench] building ~5.5B-parameter model on the device", file=sys.stderr, flush=True)
    model = build_model(L, torch, args.seed)
    img = syn.latents(args.seed + 1, n_img).to("cuda")
    txt = syn.text_features(args.seed + 2, n_txt).to("cuda")
    ids = L.flux3_build_ids(lay.img_h, lay.img_w, n_txt).to("cuda")
    table = L.flux3_rope_table(ids)
    ws = L.workspace(L.flux3_stack_workspace_size(n_img, 0, n_txt))
    v = torch.empty((n_img, 128), dtype=torch.float32, device="cuda")
    x = img.float().contiguous()
    xb = img.clone()
    sig = L.flux3_sigmas(16).tolist()

    def step(k):
        s0, s1 = sig[k % 16], sig[k % 16 + 1]
        L.flux3_stack_forward(model, xb, None, txt, table, s0, s1, v, ws)
        L.flux3_euler_step(x, xb, v, s0, s1)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    # The library's launch timer records HIP events around launches of the
    # block's kernels, on the stream each runs on.  First an untimed pass of
    # the same steps with every block kernel timed (where a step's time goes,
    # which kernel dominates; a kernel fused into another launch has no
    # records of its own); then the timed steps with the dominant kernel's
    # launches timed (two event packets per launch; all five kinds at once
    # would add ≈1.7% to the step).
    in_stack = None
    timed_kind = None
    timer_cap = args.steps * 6 * (5 + 5 + 28) + 64
    if not args.no_kernel_timer:
        nb = max(1, min(args.steps, 5))
        L.flux3_timer_start(TIMED, timer_cap)
        for k in range(nb):
            step(k)
        torch.cuda.synchronize()
        in_stack = in_stack_kernels(L.flux3_timer_stop(timer_cap), nb)
        in_stack["steps"] = nb
        timed_kind = max((k for k in TIMED if TIMED[k][0] in in_stack),
                         key=lambda k: in_stack[TIMED[k][0]]["ms_per_step"])
        L.flux3_timer_start([timed_kind], timer_cap)
    t0 = time.perf_counter()
    e0.record(st)
    for k in range(args.steps):
        step(k)
        marks[k].record(st)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed = None
    if timed_kind is not None:
        timed = in_stack_kernels(L.flux3_timer_stop(timer_cap), args.steps)[TIMED[timed_kind][0]]
    ms = e0.elapsed_time(e1) / args.steps
    import statistics
    step_ms = [e0.elapsed_time(marks[0])] + [marks[k - 1].elapsed_time(marks[k]) for k in range(1, args.steps)]
    median_ms = statistics.median(step_ms)
    assert torch.isfinite(v).all().item(), "non-finite velocity"
    flops = stack_flops(n_img, 0, n_txt)
    tflops = flops / (ms * 1e-3) / 1e12

    # Per-kernel timing at the joint-block shape (4608 rows), same stream.
    fx = kernel_fixtures(L, torch, model.single[0], table, n_img, n)
    per_kernel = {}
    cold_fx = {} if args.no_fixtures else cold_fixtures(L, torch, model.single[0], table, n_img, n)
    if not args.no_fixtures:
        print("[bench] per-kernel timing", file=sys.stderr, flush=True)
    for name, (fn, work, unit) in ({} if args.no_fixtures else fx).items():
        kms = event_time_ms(torch, fn, args.kernel_reps)
        med = median_event_ms(torch, fn, args.kernel_reps)
        if unit == "flop":
            per_kernel[name] = {"ms": round(kms, 4), "tflops": round(work / kms / 1e9, 1),
                                "median_ms": round(med, 4)}
        else:
            per_kernel[name] = {"ms": round(kms, 4), "gbs": round(work / kms / 1e6, 1), "median_ms": round(med, 4)}
            if name in cold_fx:
                cms = event_time_ms(torch, cold_fx[name], args.kernel_reps)
                per_kernel[name].update({"hbm_ms": round(cms, 4), "hbm_gbs": round(work / cms / 1e6, 1),
                                         "hbm_frac": round(work / cms / 1e6 / PEAK_HBM_GBS, 3)})
    del cold_fx
    torch.cuda.synchronize()
    # Dominant kernel: most time per step.  With the launch timer: its
    # launches at the joint block's 4608 rows inside the timed steps (28 per
    # step); without it: its back-to-back fixture at 4608 rows.
    if timed:
        dom = TIMED[timed_kind][0]
        dom_ms = timed["rows"][str(n)]["avg_ms"]
        dom_launches = timed["rows"][str(n)]["launches"]
        basis = (f"HIP events around each of its {dom_launches} launches at {n} rows in the "
                 f"{args.steps} timed steps (the library's launch timer, on the launch's stream)")
        if dom == "gemm_in_proj_swiglu":
            basis += ("; at this size the launch also applies the QK RMSNorm + RoPE to q and k in its "
                      "epilogue, and work_per_launch counts the projection's FLOPs alone")
    else:
        dom = max(per_kernel, key=lambda k: per_kernel[k]["ms"])
        dom_ms = per_kernel[dom]["ms"]
        basis = f"HIP events around {args.kernel_reps} back-to-back launches at {n} rows"
    dom_work, dom_unit = fx[dom][1], fx[dom][2]
    if dom_unit == "flop":
        achieved = dom_work / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom)}
    else:
        achieved = dom_work / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof.update({"avg_ms": round(dom_ms, 4), "work_per_launch": dom_work, "measured": basis})

    loops = None
    if not args.no_sampler_loop:
        print("[bench] 16-step sampler loop: one flux3_sample call, eager and as a HIP graph",
              file=sys.stderr, flush=True)
        loops = {"4608tok": sampler_loop(L, torch, model, img, txt, table, n_img, n_txt, 16)}
        small = syn.WORKLOADS["block_128px_96tok"]
        s_img = syn.latents(args.seed + 3, small.n_img).to("cuda")
        s_txt = syn.text_features(args.seed + 4, small.n_txt).to("cuda")
        s_table = L.flux3_rope_table(L.flux3_build_ids(small.img_h, small.img_w, small.n_txt).to("cuda"))
        loops["96tok"] = sampler_loop(L, torch, model, s_img, s_txt, s_table, small.n_img, small.n_txt, 16)

    fp8 = None
    if not args.no_fp8:
        print("[bench] fp8r blocks: stack step and one joint block", file=sys.stderr, flush=True)
        fp8 = fp8r(L, torch, syn, model, img, txt, table, n_img, n_txt, args.seed + 11)

    cfg = None
    if not args.no_cfg:
        print("[bench] base checkpoint: guided pack, 50-step loop", file=sys.stderr, flush=True)
        cfg = cfg_base(L, torch, syn, model, args.seed)

    long_ctx = None
    if not args.no_long:
        print("[bench] stack step at the longest sequence (49,136 tokens)", file=sys.stderr, flush=True)
        long_ctx = long_step(L, torch, syn, model, args.seed)

    configs = None
    if not args.no_configs:
        print("[bench] blocks at 96 / 4608 / 8704 tokens, stack step at 20,992 tokens", file=sys.stderr, flush=True)
        configs = config_lines(L, torch, syn, model, args.seed + 20)

    print("[bench] peak probes", file=sys.stderr, flush=True)
    peaks = probe_peaks(torch)
    roof["frac_of_probe_peak"] = round(roof["achieved"] / (peaks["mfma_bf16_tflops"] if roof["unit"] == "TFLOP/s"
                                                           else peaks["hbm_copy_gbs"]), 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle, one block)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.seed)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "median_ms_per_step": round(median_ms, 3),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 3),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "steps_per_s": round(1e3 / ms, 3),
        "image_s_16_steps": round(16 * ms / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents and text features, N(0,0.02) random-init weights)",
        "config": {"workload": "stack_t2i_1024_4608tok", "image_tokens": n_img, "text_tokens": n_txt,
                   "blocks": "5 per-stream + 28 joint", "params": "5.55B", "tflop_per_step": round(flops / 1e12, 3),
                   "sampler": "flow map, 16-step shifted schedule (alpha 6.93)", "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "peaks": peaks,
        "kernels_in_stack": in_stack,
        "kernels": per_kernel or None,
        "configs": configs,
        "sampler_loop": loops,
        "fp8r": fp8,
        "cfg_base": cfg,
        "long_context": long_ctx,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
