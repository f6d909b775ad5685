"""Host-side parts of bench.py (no GPU): the work counts it divides by, the
code digest that gates its measured-traffic figures, and the one-GPU rule."""
import os
import subprocess
import sys

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_block_and_stack_flops():
    for n in (96, 4608, 8704, 20992):
        assert bench.block_flops(n) == O.block_flops(n)
    # 45.73 TFLOP per 1024^2 text-to-image step, 339.2 with four references
    assert bench.stack_flops(4096, 0, 512) / 1e12 == pytest.approx(45.73, abs=0.01)
    assert bench.stack_flops(4096, 16384, 512) / 1e12 == pytest.approx(339.2, abs=0.1)


def test_launch_timer_work_counts():
    """The per-launch work the bench divides the launch timer's times by: the
    three MFMA kernels add up to the oracle's block FLOP count, and the
    memory-bound kernels' bytes are those of one pass over their operands."""
    flop = {k: w for k, (_, w, unit) in bench.TIMED.items() if unit == "flop"}
    assert set(flop) == {"in_proj", "attention", "out_proj"}
    for n in (96, 4608, 8704):
        assert sum(w(n) for w in flop.values()) == O.block_flops(n)
    _, ln, unit = bench.TIMED["ln_modulate"]
    assert unit == "byte" and ln(4608) == 4608 * 3072 * (4 + 2)               # fp32 in, bf16 out
    _, qk, unit = bench.TIMED["qk_norm_rope"]
    assert unit == "byte" and qk(4608) == 4608 * (2 * 3072 * 2 * 2 + 64 * 2 * 4)  # q, k in/out + table
    # the kinds the library's timer knows, numbered as the C header numbers them
    import re
    import latent_flow_matching_flux3_amd._lib as LL
    assert set(bench.TIMED) == set(LL.TIMER_KINDS)
    header = open(os.path.join(ROOT, "include", "flux3_dit.h")).read()
    defs = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"#define FLUX3_TIMER_(\w+) (\d+)", header)}
    assert defs == LL.TIMER_KINDS


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  /* one */\n}\n")
    d0 = bench.code_digest(str(a))
    a.write_text("// other header\n\nint f(int x)\n{\n    return x + 1;\n}\n")
    assert bench.code_digest(str(a)) == d0
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.code_digest(str(a)) != d0


def test_traffic_figures_match_current_code():
    """The measured-traffic table was taken on the kernels as they are: a
    change of their code makes the bench report traffic as null until the
    counters are taken again (this test then fails as a reminder)."""
    for k in bench.TRAFFIC:
        assert bench.measured_traffic(k) is not None, k


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout
