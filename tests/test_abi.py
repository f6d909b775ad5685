"""The C ABI: the library loads and exports every function include/flux3_dit.h
declares; host-side argument checks return status codes (no GPU needed: no
case below reaches a HIP call)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flux3_dit.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flux3_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import latent_flow_matching_flux3_amd as L
    L.lib()
    return L


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 15
    raw = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(L.EXPORTS) == names


def test_version(L):
    assert L.flux3_version() >= 100


def test_build_ids_matches_oracle(L):
    for h, w, nt, refs in ((0, 0, 5, []), (3, 4, 0, []), (2, 3, 4, [(1, 2), (3, 1)]), (64, 64, 512, [(64, 64)])):
        ids = L.flux3_build_ids(h, w, nt, refs).numpy().astype(np.float64)
        np.testing.assert_array_equal(ids, O.build_ids(h, w, nt, refs))


def test_build_ids_cfg_is_the_two_samples_ids(L):
    """Packed ids = sample 0's ids (image, refs, text 0), then sample 1's
    text ids and its image and reference ids (bit-exact)."""
    for h, w, n0, n1, refs in [(2, 3, 2, 3, [(1, 2)]), (4, 4, 80, 512, []), (3, 5, 0, 7, [(2, 2), (1, 3)])]:
        got = L.flux3_build_ids_cfg(h, w, n0, n1, refs).numpy().astype(np.float64)
        s0 = O.build_ids(h, w, n0, refs)
        s1 = O.build_ids(h, w, n1, refs)
        n_shared = h * w + sum(a * b for a, b in refs)
        want = np.concatenate([s0, s1[n_shared:], s1[:n_shared]])
        np.testing.assert_array_equal(got, want)


def test_sigmas_match_oracle(L):
    for steps in (1, 16, 50):
        np.testing.assert_allclose(L.flux3_sigmas(steps).numpy(), O.sigmas(steps), rtol=1e-7, atol=1e-7)


def test_error_codes(L):
    lib = L.lib()
    n = C.c_int(0)
    assert lib.flux3_build_ids(-1, 2, 0, None, 0, None, C.byref(n)) == L.EINVAL
    assert b"non-negative" in lib.flux3_last_error()
    assert lib.flux3_build_ids(1, 1, 1, None, 0, None, C.byref(n)) == L.EINVAL
    # unsupported GEMM shape
    assert lib.flux3_linear(16, 128, 16, 128, 16, 64, None, 4, 64, 100, None) == L.EUNSUPPORTED
    # null pointer
    assert lib.flux3_linear(None, 128, 16, 128, 16, 64, None, 4, 64, 128, None) == L.EINVAL
    # misaligned pointer
    assert lib.flux3_linear(18, 128, 16, 128, 16, 64, None, 4, 64, 128, None) == L.EINVAL
    # bad leading dimension
    assert lib.flux3_linear(16, 100, 16, 128, 16, 64, None, 4, 64, 128, None) == L.EINVAL
    # segments that do not cover the rows
    segs = (C.c_int * 3)(0, 3, 6)
    assert lib.flux3_ln_modulate(16, 3072, 16, 3072, 7, segs, 2, 16, 9216, None) == L.EINVAL
    segs = (C.c_int * 3)(0, 3, 3)
    assert lib.flux3_ln_modulate(16, 3072, 16, 3072, 3, segs, 2, 16, 9216, None) == L.EINVAL
    # too many segments
    segs = (C.c_int * 10)(*range(10))
    assert lib.flux3_ln_modulate(16, 3072, 16, 3072, 9, segs, 9, 16, 9216, None) == L.EINVAL
    # workspace too small for the block
    w = L.BlockWeightsC(16, 16, 16, 16)
    segs = (C.c_int * 2)(0, 10)
    assert lib.flux3_block_forward(16, 10, segs, 1, 16, C.byref(w), 16, 16, 100, None) == L.EWORKSPACE
    assert lib.flux3_block_forward(16, 10, segs, 1, 16, C.byref(w), 16, None, 1 << 30, None) == L.EWORKSPACE
    # launch timer: not armed, no kinds, unknown kind, capacity out of range
    cnt = C.c_int(-1)
    assert lib.flux3_timer_stop(None, None, None, 0, C.byref(cnt)) == L.EINVAL
    assert lib.flux3_timer_start(0, 10) == L.EINVAL
    assert lib.flux3_timer_start(1 << 5, 10) == L.EINVAL
    assert lib.flux3_timer_start(1, 0) == L.EINVAL and lib.flux3_timer_start(1, (1 << 20) + 1) == L.EINVAL
    # empty inputs are a no-op
    assert lib.flux3_attention(None, 3072, None, 3072, None, 3072, None, 3072, 0, None) == L.OK
    assert lib.flux3_attention_ws(None, 3072, None, 3072, None, 3072, None, 3072, 0, None, 0, None) == L.OK
    # the balanced attention schedule needs its workspace where it applies (4608 rows: 864 items)
    assert L.flux3_attention_workspace_size(4608) > 512 * 2 * 128 * 128 * 4
    assert L.flux3_attention_workspace_size(2688) == 0 and L.flux3_attention_workspace_size(0) == 0
    # where the balanced schedule applies: 24 * ceil(n/128) items, more than one round of 512, not
    # a whole number of rounds, at most three whole rounds, leftover items short of 7/8 of a round
    for n, used in [(2689, True), (4096, True), (4608, True), (8272, True), (8704, True),
                    (5376, False),     # 1008 items: 496 leftover, nearly a whole round
                    (10880, False),    # 2040 items: 3 rounds + 504 leftover
                    (10752, False),    # 2016 items: 3 rounds + 480 leftover (> 7/8)
                    (12288, False),    # 2304 items: 4 whole rounds + 256 (past three rounds)
                    (20992, False), (49136, False), (65536, False)]:
        assert (L.flux3_attention_workspace_size(n) > 0) == used, n
    assert lib.flux3_attention_ws(16, 3072, 16, 3072, 16, 3072, 16, 3072, 4608, 16, 1000, None) == L.EWORKSPACE
    assert lib.flux3_attention_ws(16, 3072, 16, 3072, 16, 3072, 16, 3072, 4608, None, 1 << 30, None) == L.EINVAL
    assert lib.flux3_block_forward(None, 0, None, 0, None, None, None, None, 0, None) == L.OK
    # workspace sizes grow with n and are 0 for n = 0
    assert L.flux3_block_workspace_size(0) == 0
    assert L.flux3_block_workspace_size(4608) >= 4608 * (3072 + 9216 + 12288) * 2
    assert L.flux3_stack_workspace_size(4096, 0, 512) > L.flux3_block_workspace_size(4608)
    assert L.flux3_stack_workspace_size(0, 0, 512) == 0
