"""GPU test of the allocation-free entry point ``w4a16_linear_noalloc``, called through the C ABI.

Its output is compared with ``w4a16_linear``'s (with a caller workspace) and with the oracle, on
calls in a row of decreasing size that share the library's device scratch: a split plan, the
exact-code form (group sums in the scratch), then a smaller split plan.  Plans that fit the
scratch are the same plans, so the outputs are bit-identical; each also meets the tolerance.
"""

import ctypes

import numpy as np
import pytest

import oracle as O
from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bits, to_device

pytestmark = pytest.mark.gpu

# (M, N, K, seed): 512-row down projection (policy split: fp32 partials in the scratch), 1100 rows
# in the exact-code form (activation group sums in the scratch), a smaller split plan
CALLS = [(512, 2560, 9728, 91), (1100, 640, 2560, 92), (100, 700, 4096, 93)]


def _sample_rows(M):
    return np.unique(np.r_[0:8, M // 2:M // 2 + 8, M - 8:M]) if M > 64 else np.arange(M)


def test_noalloc_matches_linear_on_calls_in_a_row(lib):
    import torch
    L = lib.load()
    for M, N, K, seed in CALLS:
        plan = lib.w4a16_plan(M, N, K)
        assert plan["workspace_bytes"] <= lib.NOALLOC_SCRATCH_BYTES, (M, N, K)
        assert plan["workspace_bytes"] > 0, (M, N, K)        # each case uses the scratch
        p = synth.random_problem(seed, M, N, K)
        x, wq, s, b = to_device(p)
        y_ref_call = lib.w4a16_linear(x, wq, s, b)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        announce(f"w4a16_linear_noalloc M={M} N={N} K={K} plan split={plan['split_k']} variant={plan['variant']}")
        st = L.w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                                    M, N, K, 128, 0, None)
        assert st == 0, lib.w4a16_status_string(st)
        torch.cuda.synchronize()
        got, want = bits(y), bits(y_ref_call)
        assert np.array_equal(got, want), f"noalloc differs from w4a16_linear at M={M} N={N} K={K}"
        rows = _sample_rows(M)
        y_ref, A = O.reference(p["x"][rows], p["wq"], p["scales"], p["biases"])
        r = O.check(got[rows], y_ref, A)
        assert r.ok, str(r)


def test_noalloc_forced_split_beyond_the_scratch_is_rejected(lib):
    import torch
    L = lib.load()
    M, N, K = 512, 2560, 9728
    S = 8                                        # 8 * 512 * 2560 * 4 B = 40 MiB of partials
    assert S * M * N * 4 > lib.NOALLOC_SCRATCH_BYTES
    p = synth.random_problem(94, M, N, K)
    x, wq, s, b = to_device(p)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    announce(f"w4a16_linear_noalloc forced split {S} beyond the scratch")
    assert L.w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                                  M, N, K, 128, S, None) == 5
    # a forced split that fits runs, and agrees with qmm_w4a16 at the same split
    st = L.w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                                M, N, K, 128, 4, None)
    assert st == 0
    y2 = lib.qmm_w4a16(x, wq, s, b, split_k=4)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2))


def test_noalloc_decode_rows_and_side_stream(lib):
    """M <= 8 takes the matvec (no scratch); a call on a side stream orders with that stream."""
    import torch
    L = lib.load()
    M, N, K = 4, 9728, 2560
    p = synth.random_problem(95, M, N, K)
    x, wq, s, b = to_device(p)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    announce(f"w4a16_linear_noalloc M={M} on a side stream")
    st = L.w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                                M, N, K, 128, 0, ctypes.c_void_p(side.cuda_stream))
    assert st == 0
    side.synchronize()
    y_ref, A = O.reference(p["x"], p["wq"], p["scales"], p["biases"])
    r = O.check(bits(y), y_ref, A)
    assert r.ok, str(r)
