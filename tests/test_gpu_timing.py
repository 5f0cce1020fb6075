"""GPU: kernel timestamps (w4a16_time_next_launch) on every contraction launch site.

An armed request launches the next tile or matvec kernel through hipExtLaunchKernel with the
caller's events.  That launch packs the kernel arguments itself, so each case runs once plainly
and once timed on the same inputs and requires the two outputs to be identical bit for bit
(same kernel, same inputs).  The kernel span must be positive and no longer than events
recorded on the stream around the same call.  A request met by a launch under HIP graph capture
is consumed by a plain launch: the replays match the eager result and the events stay untouched.
"""

import numpy as np
import pytest

from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bits, to_device

pytestmark = pytest.mark.gpu


def _dev(seed, M, N, K, nbits=4):
    p = synth.random_problem(seed, M, N, K, bits=nbits)
    return to_device(p)


def _cases(lib):
    """(name, callable returning the output tensors) for each launch site and kernel family."""
    cases = []

    def linear(name, seed, M, N, K, **kw):
        x, wq, s, b = _dev(seed, M, N, K)
        cases.append((name, lambda: [lib.linear(x, wq, s, b, **kw)]))

    linear("qmm 64-row tile, ragged", 31, 33, 96, 256)
    linear("qmm split 2 (tile + slice sum)", 32, 70, 200, 1024, path="qmm", split_k=2)
    linear("qmm exact-code 128-row tile", 33, 1100, 256, 384)
    linear("skinny 32-row tile", 34, 24, 1000, 1024)
    for (N, K, M, name) in [(4000, 256, 3, "qmv burst"), (1000, 16384, 1, "qmv packed burst"),
                            (2600, 8320, 5, "qmv 16-column K-split"), (16390, 384, 8, "qmv 64-column"),
                            (33000, 256, 1, "qmv wide")]:
        linear(name, 35, M, N, K)
    linear("row-amortized matvec (skinny rows)", 36, 12, 2600, 1024)

    x, wq, s, b = _dev(37, 64, 384, 512)
    _, wk, sk, bk = _dev(38, 64, 256, 512)
    cases.append(("grouped q|k", lambda: lib.w4a16_linear_grouped(x, [(wq, s, b), (wk, sk, bk)])))
    _, wu, su, bu = _dev(39, 64, 384, 512)
    cases.append(("gate/up pair", lambda: [lib.w4a16_gate_up_swiglu(x, (wq, s, b), (wu, su, bu))]))
    cases.append(("w4a8", lambda: [lib.w4a8_linear(x, wq, s, b)]))

    for nbits, M, mode, name in [(3, 1, lib.QMV_BURST, "3-bit packed burst"), (3, 5, lib.QMV_BURST, "3-bit burst"),
                                 (2, 2, lib.QMV_AMORTIZED, "2-bit row-amortized"),
                                 (8, 1, lib.QMV_PER_ROW, "8-bit per row")]:
        xa, wa, sa, ba = _dev(40 + nbits, M, 1000, 1024, nbits)
        cases.append((name, lambda xa=xa, wa=wa, sa=sa, ba=ba, nbits=nbits, mode=mode:
                      [lib.qmv_affine(xa, wa, sa, ba, nbits, mode=mode)]))
    return cases


def test_timed_launch_matches_plain_launch_on_every_site(lib):
    import torch
    for name, fn in _cases(lib):
        announce(f"timed launch: {name}")
        plain = [bits(y) for y in fn()]
        k0, k1, c0, c1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        k0.record()
        k1.record()
        torch.cuda.synchronize()
        c0.record()
        lib.w4a16_time_next_launch(k0, k1)
        outs = fn()
        c1.record()
        torch.cuda.synchronize()
        timed = [bits(y) for y in outs]
        assert all(np.array_equal(a, t) for a, t in zip(plain, timed)), f"{name}: timed launch differs"
        kernel_ms, call_ms = k0.elapsed_time(k1), c0.elapsed_time(c1)
        assert 0.0 < kernel_ms <= call_ms, f"{name}: kernel {kernel_ms} ms, call {call_ms} ms"


def test_request_is_consumed_and_can_be_cancelled(lib):
    import torch
    x, wq, s, b = _dev(50, 40, 256, 512)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    k1.record()
    torch.cuda.synchronize()
    lib.w4a16_time_next_launch(k0, k1)
    lib.linear(x, wq, s, b)
    torch.cuda.synchronize()
    first = k0.elapsed_time(k1)
    for _ in range(3):                       # no request armed: the events keep the first span
        lib.linear(x, wq, s, b)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == first
    lib.w4a16_time_next_launch(k0, k1)
    lib.w4a16_time_next_launch(None, None)   # cancelled before any launch
    lib.linear(x, wq, s, b)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == first


def test_request_met_under_graph_capture_launches_plainly(lib):
    import torch
    x, wq, s, b = _dev(51, 40, 256, 512)
    eager = bits(lib.linear(x, wq, s, b))
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    k1.record()
    torch.cuda.synchronize()
    before = k0.elapsed_time(k1)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        y = lib.linear(x, wq, s, b)                  # warm-up on the capture stream
        torch.cuda.synchronize()
        lib.w4a16_time_next_launch(k0, k1)
        with torch.cuda.graph(graph, stream=stream):
            y = lib.linear(x, wq, s, b)
    for _ in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), eager)
        lib.linear(x, wq, s, b)                      # eager work between the replays
        torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == before             # the captured launch did not take the events
