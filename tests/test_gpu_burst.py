"""GPU parity of the burst matvec (4-bit, up to four decode rows; every wave issues all of its
loads at once) through the C ABI, in both of its forms: 16 columns per workgroup, and the packed
form (4 K slices in the MFMA's spare rows, 4 columns per workgroup).  Each wave and group count
the policy gives either form (1 to 16 waves; 1 to 5 groups, or steps of 4 groups, each), integer
inputs bit for bit, random inputs against the CPU oracle within the tolerance of ``O.check``,
and sentinel rows around the output that no write may touch.
"""

import numpy as np
import pytest

from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bf16_from_bits, bits, to_device
from test_gpu_parity import SENTINEL, _exact_case, assert_parity, run

pytestmark = pytest.mark.gpu

BURST = 4   # the plan's instance index of the burst kernel

# (N, K) and what the plan makes of it: the packed form (tile_n 4) at 1 and 2 rows below 2048
# column blocks (below 1664 under 32 groups where the wide kernel applies), and at 3 and 4 rows
# up to 160 blocks and 64 groups; 16 columns otherwise
SHAPES = [
    (96, 128),      # one group: a single wave (packed at every M)
    (3, 1280),      # fewer columns than one packed workgroup covers
    (1, 640),       # a single column
    (33, 640),      # five groups: two packed waves (4 + 1 groups), ragged N
    (160, 2560),    # 20 groups: five packed waves
    (9728, 2560),   # packed at 1-2 rows (2432 workgroups); at 3-4 rows ten waves of two groups
    (200, 8192),    # 64 groups: sixteen packed waves of one step
    (300, 9728),    # 76 groups: ten packed waves of two steps at 1-2 rows; sixteen of five at 3-4
    (50, 10240),    # 80 groups: packed at 1-2 rows; sixteen waves of five at 3-4
    (40, 16384),    # 128 groups: sixteen packed waves of two steps at 1-2 rows (the others at 3-4)
    (24600, 384),   # 1538 column blocks: packed, one wave of two steps, at 1-2 rows; one wave of three groups at 3-4
    (32744, 1152),  # 2047 blocks, the last ragged, 9 groups (the wide kernel needs an even count):
                    # packed at 1-2 rows; three waves of three groups at 3-4
]


def _plan(lib, M, N, K):
    """The plan, which is the burst kernel's except for more than 80 groups at 3 and 4 rows."""
    p = lib.w4a16_plan(M, N, K, 128, lib.PATH_QMV)
    if M <= 2 or K // 128 <= 80:
        assert p["variant"] == BURST and p["tile_n"] in (4, 16), p
    return p


def _plan_any(lib, M, N, K):
    return lib.w4a16_plan(M, N, K, 128, lib.PATH_QMV)


def test_both_forms_are_covered(lib):
    """The packed form at every row count, the 16-column form at 3 and 4 rows (the only rows it
    serves)."""
    forms = {(M, _plan_any(lib, M, N, K)["variant"], _plan_any(lib, M, N, K)["tile_n"])
             for N, K in SHAPES for M in (1, 2, 3, 4)}
    assert {(M, BURST, 4) for M in (1, 2, 3, 4)} <= forms and {(M, BURST, 16) for M in (3, 4)} <= forms


@pytest.mark.parametrize("kind", ["sums", "pow2"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_burst_integer_cases_are_bit_exact(lib, N, K, kind):
    """Inputs whose projection is exact in fp32 and bf16: every output bit for bit, at 1..4 rows."""
    for M in (1, 2, 3, 4):
        _plan(lib, M, N, K)
        p, expect = _exact_case(kind, M, N, K, seed=5000 + 7 * M + N + K + (kind == "pow2"))
        y = run(lib, p, "qmv")
        assert np.array_equal(y, expect), f"M={M}"


@pytest.mark.parametrize("N,K", SHAPES)
def test_burst_random_cases_match_oracle(lib, N, K):
    for M in (1, 2, 3, 4):
        p = synth.random_problem(600 + M + N % 97, M, N, K)
        y = run(lib, p, "qmv")
        assert_parity(y, p)
        assert np.array_equal(run(lib, p, "qmv"), y), "repeat run differs"


@pytest.mark.parametrize("M,N,K", [(4, 1000, 2560), (1, 40, 10240), (3, 17, 128), (1, 1001, 2560), (2, 9728, 9728),
                                   (4, 3000, 2560)])
def test_burst_writes_only_its_output(lib, M, N, K):
    """A sentinel row above and below y: untouched, and every element of y written."""
    import torch
    p = synth.random_problem(M * 13 + N, M, N, K)
    _plan(lib, M, N, K)
    x, wq, s, b = to_device(p)
    big = bf16_from_bits(np.full((M + 2, N), SENTINEL, dtype=np.uint16))
    y = big[1:M + 1]
    announce(f"burst guard M={M} N={N} K={K}")
    lib.qmv_w4a16(x, wq, s, b, y=y)
    torch.cuda.synchronize()
    out = bits(big)
    assert np.all(out[0] == SENTINEL) and np.all(out[-1] == SENTINEL), "write outside [M, N]"
    assert not np.any(out[1:-1] == SENTINEL), "element of y left unwritten"
    assert_parity(out[1:-1], p)


def test_burst_calls_in_a_graph_replay(lib):
    """Captured burst calls (the packed form at one row, the 16-column form at four, the
    width-generic form at 3 bits) replay like the eager calls; replays alternate with eager work
    on the same outputs."""
    import torch
    cases = [(1, 2600, 2560, 4), (4, 4000, 2560, 4), (2, 1000, 2560, 3)]
    probs = [synth.random_problem(700 + i, M, N, K, bits=nb) for i, (M, N, K, nb) in enumerate(cases)]
    devs = [to_device(p) for p in probs]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0") for M, N, _, _ in cases]
    announce("burst graph replay")

    def calls():
        for (M, N, K, nb), d, y in zip(cases, devs, ys):
            if nb == 4:
                lib.qmv_w4a16(*d, y=y)
            else:
                lib.qmv_affine(*d, nb, y=y, mode=lib.QMV_BURST)

    calls()
    torch.cuda.synchronize()
    refs = [bits(y) for y in ys]
    assert lib.w4a16_plan(1, 2600, 2560, 128, lib.PATH_QMV)["tile_n"] == 4
    assert lib.w4a16_plan(4, 4000, 2560, 128, lib.PATH_QMV)["tile_n"] == 16
    for p, r in zip(probs[:2], refs[:2]):
        assert_parity(r, p)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            calls()
    torch.cuda.synchronize()
    for i in range(3):
        for y in ys:
            y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for y, r in zip(ys, refs):
            assert np.array_equal(bits(y), r), f"replay {i}"
        calls()                                            # eager, same outputs
        torch.cuda.synchronize()
        for y, r in zip(ys, refs):
            assert np.array_equal(bits(y), r), f"eager call after replay {i}"


# 5 to 8 rows: the 16-column form with 8 row slots (below 1024 column blocks, up to 64 groups)
ROWS8_SHAPES = [(96, 128), (33, 640), (9728, 2560), (200, 8192), (1000, 4096)]


@pytest.mark.parametrize("kind", ["sums", "pow2"])
@pytest.mark.parametrize("N,K", ROWS8_SHAPES)
def test_burst_eight_row_slots_integer_cases_are_bit_exact(lib, N, K, kind):
    for M in (5, 6, 7, 8):
        p = lib.w4a16_plan(M, N, K, 128, lib.PATH_QMV)
        assert p["variant"] == BURST and p["tile_n"] == 16, p
        case, expect = _exact_case(kind, M, N, K, seed=5600 + 7 * M + N + K + (kind == "pow2"))
        assert np.array_equal(run(lib, case, "qmv"), expect), f"M={M}"


@pytest.mark.parametrize("N,K", ROWS8_SHAPES)
def test_burst_eight_row_slots_match_oracle(lib, N, K):
    for M in (5, 8):
        p = synth.random_problem(640 + M + N % 89, M, N, K)
        assert_parity(run(lib, p, "qmv"), p)
