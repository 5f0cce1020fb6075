"""GPU parity of the burst matvec (4-bit, up to four decode rows; every wave issues all of its
loads at once) through the C ABI: each wave and group count the policy gives it (1 to 16 waves,
1 to 5 groups each), integer inputs bit for bit, random inputs against the CPU oracle within the
tolerance of ``O.check``, and sentinel rows around the output that no write may touch.
"""

import numpy as np
import pytest

from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bf16_from_bits, bits, to_device
from test_gpu_parity import SENTINEL, _exact_case, assert_parity, run

pytestmark = pytest.mark.gpu

BURST = 4   # the plan's instance index of the burst kernel

# (N, K) and what the plan makes of it at 1..4 rows
SHAPES = [
    (96, 128),      # one group: a single wave
    (33, 640),      # five groups over three waves (2, 2, 1), ragged N
    (160, 2560),    # 20 groups: ten waves of two
    (9728, 2560),   # 608 column blocks: ten waves of two
    (200, 8192),    # 64 groups: sixteen waves of four
    (300, 9728),    # 76 groups: fifteen waves of five and one of one
    (50, 10240),    # 80 groups: sixteen waves of five, the largest share
    (24600, 384),   # 1538 column blocks: one wave of three groups
    (32744, 1280),  # 2047 column blocks, the last ragged: four waves of three (the last of one)
]


@pytest.mark.parametrize("kind", ["sums", "pow2"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_burst_integer_cases_are_bit_exact(lib, N, K, kind):
    """Inputs whose projection is exact in fp32 and bf16: every output bit for bit, at 1..4 rows."""
    for M in (1, 2, 3, 4):
        assert lib.w4a16_plan(M, N, K, 128, lib.PATH_QMV)["variant"] == BURST
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


@pytest.mark.parametrize("M,N,K", [(4, 1000, 2560), (1, 40, 10240), (3, 17, 128)])
def test_burst_writes_only_its_output(lib, M, N, K):
    """A sentinel row above and below y: untouched, and every element of y written."""
    import torch
    p = synth.random_problem(M * 13 + N, M, N, K)
    assert lib.w4a16_plan(M, N, K, 128, lib.PATH_QMV)["variant"] == BURST
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
