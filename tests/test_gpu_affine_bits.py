"""GPU parity of the width-generic affine matvec (``qmv_affine``: 1, 2, 3, 4 and 8 bits per code,
M <= 8) against the oracle, through the C ABI.

The kernels (row-amortized, per-row and the burst form) and the policy are checked at every width
on ragged shapes (N not a multiple of the 16-column block, group counts not a multiple of the
four waves that split K), with the same per-element tolerance as the 4-bit paths.  Closed-form cases are
bit-exact: one-hot activations return the codes themselves (so the unpack order is pinned
position by position), and integer or power-of-two affine sums are exact in fp32.
"""

import ctypes

import numpy as np
import pytest

import oracle as O
from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bits as to_bits, to_device

pytestmark = pytest.mark.gpu

WIDTHS = (1, 2, 3, 4, 8)
MODES = {"policy": 0, "amortized": 1, "per_row": 2, "burst": 4}


def burst_applies(M, N, K):
    """Shapes of the burst forms: packed at most 4 rows, below 2048 column blocks of 16 and 128
    groups, beyond 160 blocks or 64 groups only up to 2 rows; 16 columns at 3 to 8 rows below
    1024 blocks, up to 80 groups at 3-4 rows and 64 at 5-8."""
    blocks, G = -(-N // 16), K // 128
    packed = M <= 4 and blocks < 2048 and G <= 128 and (M <= 2 or (blocks <= 160 and G <= 64))
    return packed or (3 <= M <= 8 and blocks < 1024 and G <= (80 if M <= 4 else 64))


def run_affine(lib, p, nbits, mode, dev=None):
    import torch
    announce(f"qmv_affine bits={nbits} mode={mode} M={p['M']} N={p['N']} K={p['K']}")
    x, wq, s, b = dev if dev is not None else to_device(p)
    y = lib.qmv_affine(x, wq, s, b, nbits, mode=MODES[mode])
    torch.cuda.synchronize()
    return to_bits(y)


def assert_parity(y_bits, p, nbits):
    y_ref, A = O.reference(p["x"], p["wq"], p["scales"], p["biases"], bits=nbits)
    r = O.check(y_bits, y_ref, A)
    assert r.ok, str(r)


AFFINE_CASES = [          # (M, N, K): ragged N; G = 2, 3, 20, 76, 128 groups
    (1, 1000, 256),
    (2, 4000, 2560),
    (1, 24600, 384),
    (5, 1000, 384),
    (8, 2056, 2560),
    (4, 150, 2560),          # burst form with 4-row slots
    (3, 1001, 8192),         # 64 groups at 3 rows: sixteen burst waves
    (2, 2560, 9728),         # 76 groups: two burst steps per wave
    (1, 502, 16384),         # 128 groups: the burst form's largest
    (1, 3, 640),             # fewer columns than one burst workgroup
    (4, 3000, 2560),         # 16-column burst form, 4 row slots
    (7, 2056, 8192),         # 16-column burst form, 8 row slots, 64 groups
]


@pytest.mark.parametrize("nbits", WIDTHS)
@pytest.mark.parametrize("M,N,K", AFFINE_CASES)
def test_affine_matches_oracle(lib, nbits, M, N, K):
    p = synth.random_problem(40 + nbits, M, N, K, bits=nbits)
    dev = to_device(p)
    modes = ["policy", "amortized"] + (["per_row"] if M <= 2 else []) + (["burst"] if burst_applies(M, N, K) else [])
    for mode in modes:
        assert_parity(run_affine(lib, p, nbits, mode, dev), p, nbits)


def one_hot_problem(nbits, K=256, N=40, seed=11):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 2 ** nbits, (N, K))
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))
    G = K // 128
    return q, {"x": x, "wq": synth.pack_codes(q, nbits), "scales": synth.const_bf16(1.0, (N, G)),
               "biases": synth.const_bf16(0.0, (N, G)), "M": K, "N": N, "K": K}


@pytest.mark.parametrize("nbits", WIDTHS)
@pytest.mark.parametrize("mode,rows", [("amortized", 8), ("per_row", 2), ("burst", 4), ("burst", 8)])
def test_one_hot_rows_return_the_codes(lib, nbits, mode, rows):
    import torch
    q, p = one_hot_problem(nbits)
    expect = synth.to_bf16_bits(q.T.astype(np.float32))
    x, wq, s, b = to_device(p)
    announce(f"qmv_affine one-hot bits={nbits} mode={mode}")
    for r0 in range(0, p["K"], rows):
        y = lib.qmv_affine(x[r0:r0 + rows], wq, s, b, nbits, mode=MODES[mode])
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(y), expect[r0:r0 + rows]), f"bits={nbits} rows {r0}..{r0 + rows - 1}"


@pytest.mark.parametrize("nbits", WIDTHS)
@pytest.mark.parametrize("mode,M,N", [("amortized", 8, 1000), ("amortized", 3, 1000), ("per_row", 2, 1000),
                                      ("per_row", 1, 1000), ("burst", 1, 1000), ("burst", 2, 1000), ("burst", 4, 1000),
                                      ("burst", 4, 3000), ("burst", 7, 1000)])      # packed; 16 columns at 3000 / 7 rows
def test_integer_sums_are_exact(lib, nbits, mode, M, N):
    rng = np.random.default_rng(12 + nbits)
    K = 640
    q = rng.integers(0, 2 ** nbits, (N, K))
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):
        xi[m, rng.choice(K, size=rng.integers(0, 40), replace=False)] = 1
    G = K // 128
    p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q, nbits),
         "scales": synth.const_bf16(1.0, (N, G)), "biases": synth.const_bf16(0.0, (N, G)), "M": M, "N": N, "K": K}
    # the sums are integers below 2^24: exact in fp32, then one bf16 rounding on both sides
    assert np.array_equal(run_affine(lib, p, nbits, mode), synth.to_bf16_bits((xi @ q.T).astype(np.float32)))


@pytest.mark.parametrize("nbits", WIDTHS)
@pytest.mark.parametrize("mode,M,N", [("amortized", 6, 520), ("per_row", 2, 520), ("burst", 3, 520),
                                      ("burst", 3, 4000), ("burst", 6, 520)])
def test_power_of_two_affine_is_exact(lib, nbits, mode, M, N):
    rng = np.random.default_rng(20 + nbits)
    K = 384
    half = 2 ** (nbits - 1)
    q = rng.integers(0, 2 ** nbits, (N, K))
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):                # 24 entries of +-1: |sum x (q - half)| <= 24 * 128
        idx = rng.choice(K, size=24, replace=False)
        xi[m, idx] = rng.choice([-1, 1], size=24)
    G = K // 128
    p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q, nbits),
         "scales": synth.const_bf16(2.0 ** -6, (N, G)), "biases": synth.const_bf16(-half * 2.0 ** -6, (N, G)),
         "M": M, "N": N, "K": K}
    # s * P and b * X are exact multiples of 2^-6 far below 2^24 * 2^-6: the fp32 result is exact
    expect = synth.to_bf16_bits(((xi @ (q - half).T) / 64.0).astype(np.float32))
    assert np.array_equal(run_affine(lib, p, nbits, mode), expect)


SENTINEL = 0x7FA5     # a NaN pattern the kernels never produce


@pytest.mark.parametrize("nbits", WIDTHS)
@pytest.mark.parametrize("mode,M", [("amortized", 3), ("per_row", 1), ("burst", 1), ("burst", 4), ("burst", 8)])
def test_writes_stay_inside_the_output(lib, nbits, mode, M):
    """y is the head of a larger poisoned buffer: the M x N outputs are written, nothing after."""
    import torch
    from w4a16_group_quantized_qmv_amd import load
    N, K = 37, 256
    p = synth.random_problem(60 + nbits, M, N, K, bits=nbits)
    x, wq, s, b = to_device(p)
    guard = 4096
    buf = torch.full((M * N + guard,), SENTINEL, dtype=torch.int16, device="cuda:0")
    announce(f"qmv_affine guard bits={nbits} mode={mode} M={M} N={N}")
    st = load().qmv_affine(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), buf.data_ptr(), M, N, K, 128,
                           nbits, MODES[mode], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    out = buf.cpu().numpy().view(np.uint16)
    assert np.all(out[M * N:] == SENTINEL)
    assert_parity(out[:M * N].reshape(M, N), p, nbits)


def test_four_bit_affine_and_the_w4a16_matvec_agree(lib):
    """At 4 bits both entry points compute the same projection, each within the tolerance."""
    import torch
    p = synth.random_problem(70, 4, 3000, 2560)
    dev = to_device(p)
    announce("qmv_affine vs qmv_w4a16")
    y_affine = to_bits(lib.qmv_affine(*dev, 4, mode=MODES["amortized"]))
    y_w4 = to_bits(lib.qmv_w4a16(*dev))
    torch.cuda.synchronize()
    assert_parity(y_affine, p, 4)
    assert_parity(y_w4, p, 4)
