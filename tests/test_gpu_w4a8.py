"""GPU parity of the W4A8 path (int8 activations on the int8 matrix cores) through the C ABI.

Bar:
* the activation quantizer is integer / byte work: codes, row scales and group sums are compared
  bit-exactly with the oracle's per-row int8 quantizer (the codes after undoing the documented
  operand order k0 k2 k4 k6 k1 k3 k5 k7 of every run of 8);
* closed-form projections (scale 1 / bias 0, power-of-two affine, bias only) with one-hot rows
  of 127 are bit-exact: the kernel's fp32 result is an exact integer multiple, rounded once;
* random projections are within the per-element tolerance
  ``|y - y_ref| <= 2^-8 |y_ref| + 2^-10 sum_k |sx xq w|`` of the oracle's W4A8 reference.
"""

import numpy as np
import pytest

import oracle as O
from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bf16_from_bits, bits, to_device

pytestmark = pytest.mark.gpu


def unpermute_codes(xq: np.ndarray) -> np.ndarray:
    """Stored xq (runs of 8 as k0 k2 k4 k6 k1 k3 k5 k7) -> natural order."""
    M, K = xq.shape
    runs = xq.reshape(M, K // 8, 8)
    out = np.empty_like(runs)
    out[:, :, 0::2] = runs[:, :, 0:4]
    out[:, :, 1::2] = runs[:, :, 4:8]
    return out.reshape(M, K)


def quantize_on_gpu(lib, x_bits):
    import torch
    announce(f"w4a8_quantize_rows M={x_bits.shape[0]} K={x_bits.shape[1]}")
    xq, sx, xsum = lib.w4a8_quantize_rows(bf16_from_bits(x_bits))
    torch.cuda.synchronize()
    return (xq.cpu().numpy(), sx.cpu().numpy(), xsum.view(torch.int16).cpu().numpy().view(np.uint16))


def check_quantizer(lib, x_bits):
    xq, sx, xsum = quantize_on_gpu(lib, x_bits)
    ref_q, ref_s = O.quantize_rows_int8(x_bits)
    assert np.array_equal(sx.view(np.uint32), ref_s.view(np.uint32)), "row scales differ"
    assert np.array_equal(unpermute_codes(xq), ref_q), "int8 codes differ"
    M, K = x_bits.shape
    G = K // 128
    halves = O.bf16_to_f64(xsum)
    X = ref_q.astype(np.int64).reshape(M, G, 128).sum(axis=2)
    hi, lo = halves[:, 0:2 * G:2], halves[:, 1:2 * G:2]
    assert np.array_equal(hi + lo, X.astype(np.float64)), "group sums differ"
    assert np.all(np.mod(hi, 128) == 0) and np.all((lo >= 0) & (lo <= 127))
    assert np.all(xsum[:, 2 * G:] == 0), "padding of xsum must be zero"


@pytest.mark.parametrize("M,K", [(33, 256), (5, 1152), (509, 2560), (3, 9728)])
def test_quantizer_is_bit_exact(lib, M, K):
    check_quantizer(lib, synth.random_problem(7, M, 16, K)["x"])


def test_quantizer_ties_zero_row_and_extremes(lib):
    # row 0: absmax 127 gives inv = 1, so the halves 2.5, 3.5, -0.5, -1.5 round to even
    # row 1: all zeros (inv = sx = 0)
    # row 2: one huge element dominates; small ones round to 0
    # row 3: absmax 1 (inv = 127), values on an exact grid
    K = 256
    rows = np.zeros((4, K), dtype=np.float32)
    rows[0, :6] = [127.0, 2.5, 3.5, -0.5, -1.5, -127.0]
    rows[2, 0], rows[2, 1:9] = 3.0e4, 1.0
    rows[3, :5] = [1.0, -1.0, 0.5, -0.25, 0.125]
    check_quantizer(lib, synth.to_bf16_bits(rows))


def run_w4a8(lib, p, split_k=0, one_call=False):
    import torch
    announce(f"w4a8 M={p['M']} N={p['N']} K={p['K']} split={split_k} one_call={one_call}")
    x, wq, s, b = to_device(p)
    if one_call:
        y = lib.w4a8_linear(x, wq, s, b)
    else:
        xq, sx, xsum = lib.w4a8_quantize_rows(x)
        y = lib.qmm_w4a8(xq, sx, xsum, wq, s, b, split_k=split_k)
    torch.cuda.synchronize()
    return bits(y)


def assert_w4a8_parity(y_bits, p, rows=None):
    xr = p["x"] if rows is None else p["x"][rows]
    y_ref, A = O.reference_w4a8(xr, p["wq"], p["scales"], p["biases"])
    got = y_bits if rows is None else y_bits[rows]
    r = O.check(got, y_ref, A)
    assert r.ok, str(r)
    return r


# ---------------------------------------------------------------------------------- closed forms

def one_hot_rows(K, value=127.0):
    return np.where(np.eye(K, dtype=bool), synth.const_bf16(value, (K, K)), np.uint16(0))


@pytest.mark.parametrize("split", [1, 2])
def test_identity_codes_are_bit_exact(lib, split):
    # s = 1, b = 0 and x = 127 I: sx = 1, xq = x, so y[k, n] = bf16(127 q[n, k]) exactly
    K, N = 256, 96
    q = np.random.default_rng(11).integers(0, 16, (N, K))
    G = K // 128
    p = {"x": one_hot_rows(K), "wq": synth.pack_codes(q), "scales": synth.const_bf16(1.0, (N, G)),
         "biases": synth.const_bf16(0.0, (N, G)), "M": K, "N": N, "K": K}
    y = run_w4a8(lib, p, split)
    assert np.array_equal(y, synth.to_bf16_bits((127.0 * q.T).astype(np.float32))), "int8 path indexing mismatch"


def test_power_of_two_affine_is_bit_exact(lib):
    # s = 2^-6, b = -8 * 2^-6: w = (q - 8) / 64, so y[k, n] = bf16(127 (q[n, k] - 8) / 64) exactly
    K, N = 384, 160
    q = np.random.default_rng(12).integers(0, 16, (N, K))
    G = K // 128
    p = {"x": one_hot_rows(K), "wq": synth.pack_codes(q), "scales": synth.const_bf16(2.0 ** -6, (N, G)),
         "biases": synth.const_bf16(-8.0 * 2.0 ** -6, (N, G)), "M": K, "N": N, "K": K}
    y = run_w4a8(lib, p, 1)
    expect = synth.to_bf16_bits((127.0 * (q.T - 8) / 64.0).astype(np.float32))
    assert np.array_equal(y, expect)


def test_bias_term_closed_form(lib):
    # s = 0 (every code contributes nothing), per-group biases b[n, g] = (n % 7 - 3) / 4 and x rows
    # on the int8 grid with absmax 127: y = sum_g b[n, g] X[m, g] exactly (small integers / 4)
    K, N, M = 2560, 130, 40
    G = K // 128
    rng = np.random.default_rng(13)
    xv = rng.integers(-3, 4, (M, K)).astype(np.float32)
    xv[:, 0] = 127.0
    bias = ((np.arange(N)[:, None] % 7 - 3) / 4.0 + 0 * np.arange(G)[None, :]).astype(np.float32)
    bias[:, 1::2] *= -1
    p = {"x": synth.to_bf16_bits(xv), "wq": synth.pack_codes(rng.integers(0, 16, (N, K))),
         "scales": synth.const_bf16(0.0, (N, G)), "biases": synth.to_bf16_bits(bias), "M": M, "N": N, "K": K}
    y = run_w4a8(lib, p, 1)
    X = xv.reshape(M, G, 128).sum(axis=2)
    expect = synth.to_bf16_bits((X @ bias.T).astype(np.float32))
    assert np.array_equal(y, expect)


# ---------------------------------------------------------------------------------- random parity

@pytest.mark.parametrize("split", [0, 1, 2])
def test_tiny_config(lib, split):
    p = synth.problem(1, "tiny")                  # M=33, K=256, N=96: ragged in M and N
    assert_w4a8_parity(run_w4a8(lib, p, split), p)


@pytest.mark.parametrize("M,N,K,split", [
    (1, 96, 256, 0), (8, 200, 1152, 0), (31, 130, 2560, 0), (64, 1024, 2560, 3), (100, 257, 4096, 0),
    (129, 384, 1280, 5), (300, 1000, 2560, 0),
    (250, 9728, 384, 0), (90, 40000, 256, 0)])     # wide grids: ragged rows, ragged columns
def test_random_shapes(lib, M, N, K, split):
    p = synth.random_problem(21, M, N, K)
    assert_w4a8_parity(run_w4a8(lib, p, split), p)


@pytest.mark.parametrize("shape,M", [("q", 128), ("k", 512), ("o", 509), ("down", 512), ("gate", 128)])
def test_prefill_shapes_sampled_rows(lib, shape, M):
    # 128- and 512-token prefill projections (M = 509: ragged tiles; down: K = 9728, split-K)
    cfg = 3 if M == 128 else 4
    p = synth.problem(cfg, shape, M)
    y = run_w4a8(lib, p)
    rows = np.unique(np.r_[0, 1, 31, 32, 63, 64, M // 2, M - 2, M - 1])
    assert_w4a8_parity(y, p, rows)


def test_long_prefill_gate_sampled_rows(lib):
    p = synth.problem(5, "gate", 4096)
    y = run_w4a8(lib, p)
    assert_w4a8_parity(y, p, np.r_[0, 127, 128, 2047, 4094, 4095])


def test_one_call_matches_two_calls_and_is_deterministic(lib):
    p = synth.random_problem(22, 200, 640, 2560)
    a = run_w4a8(lib, p, one_call=True)
    assert np.array_equal(a, run_w4a8(lib, p, 0))
    assert np.array_equal(a, run_w4a8(lib, p, one_call=True))
    assert_w4a8_parity(a, p)


def test_forced_split_without_workspace_is_rejected(lib):
    import torch
    p = synth.random_problem(23, 64, 256, 2560)
    x, wq, s, b = to_device(p)
    xq, sx, xsum = lib.w4a8_quantize_rows(x)
    y = torch.empty((64, 256), dtype=torch.bfloat16, device=x.device)
    st = lib.load().qmm_w4a8(xq.data_ptr(), sx.data_ptr(), xsum.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(),
                             y.data_ptr(), 64, 256, 2560, 128, 4, None, 0, None)
    assert st == 5
    short = torch.empty(16, dtype=torch.float32, device=x.device)
    with pytest.raises(ValueError):
        lib.w4a8_linear(x, wq, s, b, workspace=short)
