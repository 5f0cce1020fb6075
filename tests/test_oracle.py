"""Pins for the CPU oracle (``-m "not gpu"``).

Each test fixes the oracle to something other than itself: a library routine
(torch's bf16 conversions), a closed form (identity activations, all-zero
codes, power-of-two affine parameters, a rational worked example), an exact
brute force on tiny inputs, a mathematical bound (the quantization round
trip) or an invariant (scaling by 2).  ``test_pins_catch_planted_mistakes``
plants plausible mistakes in copies of the oracle and shows that every one of
them fails at least one pin.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from w4a16_group_quantized_qmv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_w4g128.json")


# ----------------------------------------------------------------------------- bf16 conversions

def test_bf16_widening_matches_torch_on_every_pattern():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _rne_cases():
    rng = np.random.default_rng(7)
    r = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0) ** rng.integers(-40, 40, 200000).astype(np.float32)
    u = rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)  # exact halfway cases
    edge = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45,
                     1.1754942e-38, np.inf, -np.inf], dtype=np.float32)
    near_max = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0xFF7F8000], dtype=np.uint32).view(np.float32)
    allv = np.concatenate([r, u.view(np.float32), ties, edge, near_max])
    return allv[~np.isnan(allv)]


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    v = _rne_cases()
    ours = O.f32_to_bf16_rne(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_of_nan_is_quiet_nan():
    v = np.array([np.nan, -np.nan], dtype=np.float32)
    out = O.f32_to_bf16_rne(v)
    assert np.all(np.isnan(O.bf16_to_f32(out)))


def test_generator_rounding_agrees_with_oracle_rounding():
    v = _rne_cases()
    v = v[np.isfinite(v)]
    assert np.array_equal(synth.to_bf16_bits(v), O.f32_to_bf16_rne(v))


# ----------------------------------------------------------------------------- unpacking

def test_nibble_order_literal_words():
    # element 8j+i of a row is bits 4i..4i+3 of word j: the hex digits read right to left
    words = np.array([[0x76543210, 0xFEDCBA98, 0x0000000F, 0xF0000000]], dtype=np.uint32)
    q = O.unpack_q(words, 32)
    assert q[0, :8].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    assert q[0, 8:16].tolist() == [8, 9, 10, 11, 12, 13, 14, 15]
    assert q[0, 16:24].tolist() == [15, 0, 0, 0, 0, 0, 0, 0]
    assert q[0, 24:32].tolist() == [0, 0, 0, 0, 0, 0, 0, 15]


def test_unpack_inverts_the_generator_packer():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, (37, 256)).astype(np.uint8)
    assert np.array_equal(O.unpack_q(synth.pack_codes(q), 256), q)
    assert np.array_equal(O.pack_q(q), synth.pack_codes(q))


# ----------------------------------------------------------------------------- closed forms (pin battery)

def _load_golden():
    with open(GOLDEN) as f:
        d = json.load(f)
    arr = {k: np.array(d[k]) for k in ("x_bf16", "scales_bf16", "biases_bf16")}
    wq = np.array(d["wq_u32"], dtype=np.uint64).astype(np.uint32)
    y = [[Fraction(v) for v in row] for row in d["y_exact"]]
    A = [[Fraction(v) for v in row] for row in d["abs_mass_exact"]]
    return (arr["x_bf16"].astype(np.uint16), wq, arr["scales_bf16"].astype(np.uint16),
            arr["biases_bf16"].astype(np.uint16), y, A, np.array(d["codes"]))


def pin_worked_example(ref_fn):
    """Rational worked example: every value is dyadic and every sum exact in fp64."""
    x, wq, s, b, y_exact, A_exact, _ = _load_golden()
    y, A = ref_fn(x, wq, s, b)
    ok_y = all(Fraction(float(y[m, n])) == y_exact[m][n] for m in range(y.shape[0]) for n in range(y.shape[1]))
    ok_A = all(Fraction(float(A[m, n])) == A_exact[m][n] for m in range(A.shape[0]) for n in range(A.shape[1]))
    return ok_y and ok_A


def pin_identity(ref_fn):
    """x = identity, s = 1, b = 0: y[m, n] = q[n, m] exactly."""
    rng = np.random.default_rng(11)
    K, N = 256, 40
    q = rng.integers(0, 16, (N, K))
    wq = synth.pack_codes(q)
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))
    y, _ = ref_fn(x, wq, synth.const_bf16(1.0, (N, K // 128)), synth.const_bf16(0.0, (N, K // 128)))
    return np.array_equal(y, q.T.astype(np.float64))


def pin_all_zero_codes(ref_fn):
    """q = 0 everywhere: y[m, n] = sum_g b[n, g] * sum_{k in g} x[m, k]."""
    rng = np.random.default_rng(12)
    M, K, N = 5, 384, 7
    G = K // 128
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    s = synth.to_bf16_bits(rng.uniform(0.001, 0.01, (N, G)).astype(np.float32))
    b = synth.to_bf16_bits(rng.standard_normal((N, G)).astype(np.float32))
    wq = np.zeros((N, K // 8), dtype=np.uint32)
    y, A = ref_fn(x, wq, s, b)
    xf = synth.from_bf16_bits(x).astype(np.float64)
    bf = synth.from_bf16_bits(b).astype(np.float64)
    ok = True
    for m in range(M):
        for n in range(N):
            terms = [bf[n, g] * xf[m, k] for g in range(G) for k in range(128 * g, 128 * (g + 1))]
            exact = math.fsum(terms)
            ok &= abs(y[m, n] - exact) <= 2.0 ** -45 * math.fsum(abs(t) for t in terms)
            ok &= abs(A[m, n] - math.fsum(abs(t) for t in terms)) <= 2.0 ** -45 * A[m, n]
    return bool(ok)


def pin_power_of_two_affine(ref_fn):
    """s = 2^-6, b = -8 * 2^-6 gives w = (q - 8) / 64; integer x makes y an exact multiple of 1/64."""
    rng = np.random.default_rng(13)
    M, K, N = 6, 256, 9
    q = rng.integers(0, 16, (N, K))
    xi = rng.integers(-4, 5, (M, K))
    x = synth.to_bf16_bits(xi.astype(np.float32))
    G = K // 128
    y, _ = ref_fn(x, synth.pack_codes(q), synth.const_bf16(2.0 ** -6, (N, G)), synth.const_bf16(-8 * 2.0 ** -6, (N, G)))
    exact = (xi @ (q - 8).T) / 64.0
    return np.array_equal(y, exact)


def pin_group_scales_differ(ref_fn):
    """Each group has its own scale: one-hot x at k picks column k's group scale."""
    K, N = 512, 3
    G = K // 128
    q = np.ones((N, K), dtype=np.int64)
    s_vals = np.array([[2.0 ** -(g + 1 + n) for g in range(G)] for n in range(N)], dtype=np.float32)
    b_vals = np.array([[(g + 1) * 2.0 ** -3 * (n + 1) for g in range(G)] for n in range(N)], dtype=np.float32)
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))
    y, _ = ref_fn(x, synth.pack_codes(q), synth.to_bf16_bits(s_vals), synth.to_bf16_bits(b_vals))
    expect = np.array([[s_vals[n, k // 128] + b_vals[n, k // 128] for n in range(N)] for k in range(K)], dtype=np.float64)
    return np.array_equal(y, expect)


def pin_fp32_dequant(ref_fn):
    """Dequantization keeps fp32 precision (reading R4): with x = identity, y = w exactly, and the
    chosen s*q + b needs up to 18 significand bits: exact in fp32, not representable in bf16."""
    K, N = 256, 6
    G = K // 128
    rng = np.random.default_rng(14)
    q = rng.integers(0, 16, (N, K))
    s_vals = np.array([[1 + 2.0 ** -7 * (1 + n + g) for g in range(G)] for n in range(N)], dtype=np.float32)
    b_vals = np.array([[2.0 ** -10 * (2 * n + 1) * (g + 1) for g in range(G)] for n in range(N)], dtype=np.float32)
    s_bits, b_bits = synth.to_bf16_bits(s_vals), synth.to_bf16_bits(b_vals)
    assert np.array_equal(synth.from_bf16_bits(s_bits), s_vals) and np.array_equal(synth.from_bf16_bits(b_bits), b_vals)
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))
    y, _ = ref_fn(x, synth.pack_codes(q), s_bits, b_bits)
    expect = [[Fraction(float(s_vals[n, k // 128])) * int(q[n, k]) + Fraction(float(b_vals[n, k // 128]))
               for n in range(N)] for k in range(K)]
    return all(Fraction(float(y[k, n])) == expect[k][n] for k in range(K) for n in range(N))


PIN_BATTERY = [pin_worked_example, pin_identity, pin_all_zero_codes, pin_power_of_two_affine, pin_group_scales_differ,
               pin_fp32_dequant]


def oracle_ref(x, wq, s, b):
    return O.reference(x, wq, s, b)


@pytest.mark.parametrize("pin", PIN_BATTERY, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(oracle_ref)


# ----------------------------------------------------------------------------- planted mistakes

def _mutant(kind):
    def unpack(wq, K):
        w = np.asarray(wq, dtype=np.uint32)
        q = np.empty((w.shape[0], K), dtype=np.uint8)
        for i in range(8):
            shift = 4 * (7 - i) if kind == "high_nibble_first" else 4 * i
            q[:, i::8] = (w >> np.uint32(shift)) & np.uint32(0xF)
        if kind == "codes_off_by_one_word":
            q = np.roll(q, 8, axis=1)
        return q

    def ref(x, wq, s, b):
        x64 = O.bf16_to_f64(x)
        K = x64.shape[1]
        q = unpack(wq, K).astype(np.float32)
        sf = O.bf16_to_f32(s)
        bf = O.bf16_to_f32(b)
        gk = np.arange(K) // 128
        if kind == "group_of_64":
            gk = np.minimum(np.arange(K) // 64, sf.shape[1] - 1)
        if kind == "group_index_modulo":
            gk = np.arange(K) % sf.shape[1]
        if kind == "first_group_only":
            gk = np.zeros(K, dtype=np.int64)
        sk, bk = sf[:, gk], bf[:, gk]
        if kind == "scale_bias_swapped":
            sk, bk = bk, sk
        w = np.multiply(sk, q, dtype=np.float32)
        if kind == "bias_dropped":
            pass
        elif kind == "bias_sign_flipped":
            w = w - bk
        else:
            w = w + bk
        if kind == "dequant_in_bf16":
            w = O.bf16_to_f32(O.f32_to_bf16_rne(w))
        if kind == "x_bits_read_as_fp16":
            x64 = np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
        w64 = w.astype(np.float64)
        if kind == "accumulate_fp32":
            y = (x64.astype(np.float32) @ w.T).astype(np.float64)
        elif kind == "k_reversed_for_x":
            y = x64[:, ::-1] @ w64.T
        else:
            y = x64 @ w64.T
        return y, np.abs(x64) @ np.abs(w64).T
    return ref


MUTANTS = ["high_nibble_first", "codes_off_by_one_word", "group_of_64", "group_index_modulo", "first_group_only",
           "scale_bias_swapped", "bias_dropped", "bias_sign_flipped", "dequant_in_bf16",
           "x_bits_read_as_fp16", "accumulate_fp32", "k_reversed_for_x"]


def test_mutation_harness_is_faithful():
    # the unmutated harness reproduces the oracle, so failures below come from the planted mistake
    x, wq, s, b, *_ = _load_golden()
    y0, A0 = O.reference(x, wq, s, b)
    y1, A1 = _mutant("none")(x, wq, s, b)
    assert np.array_equal(y0, y1) and np.array_equal(A0, A1)


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    failed = [p.__name__ for p in PIN_BATTERY if not p(_mutant(kind))]
    assert failed, f"planted mistake {kind!r} passed every pin"


# ----------------------------------------------------------------------------- brute force

def test_brute_force_tiny_config():
    """Brute force with exact products and fsum on the 33x256 -> 96 workload."""
    p = synth.problem(1, "tiny")
    y, A = O.reference(p["x"], p["wq"], p["scales"], p["biases"])
    yb, Ab = O.brute_force(p["x"], p["wq"], p["scales"], p["biases"])
    assert np.all(np.abs(y - yb) <= 2.0 ** -40 * Ab)
    assert np.all(np.abs(A - Ab) <= 2.0 ** -40 * Ab)


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (3, 128, 5), (2, 384, 3)])
def test_brute_force_ragged_small(M, K, N):
    p = synth.random_problem(100 + M * 7 + N, M, N, K)
    y, A = O.reference(p["x"], p["wq"], p["scales"], p["biases"])
    yb, Ab = O.brute_force(p["x"], p["wq"], p["scales"], p["biases"])
    assert np.all(np.abs(y - yb) <= 2.0 ** -40 * Ab)


def test_column_chunking_does_not_change_the_result():
    p = synth.random_problem(5, 4, 300, 256)
    y1, A1 = O.reference(p["x"], p["wq"], p["scales"], p["biases"], col_chunk=7)
    y2, A2 = O.reference(p["x"], p["wq"], p["scales"], p["biases"])
    assert np.array_equal(y1, y2) and np.array_equal(A1, A2)
    cols = np.array([299, 0, 17])
    y3, _ = O.reference(p["x"], p["wq"], p["scales"], p["biases"], columns=cols)
    assert np.array_equal(y3, y2[:, cols])


# ----------------------------------------------------------------------------- invariants

def test_scaling_by_two_is_exact():
    p = synth.random_problem(21, 7, 33, 256)
    x2 = synth.to_bf16_bits(2 * synth.from_bf16_bits(p["x"]))
    y1, _ = O.reference(p["x"], p["wq"], p["scales"], p["biases"])
    y2, _ = O.reference(x2, p["wq"], p["scales"], p["biases"])
    assert np.array_equal(y2, 2 * y1)


def test_first_rows_of_a_longer_draw_match():
    a = synth.activations(4, 0, 512, 2560)
    b = synth.activations(4, 0, 509, 2560)
    assert np.array_equal(a[:509], b)


# ----------------------------------------------------------------------------- quantizer

def test_quantizer_implementations_agree_bit_exactly():
    rng = np.random.default_rng(31)
    W = (0.02 * rng.standard_normal((24, 512))).astype(np.float32)
    W[3, :128] = 0.125            # degenerate group: scale 0
    W[5, 128:256] = -1.5          # degenerate group, negative
    W[7, :] *= 1e4                # large range
    W[8, :] *= 1e-30              # subnormal-range scales
    a = O.quantize_w4g128(W)
    b = synth.quantize(W)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _roundtrip_bound(W, s_bits, b_bits):
    G = s_bits.shape[1]
    Wg = W.reshape(W.shape[0], G, 128).astype(np.float64)
    mn, mx = Wg.min(axis=2), Wg.max(axis=2)
    s = O.bf16_to_f64(s_bits)
    mag = np.maximum(np.abs(mn), np.abs(mx))
    # s/2 from rounding to the nearest code; 2^-9 (|min| + (max-min)) covers the grid ends moved by
    # rounding s and b to bf16; 2^-20 (...) covers the fp32 roundings of (W - b) / s and of s*q + b.
    return s / 2 + 2.0 ** -9 * (np.abs(mn) + (mx - mn)) + 2.0 ** -20 * (mag + s)


@pytest.mark.parametrize("cfg,shape", [(1, "tiny"), (2, "decode0"), (3, "k"), (4, "down")])
def test_quantization_round_trip_bound(cfg, shape):
    idx = synth.shape_index(cfg, shape)
    _, K, N, _ = synth.CONFIGS[cfg]["runs"][idx]
    N = min(N, 512)
    W = np.float32(synth.W_STD) * synth.rng(cfg, idx, synth.ROLE_W, 0).standard_normal((N, K), dtype=np.float32)
    wq, s, b = synth.quantize(W)
    w_hat = O.dequant_f32(wq, s, b, K).astype(np.float64)
    err = np.abs(W.astype(np.float64) - w_hat).reshape(N, K // 128, 128)
    bound = _roundtrip_bound(W, s, b)[:, :, None]
    assert np.all(err <= bound)
    # and the plain scale/2 bound holds for the overwhelming majority of weights
    assert np.mean(err <= O.bf16_to_f64(s)[:, :, None] / 2 * (1 + 2.0 ** -18)) > 0.99


# ----------------------------------------------------------------------------- tolerance check

def test_check_accepts_inside_and_rejects_outside_the_bound():
    y_bits = synth.to_bf16_bits(np.array([[1.0, -2.0, 0.0, 4.0]], dtype=np.float32))
    y = synth.from_bf16_bits(y_bits).astype(np.float64)
    A = np.array([[10.0, 10.0, 10.0, 10.0]])
    bound = lambda yr: O.TOL_REL * np.abs(yr) + O.TOL_MASS * A
    # choose y_ref so that |y - y_ref| = 0.99 * bound (solve for a reference above y)
    d_in = 0.99 * O.TOL_MASS * A / (1 - 0.99 * O.TOL_REL) + 0.99 * O.TOL_REL * np.abs(y) / (1 - 0.99 * O.TOL_REL)
    assert O.check(y_bits, y + d_in, A).ok
    d_out = 1.01 * (O.TOL_MASS * A + O.TOL_REL * np.abs(y)) / (1 - 1.01 * O.TOL_REL)
    r = O.check(y_bits, y + d_out, A)
    assert not r.ok and r.n_bad == 4 and r.max_ratio > 1.0
    assert np.all(np.abs(y - (y + d_in)) <= bound(y + d_in))


def test_check_rejects_nan_and_inf():
    y_ref = np.zeros((1, 3))
    A = np.ones((1, 3))
    bits = np.array([[0x7FC0, 0x7F80, 0x0000]], dtype=np.uint16)
    r = O.check(bits, y_ref, A)
    assert not r.ok and r.n_bad == 2


def test_check_exact_zero_bound():
    y_ref = np.zeros((1, 2))
    A = np.zeros((1, 2))
    assert O.check(np.array([[0, 0x8000]], dtype=np.uint16), y_ref, A).ok   # +0 and -0
    assert not O.check(np.array([[0x0001, 0]], dtype=np.uint16), y_ref, A).ok


# ----------------------------------------------------------------------------- logits_to_keep

def test_keep_last_rows():
    assert O.keep_last_rows(10, 1) == slice(9, 10)
    assert O.keep_last_rows(10, 0) == slice(0, 10)
    assert O.keep_last_rows(10, 10) == slice(0, 10)
    for bad in (-1, 11):
        with pytest.raises(ValueError):
            O.keep_last_rows(10, bad)


# ----------------------------------------------------------------------------- SwiGLU

def test_silu_closed_forms():
    z = np.array([-30.0, -2.0, -0.5, 0.0, 0.5, 2.0, 30.0])
    s = O.silu_f64(z)
    assert s[3] == 0.0
    assert abs(s[-1] - 30.0) < 1e-11 and abs(s[0]) < 1e-11
    # silu(-z) = silu(z) - z
    assert np.allclose(O.silu_f64(-z), s - z, rtol=0, atol=1e-13)
    # sigmoid(0) = 1/2: derivative of silu at 0 is 1/2
    h = 1e-6
    assert abs((O.silu_f64(h) - O.silu_f64(-h)) / (2 * h) - 0.5) < 1e-9


def test_swiglu_reference_composes_two_projections():
    p = synth.random_problem(41, 3, 16, 256)
    q = synth.random_problem(42, 3, 16, 256)
    h, g, Ag, u, Au = O.swiglu_reference(p["x"], (p["wq"], p["scales"], p["biases"]), (q["wq"], q["scales"], q["biases"]))
    g2, _ = O.reference(p["x"], p["wq"], p["scales"], p["biases"])
    u2, _ = O.reference(p["x"], q["wq"], q["scales"], q["biases"])
    assert np.array_equal(g, g2) and np.array_equal(u, u2)
    assert np.allclose(h, g2 / (1 + np.exp(-g2)) * u2, rtol=1e-15, atol=0)
    # the fused check accepts the correctly rounded result and rejects a planted 3% error
    good = O.f32_to_bf16_rne(h.astype(np.float32))
    assert O.check_swiglu(good, g, Ag, u, Au).ok
    bad = O.f32_to_bf16_rne((h * 1.03 + 0.01).astype(np.float32))
    assert not O.check_swiglu(bad, g, Ag, u, Au).ok


# The SwiGLU bound is derived from R6 by error propagation.  It is pinned against a numerical
# exploration of what a correct fused kernel may return, not against a copy of its formula:
#   soundness  every result a kernel could legitimately produce -- gate and up sums anywhere in
#              their R6 boxes, SiLU and the product in fp32, one rounding to bf16 -- is accepted;
#   tightness  in a configuration where one term of the bound dominates, the bound (read back
#              from the check's own error ratio) is within 1.15x of the worst legitimate error (measured:
#              1.005-1.10x), so the bound sits at the edge of what a correct kernel can return.
# Planted mistakes (a looser tolerance, a dropped term, a smaller slope constant) each fail one.

SWIGLU_CASES = {
    # name: (g, u, A_g, A_u, tight)
    "gate_error_at_steepest_slope": (2.3994, 3.0, 512.0, 0.0, True),    # silu' peaks near z = 2.3994
    "up_error_at_large_gate": (20.0, 0.01, 0.0, 10.24, True),
    "both_errors_at_zero": (0.0, 0.0, 51200.0, 1.024, True),            # the cross term alone
    "rounding_only": (20.0, 1.0, 0.0, 0.0, False),
    "silu_minimum": (-1.2785, 4.0, 512.0, 0.0, False),                  # the global slope bound is loose here
    "saturated_negative_gate": (-30.0, 5.0, 64.0, 64.0, False),
}


def _f32(v):
    return np.float32(v)


def _legit_results(g, u, A_g, A_u, n=401):
    """bf16 results a correct kernel may return: g~, u~ on a grid of their R6 boxes (fp32), then
    silu(g~) * u~ in fp32 arithmetic and one round-to-nearest-even to bf16."""
    e_g = O.TOL_REL * abs(g) + O.TOL_MASS * A_g
    e_u = O.TOL_REL * abs(u) + O.TOL_MASS * A_u
    gg = np.linspace(g - e_g, g + e_g, n).astype(np.float32)
    out = []
    for ut in (u - e_u, u, u + e_u):
        ut32 = _f32(ut)
        with np.errstate(over="ignore"):
            silu = gg / (_f32(1) + np.exp(-gg))        # fp32 throughout
        out.append(O.f32_to_bf16_rne((silu * ut32).astype(np.float32)))
    return np.concatenate(out)


def _exact_h(g, u):
    return g / (1.0 + math.exp(-g)) * u if g > -700 else 0.0


def _bound_from_ratio(check_fn, g, u, A_g, A_u):
    """The check's bound at one element, read back from its own error ratio."""
    h_ref = _exact_h(g, u)
    probe = O.f32_to_bf16_rne(np.array([[h_ref + 1.0 + abs(h_ref)]], dtype=np.float32))
    err = abs(float(O.bf16_to_f64(probe)[0, 0]) - h_ref)
    r = check_fn(probe, np.array([[g]]), np.array([[A_g]]), np.array([[u]]), np.array([[A_u]]))
    return err / r.max_ratio


def _swiglu_pins(check_fn):
    """Names of the SwiGLU pins that ``check_fn`` fails (empty: it passes all)."""
    failed = []
    for name, (g, u, A_g, A_u, tight) in SWIGLU_CASES.items():
        legit = _legit_results(g, u, A_g, A_u)
        ones = np.ones((1, legit.size))
        r = check_fn(legit[None, :], g * ones, A_g * ones, u * ones, A_u * ones)
        if not r.ok:
            failed.append(f"sound:{name}")
        if tight:
            worst = float(np.max(np.abs(O.bf16_to_f64(legit) - _exact_h(g, u))))
            if _bound_from_ratio(check_fn, g, u, A_g, A_u) > 1.15 * worst:
                failed.append(f"tight:{name}")
    return failed


def test_check_swiglu_is_sound_and_tight():
    assert _swiglu_pins(O.check_swiglu) == []


def _swiglu_mutant(kind):
    def fn(h_bits, g_ref, A_g, u_ref, A_u):
        if kind == "tolerance_8x_looser":
            return O.check_swiglu(h_bits, g_ref, A_g, u_ref, A_u, rel=8 * O.TOL_REL, mass=8 * O.TOL_MASS)
        g_ref, u_ref = np.asarray(g_ref, np.float64), np.asarray(u_ref, np.float64)
        e_g = O.TOL_REL * np.abs(g_ref) + O.TOL_MASS * np.asarray(A_g, np.float64)
        e_u = O.TOL_REL * np.abs(u_ref) + O.TOL_MASS * np.asarray(A_u, np.float64)
        h_ref = O.silu_f64(g_ref) * u_ref
        slope = 1.0 if kind == "slope_bound_1" else 1.1
        t_g = slope * e_g * (np.abs(u_ref) + (0 if kind == "cross_term_dropped" else e_u))
        t_u = 0 if kind == "up_error_term_dropped" else np.abs(O.silu_f64(g_ref)) * e_u
        t_r = 0 if kind == "rounding_term_dropped" else O.TOL_REL * np.abs(h_ref)
        bound = t_g + t_u + t_r
        err = np.abs(O.bf16_to_f64(h_bits) - h_ref)
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err == 0, 0.0, np.inf))
        ok = bool(np.all(np.isfinite(err) & (err <= bound)))
        return O.CheckResult(ok, float(ratio.max()), (), int((err > bound).sum()), int(err.size))
    return fn


SWIGLU_MUTANTS = ["tolerance_8x_looser", "slope_bound_1", "cross_term_dropped", "up_error_term_dropped",
                  "rounding_term_dropped"]


def test_swiglu_mutant_copy_is_faithful_without_a_mistake():
    assert _swiglu_pins(_swiglu_mutant("none")) == []


@pytest.mark.parametrize("kind", SWIGLU_MUTANTS)
def test_swiglu_pins_catch_planted_mistakes(kind):
    assert _swiglu_pins(_swiglu_mutant(kind)), f"planted mistake {kind!r} passed every SwiGLU pin"


# ----------------------------------------------------------------------------- other code widths (R8)

def _load_golden_bits(bits):
    path = os.path.join(os.path.dirname(__file__), "golden", f"worked_example_w{bits}g128.json")
    with open(path) as f:
        d = json.load(f)
    assert d["bits"] == bits
    x = np.array(d["x_bf16"]).astype(np.uint16)
    wq = np.array(d["wq_u32"], dtype=np.uint64).astype(np.uint32)
    s = np.array(d["scales_bf16"]).astype(np.uint16)
    b = np.array(d["biases_bf16"]).astype(np.uint16)
    y = [[Fraction(v) for v in row] for row in d["y_exact"]]
    A = [[Fraction(v) for v in row] for row in d["abs_mass_exact"]]
    return x, wq, s, b, y, A, np.array(d["codes"])


def _bits_pin_worked_example(ref_fn, bits):
    x, wq, s, b, y_exact, A_exact, _ = _load_golden_bits(bits)
    try:
        y, A = ref_fn(x, wq, s, b, bits)
    except ValueError:
        return False
    return (all(Fraction(float(y[m, n])) == y_exact[m][n] for m in range(y.shape[0]) for n in range(y.shape[1]))
            and all(Fraction(float(A[m, n])) == A_exact[m][n] for m in range(A.shape[0]) for n in range(A.shape[1])))


def _bits_pin_identity(ref_fn, bits):
    """x = identity, s = 1, b = 0: y[m, n] = q[n, m] exactly."""
    rng = np.random.default_rng(40 + bits)
    K, N = 256, 24
    q = rng.integers(0, 1 << bits, (N, K))
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))
    try:
        y, _ = ref_fn(x, synth.pack_codes(q, bits), synth.const_bf16(1.0, (N, 2)), synth.const_bf16(0.0, (N, 2)), bits)
    except ValueError:
        return False
    return np.array_equal(y, q.T.astype(np.float64))


def _bits_pin_max_codes(ref_fn, bits):
    """Every code 2**bits - 1: y[m, n] = sum_g (s (2**bits - 1) + b) * sum_{k in g} x[m, k]."""
    rng = np.random.default_rng(50 + bits)
    M, K, N = 3, 384, 5
    G = K // 128
    q = np.full((N, K), (1 << bits) - 1)
    xi = rng.integers(-4, 5, (M, K))
    s = (2.0 ** -rng.integers(3, 8, (N, G))).astype(np.float32)
    b = (-(2.0 ** -rng.integers(2, 6, (N, G)))).astype(np.float32)
    try:
        y, _ = ref_fn(synth.to_bf16_bits(xi.astype(np.float32)), synth.pack_codes(q, bits), synth.to_bf16_bits(s),
                      synth.to_bf16_bits(b), bits)
    except ValueError:
        return False
    X = xi.reshape(M, G, 128).sum(axis=2).astype(np.float64)          # [M, G]
    expect = X @ (s.astype(np.float64) * ((1 << bits) - 1) + b.astype(np.float64)).T
    return np.array_equal(y, expect)


BITS_PINS = [_bits_pin_worked_example, _bits_pin_identity, _bits_pin_max_codes]


def _oracle_bits(x, wq, s, b, bits):
    return O.reference(x, wq, s, b, bits=bits)


@pytest.mark.parametrize("bits", [1, 2, 3, 8])
@pytest.mark.parametrize("pin", BITS_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_bits_pin(pin, bits):
    assert pin(_oracle_bits, bits)


def test_unpack_literal_words_other_widths():
    # 8-bit: bytes low first
    assert O.unpack_q(np.array([[0x04030201, 0xFF00807F]], dtype=np.uint32), 8, bits=8).tolist() == \
        [[1, 2, 3, 4, 0x7F, 0x80, 0x00, 0xFF]]
    # 2-bit: 0b11_10_01_00 repeated = 0xE4E4E4E4 -> 0, 1, 2, 3, 0, 1, 2, 3, ...
    assert O.unpack_q(np.array([[0xE4E4E4E4]], dtype=np.uint32), 16, bits=2).tolist() == [[0, 1, 2, 3] * 4]
    # 1-bit: bit i is element i
    q1 = O.unpack_q(np.array([[0x80000005]], dtype=np.uint32), 32, bits=1)[0].tolist()
    assert q1 == [1, 0, 1] + [0] * 28 + [1]
    # 4-bit keeps reading R1
    assert O.unpack_q(np.array([[0x76543210]], dtype=np.uint32), 8).tolist() == [[0, 1, 2, 3, 4, 5, 6, 7]]
    with pytest.raises(ValueError):
        O.unpack_q(np.zeros((1, 5), dtype=np.uint32), 32, bits=5)


def test_unpack_literal_words_three_bits():
    # eight 3-bit codes fill 24 stream bits and read as the octal digits right to left:
    # 1, 2, ..., 7, 0 is 0o07654321 = 0x1F58D1; four such runs fill three words
    w = np.array([[0xD11F58D1, 0x58D11F58, 0x1F58D11F]], dtype=np.uint32)
    assert O.unpack_q(w, 32, bits=3).tolist() == [[1, 2, 3, 4, 5, 6, 7, 0] * 4]
    # the codes that straddle a word: element 10 is bits 30, 31 of word 0 and bit 0 of word 1,
    # element 21 is bit 31 of word 1 and bits 0, 1 of word 2
    q = O.unpack_q(np.array([[0xC0000000, 0x00000001, 0x0]], dtype=np.uint32), 32, bits=3)[0]
    assert q.tolist() == [0] * 10 + [7] + [0] * 21
    q = O.unpack_q(np.array([[0x0, 0x80000000, 0x00000002]], dtype=np.uint32), 32, bits=3)[0]
    assert q.tolist() == [0] * 21 + [5] + [0] * 10
    # runs meet at a word boundary: bit 31 of word 2 is the top bit of element 31, bits 0, 1 of
    # word 3 the low bits of element 32
    q = O.unpack_q(np.array([[0, 0, 0x80000000, 0x00000003, 0, 0]], dtype=np.uint32), 64, bits=3)[0]
    assert q.tolist() == [0] * 31 + [4, 3] + [0] * 31
    with pytest.raises(ValueError):
        O.unpack_q(np.zeros((1, 4), dtype=np.uint32), 32, bits=3)


@pytest.mark.parametrize("bits", [1, 2, 3, 8])
def test_pack_and_unpack_are_inverse_and_match_the_input_generator(bits):
    rng = np.random.default_rng(60 + bits)
    q = rng.integers(0, 1 << bits, (7, 256))
    w = O.pack_q(q, bits)
    assert np.array_equal(w, synth.pack_codes(q, bits))
    assert np.array_equal(O.unpack_q(w, 256, bits), q)


@pytest.mark.parametrize("bits", [1, 2, 3, 8])
def test_reference_matches_brute_force_other_widths(bits):
    p = synth.random_problem(70 + bits, 3, 5, 256, bits=bits)
    y, A = O.reference(p["x"], p["wq"], p["scales"], p["biases"], bits=bits)
    yb, Ab = O.brute_force(p["x"], p["wq"], p["scales"], p["biases"], bits=bits)
    assert np.allclose(y, yb, rtol=0, atol=1e-12 * max(1.0, float(np.abs(Ab).max())))
    assert np.allclose(A, Ab, rtol=1e-12, atol=0)


def test_brute_force_decodes_straddling_three_bit_codes():
    # hand-packed 3-bit rows (reading R8): element 10 is bits 30, 31 of word 0 and bit 0 of word 1
    # (code 7), element 21 is bit 31 of word 1 and bits 0, 1 of word 2 (code 5), and elements 31
    # and 32 meet at the boundary of two runs (bit 31 of word 2 is the top bit of element 31, bits
    # 0, 1 of word 3 the low bits of element 32: codes 4 and 3); every other code is 0
    K = 128
    words = np.zeros((2, K * 3 // 32), dtype=np.uint32)
    words[0, 0], words[0, 1] = 0xC0000000, 0x00000001
    words[1, 1], words[1, 2], words[1, 3] = 0x80000000, 0x80000002, 0x00000003
    s = synth.const_bf16(1.0, (2, 1))
    b = synth.const_bf16(0.0, (2, 1))
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))   # y = q^T
    y, _ = O.brute_force(x, words, s, b, bits=3)
    expect = np.zeros((K, 2))
    expect[10, 0] = 7
    expect[21, 1], expect[31, 1], expect[32, 1] = 5, 4, 3
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("bits", [1, 2, 8])
def test_quantization_round_trip_bound_other_widths(bits):
    rng = np.random.default_rng(80 + bits)
    N, K = 64, 512
    W = np.float32(synth.W_STD) * rng.standard_normal((N, K)).astype(np.float32)
    wq, s, b = synth.quantize(W, bits=bits)
    wq_o, s_o, b_o = O.quantize_affine(W, bits)           # the oracle's own loop quantizer agrees
    assert np.array_equal(wq, wq_o) and np.array_equal(s, s_o) and np.array_equal(b, b_o)
    w_hat = O.dequant_f32(wq, s, b, K, bits=bits).astype(np.float64)
    err = np.abs(W.astype(np.float64) - w_hat).reshape(N, K // 128, 128)
    assert np.all(err <= _roundtrip_bound(W, s, b)[:, :, None])


def _bits_mutant(kind):
    """A copy of the oracle's width-generic unpack with one plausible mistake."""
    def unpack(wq, K, bits):
        per = 32 // bits
        w = np.asarray(wq, dtype=np.uint32)
        if kind == "fixed_eight_per_word":
            per = 8
        if w.shape[1] * per != K:
            raise ValueError("shape")
        q = np.empty((w.shape[0], K), dtype=np.uint8)
        mask = (1 << bits) - 1 if kind != "four_bit_mask" else 0xF
        for i in range(per):
            shift = bits * i if kind != "high_bits_first" else 32 - bits * (i + 1)
            if kind == "nibble_stride":
                shift = (4 * i) % 32
            q[:, i::per] = (w >> np.uint32(shift)) & np.uint32(mask)
        return q

    def ref(x, wq, s, b, bits):
        K = np.asarray(x).shape[1]
        q = unpack(wq, K, bits).astype(np.float32)
        g = np.arange(K) // 128
        w = (O.bf16_to_f32(s)[:, g] * q + O.bf16_to_f32(b)[:, g]).astype(np.float64)
        x64 = O.bf16_to_f64(x)
        return x64 @ w.T, np.abs(x64) @ np.abs(w).T
    return ref


BITS_MUTANTS = ["fixed_eight_per_word", "four_bit_mask", "high_bits_first", "nibble_stride"]


@pytest.mark.parametrize("bits", [1, 2, 8])
@pytest.mark.parametrize("kind", BITS_MUTANTS)
def test_bits_pins_catch_planted_mistakes(kind, bits):
    if kind == "four_bit_mask" and bits == 4:
        pytest.skip("not a mistake at 4 bits")
    failed = [p.__name__ for p in BITS_PINS if not p(_bits_mutant(kind), bits)]
    assert failed, f"planted mistake {kind!r} at {bits} bits passed every pin"


def test_bits_mutant_copy_is_faithful_without_a_mistake():
    # the mutant harness itself, with no mistake planted, passes every pin (so failures above
    # come from the planted mistakes)
    for bits in (1, 2, 8):
        assert all(p(_bits_mutant("none"), bits) for p in BITS_PINS)


# ----------------------------------------------------------------------------- W4A8 quantizer (R9)
#
# Pins of the per-row int8 activation quantizer, each independent of the oracle's numpy code:
# rows on an exact int8 grid, exact rounding ties, the zero row, the absmax element, the
# round-trip bound, and a pure-Python quantizer.  Each pin takes a quantizer (x_bits -> (xq, sx))
# so that planted mistakes can be shown to fail at least one of them.

def _grid_rows(rng, M, K):
    """Rows x = c * j with integer j in [-127, 127], |j| = 127 somewhere, c a power of two."""
    j = rng.integers(-127, 128, (M, K))
    j[np.arange(M), rng.integers(0, K, M)] = rng.choice([-127, 127], M)
    c = 2.0 ** rng.integers(-12, 4, M)
    return j, c, synth.to_bf16_bits((j * c[:, None]).astype(np.float32))


def _a8_pin_grid(qf):
    j, c, x = _grid_rows(np.random.default_rng(60), 6, 384)
    xq, sx = qf(x)
    return np.array_equal(np.asarray(xq, np.int64), j) and np.array_equal(np.asarray(sx, np.float64), c)


def _a8_pin_ties(qf):
    """x = c * (j + 1/2) next to an element 127 c: x * inv is an exact tie, broken to even."""
    rng = np.random.default_rng(61)
    M, K = 4, 256
    j = rng.integers(-126, 126, (M, K))
    v = (j + 0.5).astype(np.float64)
    v[:, 0] = 127.0
    c = 2.0 ** rng.integers(-8, 2, M)
    xq, _ = qf(synth.to_bf16_bits((v * c[:, None]).astype(np.float32)))
    expect = np.rint(v).astype(np.int64)          # numpy rint: ties to even, exact here
    return np.array_equal(np.asarray(xq, np.int64), expect)


def _a8_pin_zero_row(qf):
    x = synth.to_bf16_bits(np.random.default_rng(62).standard_normal((3, 256)).astype(np.float32))
    x[1] = 0
    xq, sx = qf(x)
    return float(sx[1]) == 0.0 and not np.any(np.asarray(xq)[1]) and float(sx[0]) > 0


def _a8_pin_absmax_and_bound(qf):
    """Random rows: the largest |x| maps to +-127 and |x - sx xq| <= sx / 2 + 2^-22 max|x|."""
    rng = np.random.default_rng(63)
    x = synth.to_bf16_bits((rng.standard_normal((8, 640)) * 2.0 ** rng.integers(-6, 6, (8, 1))).astype(np.float32))
    xq, sx = qf(x)
    xf = O.bf16_to_f64(x)
    a = np.max(np.abs(xf), axis=1)
    xq = np.asarray(xq, np.float64)
    sx = np.asarray(sx, np.float64)
    top = np.abs(xq[np.arange(8), np.argmax(np.abs(xf), axis=1)])
    err = np.abs(xf - sx[:, None] * xq)
    return (np.all(top == 127) and np.all(np.abs(xq) <= 127)
            and np.all(err <= (sx / 2 + 2.0 ** -22 * a)[:, None]))


def _a8_pin_python_loops(qf):
    """Against a quantizer written with Python floats and loops (fp64 then one fp32 rounding)."""
    rng = np.random.default_rng(64)
    x = synth.to_bf16_bits(rng.standard_normal((3, 200)).astype(np.float32))
    xq, sx = qf(x)
    for m in range(3):
        row = [O.bf16_to_f64(x[m, k:k + 1])[0] for k in range(200)]
        a = max(abs(v) for v in row)
        inv = _f32(127.0 / a)
        if float(sx[m]) != _f32(a / 127.0):
            return False
        if [int(q) for q in xq[m]] != [max(-127, min(127, round(_f32(v * inv)))) for v in row]:
            return False
    return True


def _f32(v):
    return float(np.float32(v))


A8_PINS = [_a8_pin_grid, _a8_pin_ties, _a8_pin_zero_row, _a8_pin_absmax_and_bound, _a8_pin_python_loops]


@pytest.mark.parametrize("pin", A8_PINS, ids=lambda p: p.__name__)
def test_int8_quantizer_passes_pin(pin):
    assert pin(O.quantize_rows_int8)


def _a8_mutant(kind):
    """A copy of the oracle's quantizer with one plausible mistake."""
    def qf(x_bits):
        x = O.bf16_to_f32(x_bits)
        a = np.max(np.abs(x), axis=1)
        if kind == "per_tensor_scale":
            a = np.full_like(a, np.max(a))
        top = np.float32(128 if kind == "scale_128" else 127)
        with np.errstate(divide="ignore"):
            inv = np.where(a > 0, top / a, np.float32(0)).astype(np.float32)
        sx = (a / top).astype(np.float32)
        prod = (x * inv[:, None]).astype(np.float32)
        if kind == "truncate":
            r = np.trunc(prod)
        elif kind == "ties_away":
            r = np.sign(prod) * np.floor(np.abs(prod) + 0.5)
        else:
            r = np.rint(prod)
        return np.clip(r, -127, 127).astype(np.int8), sx
    return qf


A8_MUTANTS = ["per_tensor_scale", "scale_128", "truncate", "ties_away"]


@pytest.mark.parametrize("kind", A8_MUTANTS)
def test_int8_quantizer_pins_catch_planted_mistakes(kind):
    failed = [p.__name__ for p in A8_PINS if not p(_a8_mutant(kind))]
    assert failed, f"planted mistake {kind!r} passed every pin"


def test_int8_mutant_copy_is_faithful_without_a_mistake():
    assert all(p(_a8_mutant("none")) for p in A8_PINS)


def test_w4a8_reference_equals_w4a16_reference_on_grid_rows():
    # on rows that the int8 grid represents exactly, sx * xq == x and the two references agree bit for bit
    rng = np.random.default_rng(65)
    _, _, x = _grid_rows(rng, 5, 512)
    p = synth.random_problem(66, 5, 40, 512)
    y8, A8 = O.reference_w4a8(x, p["wq"], p["scales"], p["biases"])
    y16, A16 = O.reference(x, p["wq"], p["scales"], p["biases"])
    assert np.array_equal(y8, y16) and np.array_equal(A8, A16)


@pytest.mark.parametrize("M,K,N", [(3, 256, 5), (2, 384, 7)])
def test_w4a8_reference_matches_brute_force(M, K, N):
    p = synth.random_problem(67 + M, M, N, K)
    y, A = O.reference_w4a8(p["x"], p["wq"], p["scales"], p["biases"])
    yb, Ab = O.brute_force_w4a8(p["x"], p["wq"], p["scales"], p["biases"])
    assert np.allclose(y, yb, rtol=0, atol=1e-12 * np.max(Ab)) and np.allclose(A, Ab, rtol=1e-12, atol=0)


def test_w4a8_zero_row_projects_to_zero():
    p = synth.random_problem(68, 3, 9, 256)
    x = p["x"].copy()
    x[2] = 0
    y, A = O.reference_w4a8(x, p["wq"], p["scales"], p["biases"])
    assert not np.any(y[2]) and not np.any(A[2])
