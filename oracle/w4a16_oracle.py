"""Plain, slow, obviously correct CPU oracle for the W4A16 group-quantized projection.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What the method computes
------------------------
``y[m, n] = sum_k x[m, k] * w[n, k]``, a projection ("quantized linear") of bf16
activations ``x [M, K]`` by 4-bit affine-quantized weights, where
``w[n, k] = s[n, g] * q[n, k] + b[n, g]`` with ``g = k // 128``.

Sources on the pages:

* tiny-llm book, "Week 2 Day 6: SIMD-Matrix Prefill", opening scope list:
  weights have four bits and group size 128; activations, quantization
  parameters (scale and bias) and the output are BF16; matrix accumulators
  are FP32.
* same page, "Task 3: Hoist Quantization Parameters": one scale and one bias
  cover 128 reduction values of one output column.
* same page, "Task 4: Project Only Required Logits": ``logits_to_keep`` slices
  the last rows *before* the projection.
* "Route affine qmv_wide by bit-width and batch size #5", description:
  affine quantized matvec in which a group of weights is dequantized
  (``scale * q + bias``) and reused across the input rows.

Readings where the pages are silent:

* R1 nibble order: element ``8*j + i`` of a weight row sits in bits
  ``4*i .. 4*i+3`` of 32-bit word ``j`` (low nibble first).
* R2 ``Wq`` is ``uint32 [N, K/8]`` row-major: one contiguous run of K codes
  per output column ``n``.
* R3 scales and biases are bf16 ``[N, K/128]`` row-major, indexed ``[n, k // 128]``.
* R4 dequantization is evaluated in fp32 with two roundings,
  ``f32(f32(s * q) + b)``.  ``s * q`` is exact in fp32 (8-bit by 4-bit
  significands), so a fused multiply-add gives the same value.
* R5 the reference accumulates in fp64.  Every product ``x * w`` is exact in
  fp64 (8 + 24 significand bits), so only the final sum is rounded.
* R6 per-element parity tolerance:
  ``|y - y_ref| <= 2^-8 * |y_ref| + 2^-10 * sum_k |x[m,k] * w[n,k]|``;
  NaN or Inf in ``y`` always fails.
* R7 the input quantizer (how test weights are made, not part of the method):
  per (n, g) in fp32, ``scale = (max - min) / 15``, ``bias = min``, both rounded
  to bf16 (nearest, ties to even); ``q = clamp(rint((W - b) / s), 0, 15)``
  computed from the *rounded* s and b, ties to even; a group with ``s == 0``
  gets ``q = 0``.
* R8 other bit widths ("Route affine qmv_wide by bit-width and batch size #5"
  routes affine matvecs by bit width, naming 1- and 2-bit weights; the page
  gives no format): for ``bits`` in {1, 2, 3, 4, 8} the words of a row form one
  bit stream, lowest bits first (stream bit ``t`` is bit ``t % 32`` of word
  ``t // 32``), and element ``k`` of the row is stream bits
  ``bits*k .. bits*k + bits - 1``; ``Wq`` is ``uint32 [N, K*bits/32]``.  At 1,
  2, 4 and 8 bits no code crosses a word, so element ``(32/bits)*j + i`` sits
  in bits ``bits*i .. bits*i + bits - 1`` of word ``j`` (R1 at 4 bits); at 3
  bits every 32 codes fill three words and two of them (elements 10 and 21 of
  the run) straddle a word boundary.  The group, scale, bias and R4-R7 are
  unchanged with ``2**bits - 1`` in place of 15.  ``s * q`` stays exact in
  fp32 (at most 8 + 8 significand bits).
* R9 int8 activations (W4A8; "Feature Request: Metal prefill speedup (~68%)
  on M5 Max" lists an int8 mat-mat for large batches after oMLX's int8 prefill,
  with no recipe): each activation row is quantized symmetrically to int8 with
  one fp32 scale, all in fp32: ``a = max_k |x[m, k]|``, ``inv = 127 / a`` and
  ``sx = a / 127`` (each a correctly rounded division; a zero row has
  ``inv = sx = 0``), ``xq = clamp(rint(x * inv), -127, 127)`` with the product
  rounded to fp32 and ties to even.  The projection then uses ``sx * xq`` in
  place of ``x``; weights as R1-R4.
"""

from __future__ import annotations

import math
import struct
from dataclasses import dataclass

import numpy as np

__all__ = [
    "GROUP",
    "TOL_REL",
    "TOL_MASS",
    "bf16_to_f32",
    "bf16_to_f64",
    "f32_to_bf16_rne",
    "unpack_q",
    "dequant_f32",
    "reference",
    "CheckResult",
    "check",
    "quantize_w4g128",
    "quantize_affine",
    "pack_q",
    "BITS",
    "brute_force",
    "keep_last_rows",
    "silu_f64",
    "swiglu_reference",
    "check_swiglu",
    "quantize_rows_int8",
    "reference_w4a8",
    "brute_force_w4a8",
]

GROUP = 128
BITS = (1, 2, 3, 4, 8)       # code widths of reading R8 (4 is the W4 format of R1)
TOL_REL = 2.0 ** -8
TOL_MASS = 2.0 ** -10


# --------------------------------------------------------------------------- bf16


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32, exactly.

    A bf16 value is the upper half of the fp32 pattern with the same sign,
    exponent and leading seven mantissa bits, so widening is a 16-bit shift.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16_rne(values) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest with ties to even, by definition.

    For a finite value the two bf16 candidates are its truncation toward zero
    and the next bf16 away from zero.  The nearer one is chosen, measured in
    exact float64 arithmetic; on a tie the candidate whose lowest mantissa bit
    is 0 wins.  The step past the largest finite bf16 is the infinity, which
    takes part in the comparison as the value 2^128, as IEEE 754 overflow
    rounding prescribes.  NaN maps to a quiet NaN with the same sign.
    """
    v = np.asarray(values, dtype=np.float32)
    u = v.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    lo_bits = (u & np.uint32(0xFFFF0000)).astype(np.uint32)
    hi_bits = (lo_bits + np.uint32(0x10000)).astype(np.uint32)  # next away from zero, same sign
    mag = np.abs(v.astype(np.float64))
    lo_mag = np.abs(lo_bits.view(np.float32).astype(np.float64))
    hi_is_inf = (hi_bits & np.uint32(0x7FFFFFFF)) == np.uint32(0x7F800000)
    with np.errstate(over="ignore", invalid="ignore"):
        hi_mag = np.where(hi_is_inf, 2.0 ** 128, np.abs(hi_bits.view(np.float32).astype(np.float64)))
    with np.errstate(invalid="ignore"):  # inf - inf on infinite inputs; those are replaced below
        d_lo = mag - lo_mag
        d_hi = hi_mag - mag
    lo_even = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(take_hi, hi_bits, lo_bits) >> np.uint32(16)
    finite = np.isfinite(v)
    is_inf = np.isinf(v)
    out = np.where(is_inf, (sign >> np.uint32(16)) | np.uint32(0x7F80), out)
    out = np.where(~finite & ~is_inf, (sign >> np.uint32(16)) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


# --------------------------------------------------------------------------- format


def _stream_period(bits: int) -> tuple[int, int]:
    """(codes, words) of the shortest run of whole words that holds whole codes: (32/bits, 1)
    when bits divides 32, (32, 3) at 3 bits (reading R8)."""
    if bits not in BITS:
        raise ValueError(f"bits={bits} is not one of {BITS}")
    codes = 32 // math.gcd(32, bits)
    return codes, codes * bits // 32


def unpack_q(wq, K: int, bits: int = 4) -> np.ndarray:
    """Packed words ``uint32 [N, K*bits/32]`` -> codes ``uint8 [N, K]`` (readings R1, R2, R8).

    Element ``k`` of a row is stream bits ``bits*k ..``: bits ``sh ..`` of word ``j`` and, when
    it crosses the word, the low bits of word ``j + 1``, with ``j, sh = divmod(bits*k, 32)``.
    """
    per, wpp = _stream_period(bits)
    w = np.asarray(wq, dtype=np.uint32)
    n_rows, n_words = w.shape
    if n_words * 32 != K * bits:
        raise ValueError(f"Wq has {n_words} words per row; K={K} at {bits} bits needs {K * bits // 32}")
    # each word next to its successor as one 64-bit window (a zero word after the last)
    w64 = np.concatenate([w, np.zeros((n_rows, 1), dtype=np.uint32)], axis=1).astype(np.uint64)
    mask = np.uint64((1 << bits) - 1)
    q = np.empty((n_rows, K), dtype=np.uint8)
    for i in range(per):
        # element per*r + i of every row, for every run r of wpp words
        j, sh = divmod(bits * i, 32)
        lo = w64[:, j:n_words:wpp]
        hi = w64[:, j + 1:n_words + 1:wpp]
        q[:, i::per] = ((lo | (hi << np.uint64(32))) >> np.uint64(sh)) & mask
    return q


def dequant_f32(wq, scales, biases, K: int, group: int = GROUP, bits: int = 4) -> np.ndarray:
    """Dequantized weights ``w[n, k] = f32(f32(s[n,g] * q[n,k]) + b[n,g])`` (reading R4).

    Follows the affine form of "Route affine qmv_wide by bit-width and batch
    size #5" and the per-group scale/bias of "Week 2 Day 6: SIMD-Matrix
    Prefill", Task 3.
    """
    q = unpack_q(wq, K, bits).astype(np.float32)
    s = bf16_to_f32(scales)
    b = bf16_to_f32(biases)
    if s.shape != (q.shape[0], K // group) or b.shape != s.shape:
        raise ValueError(f"scales/biases must be [{q.shape[0]}, {K // group}], got {s.shape} / {b.shape}")
    g_of_k = np.arange(K) // group
    s_k = s[:, g_of_k]
    b_k = b[:, g_of_k]
    prod = np.multiply(s_k, q, dtype=np.float32)
    return np.add(prod, b_k, dtype=np.float32)


def reference(x_bits, wq, scales, biases, group: int = GROUP, columns=None, col_chunk: int = 8192,
              bits: int = 4):
    """Reference output and absolute mass, both fp64 ``[M, N']`` (readings R4, R5).

    ``y_ref = x64 @ w64ᵀ`` and ``A = |x64| @ |w64|ᵀ``, where ``x64`` is the exact
    widening of the bf16 activations and ``w64`` of the fp32 dequantized
    weights.  ``columns`` (optional index array) restricts the output columns;
    the weights are dequantized ``col_chunk`` columns at a time so that large
    vocabularies fit in memory.
    """
    x64 = bf16_to_f64(x_bits)
    if x64.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    return _project(x64, wq, scales, biases, group, columns, col_chunk, bits)


def _project(x64, wq, scales, biases, group, columns, col_chunk, bits):
    """``(x64 @ w64ᵀ, |x64| @ |w64|ᵀ)`` for fp64 activations (shared by both references)."""
    M, K = x64.shape
    wq = np.asarray(wq)
    scales = np.asarray(scales)
    biases = np.asarray(biases)
    cols = np.arange(wq.shape[0]) if columns is None else np.asarray(columns)
    y = np.empty((M, cols.size), dtype=np.float64)
    A = np.empty((M, cols.size), dtype=np.float64)
    ax = np.abs(x64)
    for c0 in range(0, cols.size, col_chunk):
        sel = cols[c0:c0 + col_chunk]
        w64 = dequant_f32(wq[sel], scales[sel], biases[sel], K, group, bits).astype(np.float64)
        y[:, c0:c0 + sel.size] = x64 @ w64.T
        A[:, c0:c0 + sel.size] = ax @ np.abs(w64).T
    return y, A


@dataclass
class CheckResult:
    ok: bool
    max_ratio: float       # max over elements of |err| / bound (inf for NaN/Inf or err > 0 = bound)
    worst: tuple           # (m, n) of the worst element
    n_bad: int
    n_total: int

    def __str__(self) -> str:
        return (f"ok={self.ok} max_err/bound={self.max_ratio:.4g} at {self.worst} "
                f"bad={self.n_bad}/{self.n_total}")


def check(y_bits, y_ref, A, rel: float = TOL_REL, mass: float = TOL_MASS) -> CheckResult:
    """Per-element parity test of a bf16 result against the fp64 reference (reading R6)."""
    y = bf16_to_f64(y_bits)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    if y.shape != y_ref.shape or A.shape != y_ref.shape:
        raise ValueError(f"shape mismatch: y {y.shape}, y_ref {y_ref.shape}, A {A.shape}")
    finite = np.isfinite(y)
    with np.errstate(invalid="ignore"):
        err = np.abs(y - y_ref)
    bound = rel * np.abs(y_ref) + mass * A
    good = finite & (err <= bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err == 0, 0.0, np.inf))
    ratio = np.where(finite, ratio, np.inf)
    if ratio.size == 0:
        return CheckResult(True, 0.0, (), 0, 0)
    flat = int(np.argmax(ratio))
    worst = tuple(int(i) for i in np.unravel_index(flat, ratio.shape))
    return CheckResult(bool(good.all()), float(ratio.flat[flat]), worst,
                       int((~good).sum()), int(good.size))


# --------------------------------------------------------------------------- quantizer (R7)


def pack_q(q, bits: int = 4) -> np.ndarray:
    """Codes ``[N, K]`` (0 .. 2**bits - 1) -> words ``uint32 [N, K*bits/32]``: element k at stream
    bits bits*k .., lowest bits first (R1, R8)."""
    per, wpp = _stream_period(bits)
    q = np.asarray(q, dtype=np.uint64)
    n_rows, K = q.shape
    if K % per:
        raise ValueError(f"K={K} is not a multiple of {per} at {bits} bits")
    n_words = K * bits // 32
    mask = np.uint64((1 << bits) - 1)
    words = np.zeros((n_rows, n_words + 1), dtype=np.uint64)   # one spare word for the carry
    for i in range(per):
        j, sh = divmod(bits * i, 32)
        v = (q[:, i::per] & mask) << np.uint64(sh)
        words[:, j:n_words:wpp] |= v & np.uint64(0xFFFFFFFF)
        words[:, j + 1:n_words + 1:wpp] |= v >> np.uint64(32)
    return words[:, :n_words].astype(np.uint32)


def quantize_w4g128(W, group: int = GROUP):
    """Reference quantizer for the input recipe (reading R7), one group at a time.

    Returns ``(wq uint32 [N, K/8], scales bf16-bits [N, G], biases bf16-bits [N, G])``.
    """
    return quantize_affine(W, 4, group)


def quantize_affine(W, bits: int = 4, group: int = GROUP):
    """The R7 quantizer at ``bits`` per code (R8): ``2**bits - 1`` levels per group.

    Returns ``(wq uint32 [N, K*bits/32], scales bf16-bits [N, G], biases bf16-bits [N, G])``.
    """
    _stream_period(bits)
    W = np.asarray(W, dtype=np.float32)
    n_rows, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    q = np.zeros((n_rows, K), dtype=np.uint8)
    s_bits = np.zeros((n_rows, G), dtype=np.uint16)
    b_bits = np.zeros((n_rows, G), dtype=np.uint16)
    levels = np.float32((1 << bits) - 1)
    for n in range(n_rows):
        for g in range(G):
            blk = W[n, g * group:(g + 1) * group]
            mn = np.float32(blk.min())
            mx = np.float32(blk.max())
            scale = np.float32(np.float32(mx - mn) / levels)
            sb = f32_to_bf16_rne(np.array([scale], dtype=np.float32))[0]
            bb = f32_to_bf16_rne(np.array([mn], dtype=np.float32))[0]
            s_bits[n, g] = sb
            b_bits[n, g] = bb
            s32 = bf16_to_f32(np.array([sb]))[0]
            b32 = bf16_to_f32(np.array([bb]))[0]
            if s32 == 0:
                continue  # degenerate group: every code is 0, so w = b
            t = np.divide(np.subtract(blk, b32, dtype=np.float32), s32, dtype=np.float32)
            q[n, g * group:(g + 1) * group] = np.clip(np.rint(t), 0, levels).astype(np.uint8)
    return pack_q(q, bits), s_bits, b_bits


# --------------------------------------------------------------------------- brute force


def _f32_round(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16_scalar(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def brute_force(x_bits, wq, scales, biases, group: int = GROUP, bits: int = 4):
    """Pure-Python loops over (m, n, k); small inputs only.

    Every weight is decoded from its word by explicit shifts, dequantized with
    two fp32 roundings, and each output is the correctly rounded fp64 sum
    (``math.fsum``) of the exact products.  Returns ``(y, A)`` as fp64 arrays.
    """
    x_bits = np.asarray(x_bits)
    wq = np.asarray(wq)
    M, K = x_bits.shape
    N = wq.shape[0]
    xs = [[_bf16_scalar(x_bits[m, k]) for k in range(K)] for m in range(M)]
    return _brute_sums(xs, _brute_weights(wq, scales, biases, K, group, bits))


def _brute_weights(wq, scales, biases, K, group, bits):
    """Every weight decoded from the row's bit stream by explicit shifts (reading R8: element k is
    stream bits ``bits*k ..``, i.e. bits ``sh ..`` of word ``j`` continued in word ``j + 1`` when
    the code crosses it, ``j, sh = divmod(bits*k, 32)``), dequantized with two fp32 roundings."""
    ws = []
    mask = (1 << bits) - 1
    n_words = wq.shape[1]
    for n in range(wq.shape[0]):
        row = []
        for k in range(K):
            j, sh = divmod(bits * k, 32)
            window = int(wq[n, j])
            if j + 1 < n_words:
                window |= int(wq[n, j + 1]) << 32
            code = (window >> sh) & mask
            s = _bf16_scalar(scales[n, k // group])
            b = _bf16_scalar(biases[n, k // group])
            row.append(_f32_round(_f32_round(s * code) + b))
        ws.append(row)
    return ws


def _brute_sums(xs, ws):
    """Correctly rounded fp64 sums of the exact products, with their absolute mass."""
    M, N, K = len(xs), len(ws), len(xs[0]) if xs else 0
    y = np.empty((M, N))
    A = np.empty((M, N))
    for m in range(M):
        xm = xs[m]
        for n in range(N):
            prods = [xm[k] * ws[n][k] for k in range(K)]
            y[m, n] = math.fsum(prods)
            A[m, n] = math.fsum(abs(p) for p in prods)
    return y, A


# --------------------------------------------------------------------------- logits_to_keep


def keep_last_rows(M: int, keep: int) -> slice:
    """Rows a projection sees under ``logits_to_keep`` ("Week 2 Day 6", Task 4).

    ``keep > 0`` selects the last ``keep`` rows, ``keep == 0`` selects every row
    (prompt scoring), anything else is an error.
    """
    if keep < 0 or keep > M:
        raise ValueError(f"logits_to_keep={keep} must be in [0, M={M}]")
    return slice(0, M) if keep == 0 else slice(M - keep, M)


# --------------------------------------------------------------------------- fused gate/up + SwiGLU


def silu_f64(z):
    """SiLU ``z * sigmoid(z) = z / (1 + exp(-z))`` in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_reference(x_bits, gate, up, group: int = GROUP, columns=None):
    """Reference for the gate/up projection pair followed by SwiGLU, all fp64.

    ``gate`` and ``up`` are ``(wq, scales, biases)`` triples of one shape.  The
    fused step is named by "Feature Request: Metal prefill speedup (~68%) on
    M5 Max" (feature list: SwiGLU fused into the mat-mat; related work: gate
    and up rows interleaved with the GLU in the mat-mat epilogue).  Returns
    ``(h_ref, g_ref, A_g, u_ref, A_u)`` with ``h = silu(g) * u``.
    """
    g_ref, A_g = reference(x_bits, *gate, group=group, columns=columns)
    u_ref, A_u = reference(x_bits, *up, group=group, columns=columns)
    return silu_f64(g_ref) * u_ref, g_ref, A_g, u_ref, A_u


def check_swiglu(h_bits, g_ref, A_g, u_ref, A_u, rel: float = TOL_REL, mass: float = TOL_MASS) -> CheckResult:
    """Per-element test of a fused SwiGLU result.

    The two projections carry the R6 error ``e_g <= rel*|g| + mass*A_g`` and
    ``e_u`` likewise.  ``|d silu/dz| <= 1.1`` everywhere, so the product
    ``silu(g) * u`` may move by ``1.1*e_g*(|u| + e_u) + |silu(g)|*e_u``; the
    final bf16 rounding adds ``rel*|h|``.
    """
    g_ref = np.asarray(g_ref, np.float64)
    u_ref = np.asarray(u_ref, np.float64)
    e_g = rel * np.abs(g_ref) + mass * np.asarray(A_g, np.float64)
    e_u = rel * np.abs(u_ref) + mass * np.asarray(A_u, np.float64)
    h_ref = silu_f64(g_ref) * u_ref
    bound = 1.1 * e_g * (np.abs(u_ref) + e_u) + np.abs(silu_f64(g_ref)) * e_u + rel * np.abs(h_ref)
    h = bf16_to_f64(h_bits)
    finite = np.isfinite(h)
    with np.errstate(invalid="ignore"):
        err = np.abs(h - h_ref)
    good = finite & (err <= bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err == 0, 0.0, np.inf))
    ratio = np.where(finite, ratio, np.inf)
    if ratio.size == 0:
        return CheckResult(True, 0.0, (), 0, 0)
    flat = int(np.argmax(ratio))
    worst = tuple(int(i) for i in np.unravel_index(flat, ratio.shape))
    return CheckResult(bool(good.all()), float(ratio.flat[flat]), worst, int((~good).sum()), int(good.size))


# --------------------------------------------------------------------------- W4A8 (R9)


def quantize_rows_int8(x_bits):
    """Per-row symmetric int8 quantizer of the activations (reading R9).

    Returns ``(xq, sx)``: int8 codes ``[M, K]`` and the fp32 row scales ``[M]``,
    so that ``sx[m] * xq[m, k]`` approximates ``x[m, k]`` within ``sx[m] / 2``
    (plus fp32 rounding of the scale).
    """
    x = bf16_to_f32(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(a > 0, np.float32(127) / a, np.float32(0)).astype(np.float32)
    sx = (a / np.float32(127)).astype(np.float32)
    prod = (x * inv[:, None]).astype(np.float32)
    xq = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return xq, sx


def reference_w4a8(x_bits, wq, scales, biases, group: int = GROUP, columns=None, col_chunk: int = 8192):
    """Reference of the W4A8 projection and its absolute mass, fp64 ``[M, N']``.

    The activations are replaced by their int8 reconstruction ``sx * xq``
    (exact in fp64: an fp32 scale times an integer below 2^7) and projected by
    the dequantized 4-bit weights as in ``reference``.
    """
    xq, sx = quantize_rows_int8(x_bits)
    x64 = sx.astype(np.float64)[:, None] * xq.astype(np.float64)
    return _project(x64, wq, scales, biases, group, columns, col_chunk, 4)


def brute_force_w4a8(x_bits, wq, scales, biases, group: int = GROUP):
    """Pure-Python loops for the W4A8 projection; small inputs only.

    The quantizer works on Python floats: a division or product of two fp32
    values evaluated in fp64 and rounded once to fp32 is the correctly rounded
    fp32 result, and ``round`` breaks ties to even.
    """
    x_bits = np.asarray(x_bits)
    M, K = x_bits.shape
    xs = []
    for m in range(M):
        row = [_bf16_scalar(x_bits[m, k]) for k in range(K)]
        a = max((abs(v) for v in row), default=0.0)
        inv = _f32_round(127.0 / a) if a > 0 else 0.0
        sx = _f32_round(a / 127.0)
        codes = [max(-127, min(127, round(_f32_round(v * inv)))) for v in row]
        xs.append([sx * c for c in codes])
    return _brute_sums(xs, _brute_weights(np.asarray(wq), scales, biases, K, group, 4))
