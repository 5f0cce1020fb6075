"""Seeded synthetic inputs for the W4A16 projection: the only code that the oracle
and the HIP path both consume.

This module makes inputs and nothing else.  It holds none of the projection's
arithmetic (no unpacking, dequantization, contraction or output rounding).  It
draws activations and fp32 weights from seeded generators, rounds activations
to bf16, and turns the fp32 weights into the packed affine format with the
input recipe below.

Input recipe (stand-in for the Qwen3-4B weights and prompts the pages benchmark
in "Week 2 Day 6: SIMD-Matrix Prefill", Task 5 and Benchmark Analysis, which are
not available here):

* activations ``x ~ N(0, 1)`` drawn in fp32, rounded to bf16 (nearest, ties to even);
* weights ``W ~ N(0, 0.02)`` drawn in fp32, quantized per 128-wide K group:
  ``scale = (max - min) / 15`` and ``bias = min`` in fp32, each rounded to bf16;
  ``q = clamp(rint((W - bias) / scale), 0, 15)`` in fp32 from the rounded
  scale and bias, ties to even, ``q = 0`` where the scale is 0;
* codes packed eight per uint32, low nibble first (element ``8j+i`` of a row in
  bits ``4i..4i+3`` of word ``j``);
* every stream comes from ``numpy.random.default_rng(SeedSequence([cfg, shape,
  role, chunk]))`` with ``role`` 0 for weights and 1 for activations; weight
  rows are drawn in chunks of 4096 output rows so that a 151936-row vocabulary
  head is generated in bounded memory.
"""

from __future__ import annotations

import numpy as np

GROUP = 128
W_STD = 0.02
ROW_CHUNK = 4096

ROLE_W = 0
ROLE_X = 1

# Projection shapes (K -> N) of one decoder layer with hidden size 2560, 32
# query heads and 8 key/value heads of dimension 128, and MLP width 9728.
LAYER_SHAPES = {
    "q": (2560, 4096),
    "k": (2560, 1024),
    "v": (2560, 1024),
    "o": (4096, 2560),
    "gate": (2560, 9728),
    "up": (2560, 9728),
    "down": (9728, 2560),
}
DECODE_SHAPES = [(2560, 9728), (9728, 2560), (2560, 4096), (2560, 1024)]
VOCAB_SHAPE = (2560, 151936)

# The five workloads.  Each entry: (shape name, K, N, list of M values).
CONFIGS = {
    1: {"name": "tiny", "runs": [("tiny", 256, 96, [33])]},
    2: {"name": "decode", "runs": [(f"decode{i}", K, N, [1, 4]) for i, (K, N) in enumerate(DECODE_SHAPES)]},
    3: {"name": "prefill128", "runs": [(p, K, N, [128]) for p, (K, N) in LAYER_SHAPES.items()]},
    4: {"name": "prefill512", "runs": [(p, K, N, [512, 509]) for p, (K, N) in LAYER_SHAPES.items()]},
    5: {"name": "prefill4096",
        "runs": [(p, *LAYER_SHAPES[p], [4096]) for p in ("gate", "up", "down")]
                + [("vocab", *VOCAB_SHAPE, [4096])]},
}


def shape_index(cfg: int, shape_name: str) -> int:
    """Position of ``shape_name`` in the config's run list (part of the seed)."""
    for i, run in enumerate(CONFIGS[cfg]["runs"]):
        if run[0] == shape_name:
            return i
    raise KeyError(f"config {cfg} has no shape {shape_name!r}")


def rng(cfg: int, shape: int, role: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, shape, role, chunk]))


def to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit pattern, nearest with ties to even (bit-level carry form).

    Finite values only; the generators never produce NaN or Inf.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def from_bf16_bits(bits) -> np.ndarray:
    """bf16 bit pattern -> fp32 (used only to build inputs from chosen values)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_codes(q, bits: int = 4) -> np.ndarray:
    """Codes ``[N, K]`` in 0 .. 2**bits - 1 -> ``uint32 [N, K*bits/32]``: a row's codes as one bit
    stream, lowest bits first (``bits`` in 1, 2, 3, 4, 8; at 1, 2, 4 and 8 no code crosses a
    word)."""
    if bits not in (1, 2, 3, 4, 8):
        raise ValueError(f"bits={bits} is not one of 1, 2, 3, 4, 8")
    q = np.asarray(q, dtype=np.uint32)
    n_rows, K = q.shape
    if (K * bits) % 32:
        raise ValueError(f"K * bits must be a multiple of 32")
    if 32 % bits == 0:
        per = 32 // bits
        qw = q.reshape(n_rows, K // per, per)
        shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))[None, None, :]
        return np.bitwise_or.reduce(qw << shifts, axis=2).astype(np.uint32)
    # codes that may cross words: spell out the stream bit by bit, then gather 32 bits per word
    stream = ((q[:, :, None] >> np.arange(bits, dtype=np.uint32)[None, None, :]) & 1).astype(np.uint32)
    stream = stream.reshape(n_rows, K * bits // 32, 32)
    weights = (np.uint32(1) << np.arange(32, dtype=np.uint32))[None, None, :]
    return (stream * weights).sum(axis=2, dtype=np.uint64).astype(np.uint32)


def quantize(W, group: int = GROUP, bits: int = 4):
    """Quantize fp32 weights ``[N, K]`` with the recipe above (vectorized over groups), with
    ``2**bits - 1`` levels per group.

    Returns ``(wq uint32 [N, K*bits/32], scales uint16 [N, K/group], biases uint16 [N, K/group])``.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    n_rows, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    Wg = W.reshape(n_rows, K // group, group)
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    levels = (1 << bits) - 1
    scale = np.divide(np.subtract(mx, mn, dtype=np.float32), np.float32(levels), dtype=np.float32)
    s_bits = to_bf16_bits(scale)
    b_bits = to_bf16_bits(mn)
    s = from_bf16_bits(s_bits)[:, :, None]
    b = from_bf16_bits(b_bits)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.divide(np.subtract(Wg, b, dtype=np.float32), s, dtype=np.float32)
    t = np.where(s == 0, np.float32(0), t)
    q = np.clip(np.rint(t), 0, levels).astype(np.uint8).reshape(n_rows, K)
    return pack_codes(q, bits), s_bits, b_bits


def weights(cfg: int, shape: int, N: int, K: int, group: int = GROUP):
    """Quantized weights for (cfg, shape): ``(wq, scales, biases)``, drawn in row chunks."""
    wq = np.empty((N, K // 8), dtype=np.uint32)
    s = np.empty((N, K // group), dtype=np.uint16)
    b = np.empty((N, K // group), dtype=np.uint16)
    for chunk, r0 in enumerate(range(0, N, ROW_CHUNK)):
        r1 = min(N, r0 + ROW_CHUNK)
        W = np.float32(W_STD) * rng(cfg, shape, ROLE_W, chunk).standard_normal((r1 - r0, K), dtype=np.float32)
        wq[r0:r1], s[r0:r1], b[r0:r1] = quantize(W, group)
    return wq, s, b


def activations(cfg: int, shape: int, M: int, K: int) -> np.ndarray:
    """bf16 activations ``[M, K]`` for (cfg, shape).

    Rows are drawn in order, so the first 509 rows of an M=512 draw equal an
    M=509 draw from the same stream.
    """
    return to_bf16_bits(rng(cfg, shape, ROLE_X).standard_normal((M, K), dtype=np.float32))


def problem(cfg: int, shape_name: str, M: int | None = None):
    """Inputs for one run of a config: dict with x, wq, scales, biases, M, N, K."""
    idx = shape_index(cfg, shape_name)
    _, K, N, Ms = CONFIGS[cfg]["runs"][idx]
    M = Ms[0] if M is None else M
    wq, s, b = weights(cfg, idx, N, K)
    x = activations(cfg, idx, M, K)
    return {"x": x, "wq": wq, "scales": s, "biases": b, "M": M, "N": N, "K": K}


def random_problem(seed: int, M: int, N: int, K: int, group: int = GROUP, bits: int = 4):
    """Inputs of an arbitrary shape from the same recipe, for tests (stream ``[0, seed, role, chunk]``);
    ``bits`` per code (1, 2, 3, 4, 8)."""
    wq = np.empty((N, K * bits // 32), dtype=np.uint32)
    s = np.empty((N, K // group), dtype=np.uint16)
    b = np.empty((N, K // group), dtype=np.uint16)
    for chunk, r0 in enumerate(range(0, N, ROW_CHUNK)):
        r1 = min(N, r0 + ROW_CHUNK)
        W = np.float32(W_STD) * rng(0, seed, ROLE_W, chunk).standard_normal((r1 - r0, K), dtype=np.float32)
        wq[r0:r1], s[r0:r1], b[r0:r1] = quantize(W, group, bits)
    x = to_bf16_bits(rng(0, seed, ROLE_X).standard_normal((M, K), dtype=np.float32))
    return {"x": x, "wq": wq, "scales": s, "biases": b, "M": M, "N": N, "K": K, "bits": bits}


def const_bf16(value: float, shape) -> np.ndarray:
    """A bf16 array of one exactly representable value (for closed-form test inputs)."""
    bits = to_bf16_bits(np.array([value], dtype=np.float32))[0]
    if float(from_bf16_bits(np.array([bits]))[0]) != value:
        raise ValueError(f"{value} is not exactly representable in bf16")
    return np.full(shape, bits, dtype=np.uint16)
