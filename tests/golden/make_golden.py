"""Writes ``worked_example_w4g128.json``: a tiny worked example whose expected
outputs are computed here with exact rational arithmetic (``fractions``), from
the format definition only.  The pages print no worked example, so this fixture
is a closed-form pin: its values come from neither the oracle nor the HIP path.

Format (the reading the oracle states): element ``8j+i`` of weight row ``n`` is
bits ``4i..4i+3`` of word ``j``; ``w[n,k] = s[n,k//128] * q[n,k] + b[n,k//128]``;
``y[m,n] = sum_k x[m,k] * w[n,k]``.  All chosen values are dyadic rationals
exactly representable in bf16, and every ``s*q + b`` is exact in fp32, so the
fp32 dequantization rounds nothing and the fp64 reference must equal the
rational result to within its final rounding.

It also writes ``worked_example_w{1,2,3,8}g128.json``: the same construction at the other
code widths (a row's codes as one bit stream, lowest bits first: element ``k`` in stream bits
``b*k .. b*k + b - 1``, stream bit ``t`` in bit ``t % 32`` of word ``t // 32``; codes in
``0 .. 2**b - 1``), again from exact rationals only.  At 1, 2, 4 and 8 bits that is element
``(32/b)j + i`` in bits ``b*i ..`` of word ``j``.

Run: ``python tests/golden/make_golden.py`` (rewrites the JSON files next to it).
"""

import json
import os
import struct
from fractions import Fraction

M, K, N, GROUP = 3, 256, 4, 128


def bf16_bits(v: Fraction) -> int:
    f = float(v)
    bits = struct.unpack("<I", struct.pack("<f", f))[0]
    assert bits & 0xFFFF == 0 and Fraction(f) == v, f"{v} not exact in bf16"
    return bits >> 16


def write(bits):
    levels = 1 << bits
    # codes: a closed form that varies with n and k and spans 0 .. 2**bits - 1
    q = [[(3 * n + 5 * k + (k // 128)) % levels for k in range(K)] for n in range(N)]
    # each row as one integer bit stream, cut into 32-bit words
    streams = [sum(q[n][k] << (bits * k) for k in range(K)) for n in range(N)]
    words = [[(streams[n] >> (32 * j)) & 0xFFFFFFFF for j in range(K * bits // 32)] for n in range(N)]
    s = [[Fraction(1, 2 ** (4 + n + g)) for g in range(K // GROUP)] for n in range(N)]
    b = [[Fraction(-(n + 1) * (g + 3), 2 ** 5) for g in range(K // GROUP)] for n in range(N)]
    # activations: small dyadic values with a pattern per row
    x = [[Fraction(((m + 1) * (k % 7) - 3), 2 ** (1 + m)) for k in range(K)] for m in range(M)]
    y = [[sum(x[m][k] * (s[n][k // GROUP] * q[n][k] + b[n][k // GROUP]) for k in range(K))
          for n in range(N)] for m in range(M)]
    A = [[sum(abs(x[m][k] * (s[n][k // GROUP] * q[n][k] + b[n][k // GROUP])) for k in range(K))
          for n in range(N)] for m in range(M)]
    if bits == 4:
        citation = ("No page prints a worked example. Closed-form values computed with exact "
                    "rationals from the affine W4 group-128 format (tiny-llm 'Week 2 Day 6: "
                    "SIMD-Matrix Prefill', scope list and Task 3) under the oracle's readings "
                    "R1-R4 (low-nibble-first packing, [N,K/8] words, [N,K/128] scale/bias).")
    else:
        citation = (f"No page prints a worked example. Closed-form values computed with exact "
                    f"rationals for {bits}-bit affine codes ('Route affine qmv_wide by bit-width and "
                    f"batch size #5' routes 1- and 2-bit affine matvecs) under the oracle's reading R8 "
                    f"(a row's codes as one bit stream, lowest bits first) and R3-R4.")
    out = {
        "citation": citation,
        "M": M, "K": K, "N": N, "group": GROUP, "bits": bits,
        "x_bf16": [[bf16_bits(v) for v in row] for row in x],
        "wq_u32": words,
        "scales_bf16": [[bf16_bits(v) for v in row] for row in s],
        "biases_bf16": [[bf16_bits(v) for v in row] for row in b],
        "codes": q,
        "y_exact": [[f"{v.numerator}/{v.denominator}" for v in row] for row in y],
        "abs_mass_exact": [[f"{v.numerator}/{v.denominator}" for v in row] for row in A],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"worked_example_w{bits}g128.json")
    with open(path, "w") as f:
        json.dump(out, f)
        f.write("\n")
    print("wrote", path)


def main():
    for bits in (4, 1, 2, 3, 8):
        write(bits)


if __name__ == "__main__":
    main()
