"""GPU parity of the grouped projections of one input (``w4a16_linear_grouped``) through the C ABI:
every projection against the CPU oracle element by element (random cases within the tolerance of
``O.check``, integer cases bit for bit), ragged projections and rows, the exact-code form, the
per-projection path for few rows, and no write outside any output.
"""

import numpy as np
import pytest

import oracle as O
from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bits, to_device
from test_gpu_parity import _exact_case

pytestmark = pytest.mark.gpu


def _devices(problems):
    """x of the first problem (shared) and each problem's (wq, scales, biases) on the GPU."""
    dev = [to_device(p) for p in problems]
    return dev[0][0], [d[1:] for d in dev]


def _check_all(ys, problems, rows=None):
    for y, p in zip(ys, problems):
        got = bits(y)
        x = p["x"] if rows is None else p["x"][rows]
        if rows is not None:
            got = got[rows]
        y_ref, A = O.reference(x, p["wq"], p["scales"], p["biases"])
        r = O.check(got, y_ref, A)
        assert r.ok, f"N={p['N']}: {r}"


def _shared_x(problems):
    """The problems with the first one's activations (the grouped call reads one x)."""
    x = problems[0]["x"]
    return [dict(p, x=x) for p in problems]


@pytest.mark.parametrize("M", [512, 509])
def test_qkv_prefill_matches_oracle(lib, M):
    """The 512-row (and ragged 509-row) q, k and v projections of the layer in one grouped launch."""
    import torch
    problems = _shared_x([synth.problem(4, name, M) for name in ("q", "k", "v")])
    plan = lib.w4a16_grouped_plan([p["N"] for p in problems], M, problems[0]["K"])
    announce(f"grouped qkv M={M} plan {plan}")
    assert plan["path"] == lib.PATH_GROUPED
    x, w = _devices(problems)
    ys = lib.w4a16_linear_grouped(x, w)
    torch.cuda.synchronize()
    rows = np.r_[0:M:5, M - 7:M]
    _check_all(ys, problems, rows=rows)


def test_qkv_128_rows_split_matches_oracle(lib):
    """The 128-row q, k and v: an under-filled grid, split along K with one grouped slice sum."""
    import torch
    M = 128
    problems = _shared_x([synth.problem(3, name) for name in ("q", "k", "v")])
    plan = lib.w4a16_grouped_plan([p["N"] for p in problems], M, problems[0]["K"])
    announce(f"grouped qkv M={M} plan {plan}")
    assert plan["path"] == lib.PATH_GROUPED and plan["split_k"] > 1
    x, w = _devices(problems)
    ys = lib.w4a16_linear_grouped(x, w)
    torch.cuda.synchronize()
    _check_all(ys, problems)


@pytest.mark.parametrize("kind", ["sums", "pow2"])
def test_split_integer_cases_are_bit_exact_and_repeat(lib, kind):
    """A split grouped launch on integer inputs: exact, and the same bits on a second call."""
    import torch
    M, K = 96, 2560
    cases = [_exact_case(kind, M, n, K, seed=3000 + i + 10 * (kind == "pow2")) for i, n in enumerate((640, 256))]
    x_bits = cases[0][0]["x"]
    xi = synth.from_bf16_bits(x_bits).astype(np.float64)
    problems = [dict(p, x=x_bits) for p, _ in cases]
    plan = lib.w4a16_grouped_plan([p["N"] for p in problems], M, K)
    announce(f"grouped split integer {kind} plan {plan}")
    assert plan["split_k"] > 1
    x, w = _devices(problems)
    first = [bits(y) for y in lib.w4a16_linear_grouped(x, w)]
    second = [bits(y) for y in lib.w4a16_linear_grouped(x, w)]
    torch.cuda.synchronize()
    for p, a, b in zip(problems, first, second):
        q = np.stack([(p["wq"] >> (4 * i)) & 0xF for i in range(8)], axis=-1).reshape(p["N"], K).astype(np.float64)
        wv = q if kind == "sums" else (q - 8) / 64.0
        assert np.array_equal(a, synth.to_bf16_bits((xi @ wv.T).astype(np.float32))), f"N={p['N']}"
        assert np.array_equal(a, b)


def test_ragged_projections_and_rows(lib):
    """Projections whose column counts are not multiples of the 128-column tile, at a ragged M."""
    import torch
    M, K = 77, 512
    problems = _shared_x([synth.random_problem(40 + i, M, n, K) for i, n in enumerate((200, 96, 1000))])
    announce(f"grouped ragged M={M} N={[p['N'] for p in problems]}")
    x, w = _devices(problems)
    ys = lib.w4a16_linear_grouped(x, w)
    torch.cuda.synchronize()
    _check_all(ys, problems)


def test_exact_code_form_above_1024_rows(lib):
    import torch
    M, K = 1100, 512
    problems = _shared_x([synth.random_problem(50 + i, M, n, K) for i, n in enumerate((384, 256))])
    plan = lib.w4a16_grouped_plan([p["N"] for p in problems], M, K)
    announce(f"grouped exact-code M={M} plan {plan}")
    assert plan["path"] == lib.PATH_GROUPED and plan["variant"] >= 10
    x, w = _devices(problems)
    ys = lib.w4a16_linear_grouped(x, w)
    torch.cuda.synchronize()
    _check_all(ys, problems, rows=np.r_[0:M:9, M - 5:M])


@pytest.mark.parametrize("kind", ["sums", "pow2"])
def test_qkv_integer_cases_are_bit_exact(lib, kind):
    """Integer and power-of-two inputs (exact in fp32 and bf16): every output bit for bit."""
    import torch
    M, K = 512, 2560
    cases = [_exact_case(kind, M, n, K, seed=2000 + i + 10 * (kind == "pow2"))
             for i, n in enumerate((4096, 1024, 1024))]
    # one x for all three: the first case's, and each expected value recomputed for it
    x_bits = cases[0][0]["x"]
    xi = synth.from_bf16_bits(x_bits).astype(np.float64)
    expects = []
    for p, _ in cases:
        q = np.stack([(p["wq"] >> (4 * i)) & 0xF for i in range(8)], axis=-1).reshape(p["N"], K).astype(np.float64)
        w = q if kind == "sums" else (q - 8) / 64.0
        expects.append(synth.to_bf16_bits((xi @ w.T).astype(np.float32)))
    problems = [dict(p, x=x_bits) for p, _ in cases]
    announce(f"grouped qkv integer {kind}")
    x, w = _devices(problems)
    ys = lib.w4a16_linear_grouped(x, w)
    torch.cuda.synchronize()
    for y, e, p in zip(ys, expects, problems):
        assert np.array_equal(bits(y), e), f"N={p['N']}"


def test_few_rows_run_each_projection_alone(lib):
    """At most 32 rows the call runs each projection's own dispatch: identical to w4a16_linear."""
    import torch
    for M in (4, 16, 32):
        problems = _shared_x([synth.random_problem(60 + i, M, n, 512) for i, n in enumerate((640, 128, 256))])
        plan = lib.w4a16_grouped_plan([p["N"] for p in problems], M, 512)
        announce(f"grouped few rows M={M} plan {plan}")
        assert plan["path"] == lib.PATH_PER_PROJECTION
        x, w = _devices(problems)
        ys = lib.w4a16_linear_grouped(x, w)
        alone = [lib.w4a16_linear(x, *wi) for wi in w]
        torch.cuda.synchronize()
        for y, a in zip(ys, alone):
            assert np.array_equal(bits(y), bits(a))
        _check_all(ys, problems)


@pytest.mark.parametrize("count", [1, 4])
def test_one_and_four_projections(lib, count):
    import torch
    M, K = 96, 256
    problems = _shared_x([synth.random_problem(70 + i, M, 128 + 64 * i, K) for i in range(count)])
    announce(f"grouped count={count}")
    x, w = _devices(problems)
    ys = lib.w4a16_linear_grouped(x, w)
    torch.cuda.synchronize()
    _check_all(ys, problems)


@pytest.mark.parametrize("K", [256, 2560])
def test_no_write_outside_any_output(lib, K):
    """The outputs are views into one buffer with poisoned gaps between and around them: every gap
    keeps its bit pattern, and every output element is written (unsplit at K = 256, split with
    the grouped slice sum at K = 2560)."""
    import torch
    M = 70
    problems = _shared_x([synth.random_problem(80 + i, M, n, K) for i, n in enumerate((136, 72, 260))])
    gap = 4096
    sizes = [M * p["N"] for p in problems]
    total = gap + sum(n + gap for n in sizes)
    poison = 0x7FC1                                      # a NaN bit pattern no result has
    buf = torch.full((total,), poison, dtype=torch.int16, device="cuda:0")
    ys, off, spans = [], gap, []
    for p, n in zip(problems, sizes):
        ys.append(buf[off:off + n].view(torch.bfloat16).view(M, p["N"]))
        spans.append((off, off + n))
        off += n + gap
    x, w = _devices(problems)
    announce(f"grouped poisoned gaps K={K} plan {lib.w4a16_grouped_plan([p['N'] for p in problems], M, K)}")
    lib.w4a16_linear_grouped(x, w, ys=ys)
    torch.cuda.synchronize()
    host = buf.cpu().numpy().view(np.uint16)
    mask = np.ones(total, dtype=bool)
    for a, b in spans:
        mask[a:b] = False
        assert not np.any(host[a:b] == poison), "an output element was not written"
    assert np.all(host[mask] == poison), "a write landed outside the outputs"
    _check_all(ys, problems)


def test_rejects_overlapping_outputs(lib):
    import torch
    M, K = 40, 256
    problems = _shared_x([synth.random_problem(90 + i, M, 128, K) for i in range(2)])
    x, w = _devices(problems)
    y = torch.empty((M, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        lib.w4a16_linear_grouped(x, w, ys=[y, y])
