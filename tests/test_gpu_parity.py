"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Bar: integer / closed-form cases bit-exact; random cases within the per-element tolerance
``|y - y_ref| <= 2^-8 |y_ref| + 2^-10 sum_k |x w|`` with no NaN/Inf.  Sizes span several tiles
with ragged tails; the full workload sizes are checked on sampled rows (all columns) or on
every element where the oracle is fast enough.
"""

import numpy as np
import pytest

import oracle as O
from w4a16_group_quantized_qmv_amd import synth

from gpu_helpers import announce, bf16_from_bits, bits, to_device

pytestmark = pytest.mark.gpu


def run(lib, p, path, split_k=None, dev=None):
    """Run one path on problem p; returns y bits.  path: 'linear' | 'qmv' | 'qmm'."""
    import torch
    announce(f"{path} M={p['M']} N={p['N']} K={p['K']} split={split_k}")
    x, wq, s, b = dev if dev is not None else to_device(p)
    if path == "linear":
        y = lib.w4a16_linear(x, wq, s, b)
    elif path == "qmv":
        y = lib.qmv_w4a16(x, wq, s, b)
    else:
        y = lib.qmm_w4a16(x, wq, s, b, split_k=split_k or 0)
    torch.cuda.synchronize()
    return bits(y)


def assert_parity(y_bits, p, rows=None, cols=None):
    x = p["x"] if rows is None else p["x"][rows]
    y_ref, A = O.reference(x, p["wq"], p["scales"], p["biases"], columns=cols)
    got = y_bits if rows is None else y_bits[rows]
    if cols is not None:
        got = got[:, cols]
    r = O.check(got, y_ref, A)
    assert r.ok, str(r)
    return r


# ---------------------------------------------------------------------------------- tiny config

@pytest.mark.parametrize("path,split", [("linear", None), ("qmm", 1), ("qmm", 2), ("qmm", 0)])
def test_tiny_config_all_paths(lib, path, split):
    p = synth.problem(1, "tiny")          # M=33, K=256, N=96: ragged in M and N
    assert_parity(run(lib, p, path, split), p)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_tiny_config_qmv_rows(lib, M):
    p = dict(synth.problem(1, "tiny"))
    p["x"] = p["x"][:M]
    p["M"] = M
    y_qmv = run(lib, p, "qmv")
    assert_parity(y_qmv, p)
    assert_parity(run(lib, p, "qmm", 1), p)


# ---------------------------------------------------------------------------------- bit-exact pins

def identity_problem(K=256, N=96, seed=5):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (N, K))
    x = np.where(np.eye(K, dtype=bool), synth.const_bf16(1.0, (K, K)), np.uint16(0))
    G = K // 128
    return q, {"x": x, "wq": synth.pack_codes(q), "scales": synth.const_bf16(1.0, (N, G)),
               "biases": synth.const_bf16(0.0, (N, G)), "M": K, "N": N, "K": K}


@pytest.mark.parametrize("split", [1, 2])
def test_identity_unpack_is_bit_exact_qmm(lib, split):
    q, p = identity_problem()
    y = run(lib, p, "qmm", split)
    expect = synth.to_bf16_bits(q.T.astype(np.float32))
    assert np.array_equal(y, expect), "nibble order / indexing mismatch on the matrix path"


@pytest.mark.parametrize("N", [96, 24600])        # row-amortized kernel / persistent wide kernel
def test_identity_unpack_is_bit_exact_qmv(lib, N):
    q, p = identity_problem(N=N)
    expect = synth.to_bf16_bits(q.T.astype(np.float32))
    for r0 in range(0, 256, 8):       # one-hot rows, eight at a time
        sub = dict(p, x=p["x"][r0:r0 + 8], M=8)
        y = run(lib, sub, "qmv")
        assert np.array_equal(y, expect[r0:r0 + 8]), f"rows {r0}..{r0 + 7}"


@pytest.mark.parametrize("path,N,K", [("qmv", 160, 512), ("qmv", 6150, 512), ("qmv", 300, 9728), ("qmv", 16400, 512),
                                      ("qmv", 24600, 512), ("qmm", 160, 512)])
def test_small_integer_sums_are_exact(lib, path, N, K):
    # qmv cases (8 rows) cover the burst kernel with 8 row slots, the dequantizing K-split, the
    # 64-column and the wide kernels
    rng = np.random.default_rng(8)
    M = 8 if path == "qmv" else 40
    q = rng.integers(0, 16, (N, K))
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):                 # at most 17 ones per row keeps every sum <= 255
        xi[m, rng.choice(K, size=rng.integers(0, 18), replace=False)] = 1
    G = K // 128
    p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q),
         "scales": synth.const_bf16(1.0, (N, G)), "biases": synth.const_bf16(0.0, (N, G)), "M": M, "N": N, "K": K}
    y = run(lib, p, path, 1)
    assert np.array_equal(y, synth.to_bf16_bits((xi @ q.T).astype(np.float32)))


@pytest.mark.parametrize("M,N,split", [(35, 203, 2), (35, 203, 3), (40, 256, 2), (40, 256, 5), (33, 97, 4)])
def test_split_slice_sums_are_exact_in_both_forms(lib, M, N, split):
    # integer sums: every split gives the exact result, with M x N odd or even, ragged N and
    # slices of one to four groups
    rng = np.random.default_rng(14)
    K = 1024
    q = rng.integers(0, 16, (N, K))
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):                 # at most 17 ones per row keeps every sum <= 255
        xi[m, rng.choice(K, size=rng.integers(0, 18), replace=False)] = 1
    G = K // 128
    p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q),
         "scales": synth.const_bf16(1.0, (N, G)), "biases": synth.const_bf16(0.0, (N, G)), "M": M, "N": N, "K": K}
    assert lib.w4a16_plan(M, N, K, 128, lib.PATH_QMM, split)["split_k"] == split
    y = run(lib, p, "qmm", split)
    assert np.array_equal(y, synth.to_bf16_bits((xi @ q.T).astype(np.float32)))


@pytest.mark.parametrize("path,N", [("qmv", 48), ("qmv", 24600), ("qmm", 48)])
def test_power_of_two_affine_is_exact(lib, path, N):
    rng = np.random.default_rng(9)
    M = 8 if path == "qmv" else 24
    K = 384
    q = rng.integers(0, 16, (N, K))
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):                 # <= 32 entries of +-1: |sum x (q - 8)| <= 256, exact in bf16 / 64
        idx = rng.choice(K, size=32, replace=False)
        xi[m, idx] = rng.choice([-1, 1], size=32)
    G = K // 128
    p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q),
         "scales": synth.const_bf16(2.0 ** -6, (N, G)), "biases": synth.const_bf16(-8 * 2.0 ** -6, (N, G)),
         "M": M, "N": N, "K": K}
    y = run(lib, p, path, 1)
    assert np.array_equal(y, synth.to_bf16_bits(((xi @ (q - 8).T) / 64.0).astype(np.float32)))


def _exact_case(kind, M, N, K, seed):
    """Integer inputs whose projection is exact in fp32 and bf16: ``sums`` (s = 1, b = 0, at most 17
    ones per row: every sum an integer <= 255) or ``pow2`` (s = 2^-6, b = -8 * 2^-6, 32 entries of
    +-1 per row: every result k / 64 with |k| <= 256)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (N, K))
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):
        if kind == "sums":
            xi[m, rng.choice(K, size=rng.integers(0, 18), replace=False)] = 1
        else:
            xi[m, rng.choice(K, size=32, replace=False)] = rng.choice([-1, 1], size=32)
    G = K // 128
    s, b = (1.0, 0.0) if kind == "sums" else (2.0 ** -6, -8 * 2.0 ** -6)
    p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q),
         "scales": synth.const_bf16(s, (N, G)), "biases": synth.const_bf16(b, (N, G)), "M": M, "N": N, "K": K}
    xf = xi.astype(np.float64)
    exact = xf @ q.T.astype(np.float64) if kind == "sums" else (xf @ (q - 8).T.astype(np.float64)) / 64.0
    return p, synth.to_bf16_bits(exact.astype(np.float32))


@pytest.mark.parametrize("kind", ["sums", "pow2"])
@pytest.mark.parametrize("shape", list(synth.LAYER_SHAPES))
def test_step_tiles_are_bit_exact(lib, shape, kind):
    """The tiles and splits the 512-row step plans (96 x 128 for gate / up, four-wave 64 x 128 with
    three slices for o / down, eight-wave 64 x 128 for q and the split k / v) on exact integer and
    power-of-two cases: the result must equal the exact value bit for bit."""
    K, N = synth.LAYER_SHAPES[shape]
    M = 512
    plan = lib.w4a16_plan(M, N, K)
    p, expect = _exact_case(kind, M, N, K, seed=1000 + 2 * list(synth.LAYER_SHAPES).index(shape) + (kind == "pow2"))
    announce(f"step tile {shape} {kind}: plan tile {plan['tile_m']}x{plan['tile_n']} variant {plan['variant']} "
             f"split {plan['split_k']}")
    y = run(lib, p, "linear")
    assert np.array_equal(y, expect), f"{shape} {kind} plan {plan}"


@pytest.mark.parametrize("path", ["qmv", "qmm"])
def test_all_zero_codes(lib, path):
    rng = np.random.default_rng(10)
    M = 5 if path == "qmv" else 70
    K, N = 1024, 200
    G = K // 128
    p = {"x": synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)),
         "wq": np.zeros((N, K // 8), dtype=np.uint32),
         "scales": synth.to_bf16_bits(rng.uniform(0.001, 0.01, (N, G)).astype(np.float32)),
         "biases": synth.to_bf16_bits((0.02 * rng.standard_normal((N, G))).astype(np.float32)),
         "M": M, "N": N, "K": K}
    assert_parity(run(lib, p, path, 1), p)


# ---------------------------------------------------------------------------------- qmv families

# (N, K, M, kernel the policy picks): 0 = 16-column dequantizing workgroups splitting K four ways,
# 1 = 64-column workgroups, 2 = persistent wide kernel (activations and their group sums staged
# in LDS once, one wave per 16-column block), 3 = row-amortized 16-column workgroups (exact codes
# on the matrix core, s * P + b * X per group; at 4 bits now only above 8 rows, on the skinny
# path), 4 = burst (every wave issues all its loads at once)
QMV_FAMILY_CASES = [
    (4000, 256, 3, 4),       # burst, ragged N
    (6150, 384, 1, 4),       # burst, odd group count, ragged N
    (4000, 256, 6, 4),       # burst with 8 row slots, ragged N
    (6150, 384, 5, 4),       # burst with 8 row slots, odd group count
    (2600, 8192, 3, 4),      # 64 groups: burst, 4 groups in each of 16 waves
    (2600, 8192, 5, 4),      # 64 groups at 5 rows: burst, 8 row slots, 16 waves of 4 groups
    (2600, 8320, 5, 0),      # 65 groups at 5 rows: the dequantizing K-split kernel
    (1000, 10240, 2, 4),     # 80 groups: packed burst, ten waves of two steps of four groups
    (1000, 16384, 1, 4),     # 128 groups at 1 row: packed burst, sixteen waves of two steps
    (20000, 8192, 2, 4),     # 1250 blocks at 2 rows: packed burst instead of the wide kernel
    (1000, 10368, 3, 0),     # 81 groups at 3 rows: past it
    (1000, 9728, 8, 0),      # long K, ragged N
    (16390, 384, 8, 1),      # 1025 blocks, odd group count
    (33000, 256, 1, 2),      # one group pair per block: every step ends a block
    (24600, 512, 5, 2),      # ragged N and M
    (30010, 1024, 8, 2),     # eight rows
    (24600, 384, 6, 1),      # odd group count: the wide kernel does not apply
    (24600, 384, 2, 4),      # packed burst from 1024 blocks: two steps per wave, odd group count
    (30000, 2560, 1, 2),     # 1875 blocks under 32 groups: the wide kernel
    (16400, 4096, 5, 2),     # wide from 1024 blocks once K >= 4096
    (16400, 4096, 4, 2),     # the same at 4 rows (the burst kernel stops at 1024 blocks there)
    (20000, 2560, 4, 4),     # burst at 1250 blocks under 32 groups: seven waves of three
    (9728, 4096, 4, 4),      # 608 blocks at K = 4096: burst, 2 groups per wave
    (9728, 4096, 7, 4),      # the same at 7 rows: burst with 8 row slots
    (24600, 9728, 8, 1),     # activations too large for the wide kernel's LDS
]


@pytest.mark.parametrize("N,K,M,variant", QMV_FAMILY_CASES)
def test_qmv_kernel_families(lib, N, K, M, variant):
    assert lib.w4a16_plan(M, N, K, 128, lib.PATH_QMV)["variant"] == variant
    p = synth.random_problem(11, M, N, K)
    y = run(lib, p, "qmv")
    assert_parity(y, p)
    assert np.array_equal(run(lib, p, "qmv"), y), "repeat run differs"


# ---------------------------------------------------------------------------------- skinny rows

# (M, N, K, tile_m the policy picks): 8 < M <= 16 runs the matvec kernels (tile_m 16), above
# that 32-row MFMA tiles with split-K (tile_m 32)
SKINNY_CASES = [
    (9, 4000, 256, 16),        # row-amortized matvec, ragged N
    (16, 8200, 384, 16),       # row-amortized matvec, odd group count
    (12, 2600, 8192, 16),      # long K above eight rows: row-amortized
    (10, 16400, 384, 16),      # 64-column matvec
    (12, 24600, 512, 16),      # wide matvec at 12 rows
    (16, 24600, 2048, 32),     # the wide matvec's activation tile would be too large: tiles
    (17, 1000, 2560, 32),      # ragged N, split-K (8 tiles)
    (24, 2560, 9728, 32),      # long K: 8 slices
    (32, 9728, 2560, 32),      # gate projection shape, 3 slices
    (32, 4096, 384, 32),       # odd group count, split limited to one slice per group pair
]


@pytest.mark.parametrize("M,N,K,tile_m", SKINNY_CASES)
def test_skinny_rows(lib, M, N, K, tile_m):
    pl = lib.w4a16_plan(M, N, K, 128, lib.PATH_AUTO)
    assert pl["path"] == lib.PATH_SKINNY and pl["tile_m"] == tile_m
    p = synth.random_problem(12, M, N, K)
    y = run(lib, p, "linear")
    assert_parity(y, p)
    assert np.array_equal(run(lib, p, "linear"), y), "repeat run differs"


def test_skinny_matches_tiled_path_on_integer_sums(lib):
    # exact integer sums: the skinny kernels and the 64-row tiles must agree bit for bit
    rng = np.random.default_rng(13)
    for M in (9, 16, 20, 32):
        K, N = 512, 1100
        q = rng.integers(0, 16, (N, K))
        xi = np.zeros((M, K), dtype=np.int64)
        for m in range(M):
            xi[m, rng.choice(K, size=rng.integers(0, 18), replace=False)] = 1
        G = K // 128
        p = {"x": synth.to_bf16_bits(xi.astype(np.float32)), "wq": synth.pack_codes(q),
             "scales": synth.const_bf16(1.0, (N, G)), "biases": synth.const_bf16(0.0, (N, G)),
             "M": M, "N": N, "K": K}
        expect = synth.to_bf16_bits((xi @ q.T).astype(np.float32))
        assert np.array_equal(run(lib, p, "linear"), expect), f"skinny M={M}"
        assert np.array_equal(run(lib, p, "qmm", 1), expect), f"tiled M={M}"


@pytest.mark.parametrize("path,split", [("qmv", None), ("qmm", 1), ("qmm", 3)])
def test_scaling_by_two_is_bit_exact(lib, path, split):
    p = synth.random_problem(77, 8 if path == "qmv" else 100, 300, 768)
    y1 = run(lib, p, path, split)
    p2 = dict(p, x=synth.to_bf16_bits(2 * synth.from_bf16_bits(p["x"])))
    y2 = run(lib, p2, path, split)
    assert np.array_equal(synth.from_bf16_bits(y2), 2 * synth.from_bf16_bits(y1))


# ---------------------------------------------------------------------------------- decode config

@pytest.mark.parametrize("shape", ["decode0", "decode1", "decode2", "decode3"])
@pytest.mark.parametrize("M", [1, 4])
def test_decode_config(lib, shape, M):
    p = synth.problem(2, shape, M)
    dev = to_device(p)
    y = run(lib, p, "linear", dev=dev)
    assert_parity(y, p)
    y_qmv = run(lib, p, "qmv", dev=dev)
    assert np.array_equal(y, y_qmv)          # linear dispatches M <= 8 to qmv


# ---------------------------------------------------------------------------------- prefill configs

@pytest.mark.parametrize("shape", list(synth.LAYER_SHAPES))
def test_prefill128_config(lib, shape):
    p = synth.problem(3, shape, 128)
    dev = to_device(p)
    assert_parity(run(lib, p, "linear", dev=dev), p)
    assert_parity(run(lib, p, "qmm", 1, dev=dev), p)


def sample_rows(M, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("shape", list(synth.LAYER_SHAPES))
def test_prefill512_config_and_ragged_prefix(lib, shape):
    p512 = synth.problem(4, shape, 512)
    y512 = run(lib, p512, "linear")
    assert_parity(y512, p512, rows=sample_rows(512))
    p509 = synth.problem(4, shape, 509)
    assert np.array_equal(p509["x"], p512["x"][:509])
    y509 = run(lib, p509, "linear")
    assert_parity(y509, p509, rows=sample_rows(509, seed=1))
    # same tiles and split for 509 and 512 rows: the shared rows agree bit for bit
    assert np.array_equal(y509, y512[:509])


@pytest.mark.parametrize("M,N,K", [(192, 16384, 256), (250, 9728, 384), (90, 40000, 1280)])
def test_96_row_tiles_match_oracle(lib, M, N, K):
    # shapes the policy gives 96 x 128 tiles (fewer rounds per compute unit than 64-row tiles):
    # ragged rows (250 = 2 x 96 + 58, 90 < 96) and columns (40000 = 312 x 128 + 64)
    plan = lib.w4a16_plan(M, N, K)
    assert (plan["tile_m"], plan["k_waves"], plan["split_k"]) == (96, 2, 1)
    p = synth.random_problem(96, M, N, K)
    y = run(lib, p, "linear")
    assert_parity(y, p)
    assert np.array_equal(y, run(lib, p, "qmm", 1))      # the forced-unsplit plan is the same plan


@pytest.mark.parametrize("split", [1, 2, 4, 19, 0])
def test_split_k_down_projection(lib, split):
    p = synth.problem(4, "down", 512)       # K = 9728: 76 groups
    dev = to_device(p)
    y = run(lib, p, "qmm", split, dev=dev)
    assert_parity(y, p, rows=sample_rows(512, 32))
    again = run(lib, p, "qmm", split, dev=dev)
    assert np.array_equal(y, again)          # fixed-order reduction: deterministic


# ---------------------------------------------------------------------------------- long prefill + vocab

@pytest.mark.parametrize("shape", ["gate", "up", "down"])
def test_prefill4096_config(lib, shape):
    p = synth.problem(5, shape, 4096)
    assert_parity(run(lib, p, "linear"), p, rows=sample_rows(4096, 24))


@pytest.fixture(scope="module")
def vocab():
    announce("generating vocab head inputs (2560 -> 151936)")
    return synth.problem(5, "vocab", 4096)


@pytest.mark.timeout(900)
def test_vocab_logits_to_keep(lib, vocab):
    import torch
    p = vocab
    x, wq, s, b = to_device(p)
    announce("vocab keep=1")
    last = bits(lib.linear(x, wq, s, b, logits_to_keep=1))
    assert last.shape == (1, p["N"])
    one = dict(p, x=p["x"][-1:], M=1)
    assert_parity(last, one)                                  # every column of the last row
    announce("vocab all rows")
    full = bits(lib.linear(x, wq, s, b, logits_to_keep=0))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    cols = np.unique(np.concatenate([rng.choice(p["N"], 4096, replace=False), [0, p["N"] - 1]]))
    assert_parity(full, p, rows=sample_rows(4096, 8), cols=cols)
    # the sliced projection and the last row of the full projection both match the oracle
    assert_parity(full[-1:], one, cols=cols)
    keep3 = bits(lib.linear(x, wq, s, b, logits_to_keep=3))
    assert np.array_equal(keep3, bits(lib.linear(x[-3:], wq, s, b)))


# ---------------------------------------------------------------------------------- scale alignment
# The ABI requires 2-byte aligned scales and biases.  The tile kernels read them four groups per
# 8-byte load only when both arrays are 8-byte aligned (and G % 4 == 0), and the wide matvec a
# group pair per 4-byte load only when they are 4-byte aligned; otherwise the per-group forms run.

def offset_by_one(t):
    """The same bf16 values in a buffer that starts 2 bytes past an aligned allocation."""
    import torch
    flat = torch.zeros(t.numel() + 1, dtype=t.dtype, device=t.device)
    flat[1:] = t.reshape(-1)
    return flat[1:].view(t.shape)


def test_tile_scales_at_two_byte_offsets_match_aligned(lib):
    # G = 20: the aligned call reads scales four groups per load, the offset one per group; the
    # per-group arithmetic is the same, so the results agree bit for bit
    import torch
    p = synth.random_problem(41, 200, 1024, 2560)
    announce("qmm scales at 2-byte offsets M=200 N=1024 K=2560")
    x, wq, s, b = to_device(p)
    so, bo = offset_by_one(s), offset_by_one(b)
    assert so.data_ptr() % 8 == 2 and bo.data_ptr() % 8 == 2
    y_al = bits(lib.linear(x, wq, s, b, path="qmm", split_k=1))
    y_off = bits(lib.linear(x, wq, so, bo, path="qmm", split_k=1))
    assert np.array_equal(y_al, y_off)
    assert_parity(y_off, p, rows=np.r_[0, 63, 64, 199])


def test_wide_matvec_scales_at_two_byte_offsets(lib):
    # 32768 columns route one row to the persistent wide kernel; offset scales take the 64-column
    # kernel instead; both within the tolerance
    p = synth.random_problem(42, 1, 32768, 256)
    assert lib.w4a16_plan(1, 32768, 256)["variant"] == 2
    announce("wide qmv scales at 2-byte offsets M=1 N=32768 K=256")
    x, wq, s, b = to_device(p)
    assert_parity(bits(lib.linear(x, wq, s, b)), p)
    assert_parity(bits(lib.linear(x, wq, offset_by_one(s), offset_by_one(b))), p)


@pytest.mark.parametrize("M", [1, 3, 6])   # packed form; 16-column form with 4 and 8 row slots
def test_burst_matvec_scales_at_two_byte_offsets(lib, M):
    # the burst kernel loads each scale and bias on its own: offset arrays give the same bits
    p = synth.random_problem(43, M, 4000, 2560)
    assert lib.w4a16_plan(M, 4000, 2560)["variant"] == 4
    announce(f"burst qmv scales at 2-byte offsets M={M} N=4000 K=2560")
    x, wq, s, b = to_device(p)
    y_al = bits(lib.linear(x, wq, s, b))
    assert np.array_equal(y_al, bits(lib.linear(x, wq, offset_by_one(s), offset_by_one(b))))
    assert_parity(y_al, p)


# ---------------------------------------------------------------------------------- memory safety

SENTINEL = 0x7FA5   # a NaN pattern the kernels never produce


@pytest.mark.parametrize("path,M,N,K,split", [("qmv", 3, 96, 256, None), ("qmm", 33, 96, 256, 1),
                                              ("qmm", 509, 200, 1024, 1), ("qmm", 509, 200, 1024, 3),
                                              ("qmv", 8, 1000, 384, None), ("qmm", 130, 4000, 256, 2)])
def test_guard_rows_and_poisoned_output(lib, path, M, N, K, split):
    import torch
    p = synth.random_problem(M * 31 + N, M, N, K)
    x, wq, s, b = to_device(p)
    big = bf16_from_bits(np.full((M + 2, N), SENTINEL, dtype=np.uint16))
    y = big[1:M + 1]
    announce(f"guard {path} M={M} N={N} K={K} split={split}")
    if path == "qmv":
        lib.qmv_w4a16(x, wq, s, b, y=y)
    else:
        lib.qmm_w4a16(x, wq, s, b, y=y, split_k=split)
    torch.cuda.synchronize()
    out = bits(big)
    assert np.all(out[0] == SENTINEL) and np.all(out[-1] == SENTINEL), "write outside [M, N]"
    assert not np.any(out[1:-1] == SENTINEL), "element of y left unwritten"
    assert_parity(out[1:-1], p)


def test_repeated_runs_are_bit_identical(lib):
    p = synth.random_problem(4242, 300, 1000, 2560)
    dev = to_device(p)
    for path, split in [("qmm", 0), ("qmm", 5)]:
        first = run(lib, p, path, split, dev=dev)
        for _ in range(9):
            assert np.array_equal(first, run(lib, p, path, split, dev=dev))
    q = dict(p, x=p["x"][:7], M=7)
    devq = to_device(q)
    first = run(lib, q, "qmv", dev=devq)
    for _ in range(9):
        assert np.array_equal(first, run(lib, q, "qmv", dev=devq))


# ---------------------------------------------------------------------------------- split-K workspace reuse
# A split launch writes every fp32 partial it later sums, so the workspace's earlier contents do
# not matter, and a captured split call replays like an eager one (no memset in the path).

def split_call(lib, p, split, ws, dev):
    import torch
    x, wq, s, b = dev
    y = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device=x.device)
    lib.qmm_w4a16(x, wq, s, b, y=y, split_k=split, workspace=ws)
    return y


def test_split_ignores_stale_workspace_and_reuses_it(lib):
    import torch
    M, N, K, split = 100, 700, 4096, 5
    p = synth.random_problem(31, M, N, K)
    dev = to_device(p)
    plan = lib.w4a16_plan(M, N, K, path=lib.PATH_QMM, split_k=split)
    assert plan["split_k"] == split
    nbytes = plan["workspace_bytes"]
    announce(f"split workspace reuse M={M} N={N} K={K} split={split} workspace={nbytes}")
    zeroed = torch.zeros(nbytes // 4 + 1, dtype=torch.int32, device="cuda:0")
    y0 = bits(split_call(lib, p, split, zeroed, dev))
    torch.cuda.synchronize()
    assert_parity(y0, p)
    # arbitrary bytes everywhere (seeded; as a fresh allocation may hold), then the same
    # workspace call after call, and another split of the same shape on it
    noise = torch.from_numpy(np.random.default_rng(7).integers(-2 ** 31, 2 ** 31, nbytes // 4 + 1,
                                                               dtype=np.int64).astype(np.int32)).to("cuda:0")
    for _ in range(4):
        assert np.array_equal(bits(split_call(lib, p, split, noise, dev)), y0)
    assert_parity(bits(split_call(lib, p, 3, noise, dev)), p)


def test_split_call_in_a_graph_replays(lib):
    """A captured split call (tile kernel, then the slice reduction) replays like the eager call;
    replays alternate with eager calls on the same workspace."""
    import torch
    M, N, K, split = 64, 1000, 2560, 4
    p = synth.random_problem(32, M, N, K)
    x, wq, s, b = to_device(p)
    plan = lib.w4a16_plan(M, N, K, path=lib.PATH_QMM, split_k=split)
    ws = torch.zeros(plan["workspace_bytes"] // 4 + 1, dtype=torch.int32, device="cuda:0")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    announce(f"split graph replay M={M} N={N} K={K} split={split}")
    lib.qmm_w4a16(x, wq, s, b, y=y, split_k=split, workspace=ws)
    torch.cuda.synchronize()
    ref = bits(y)
    assert_parity(ref, p)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            lib.qmm_w4a16(x, wq, s, b, y=y, split_k=split, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref), f"replay {i}"
        y2 = torch.empty_like(y)
        lib.qmm_w4a16(x, wq, s, b, y=y2, split_k=split, workspace=ws)     # eager, same workspace
        torch.cuda.synchronize()
        assert np.array_equal(bits(y2), ref), f"eager call after replay {i}"


def test_split_call_on_a_side_stream_keeps_its_workspace(lib):
    """A split call on the caller's side stream, with output and workspace allocated by the
    binding on torch's current stream: the side stream is kept busy first, so the call's kernels
    are still queued when it returns; the current stream then allocates memory of the
    workspace's size and fills it.  The result must match the oracle (the binding records the
    side stream on what it allocated, so that memory is not handed out again early)."""
    import torch
    M, N, K, split = 64, 2000, 4096, 4
    p = synth.random_problem(33, M, N, K)
    x, wq, s, b = to_device(p)
    nbytes = lib.w4a16_plan(M, N, K, path=lib.PATH_QMM, split_k=split)["workspace_bytes"]
    busy = torch.randn(4096, 4096, device="cuda:0")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    ref = None
    for trial in range(3):
        announce(f"side-stream split call M={M} N={N} K={K} split={split} trial={trial}")
        with torch.cuda.stream(side):
            for _ in range(6):
                busy = (busy @ busy).mul_(1.0 / 64.0)
        y = lib.qmm_w4a16(x, wq, s, b, split_k=split, stream=side)
        junk = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda:0").fill_(float("nan"))
        junk2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0").fill_(float("nan"))
        torch.cuda.synchronize()
        got = bits(y)
        assert_parity(got, p)
        if ref is None:
            ref = got
        assert np.array_equal(got, ref), f"trial {trial}"
        del junk, junk2


# ---------------------------------------------------------------------------------- error paths on the device

def test_forced_split_without_workspace_is_rejected(lib):
    import ctypes
    p = synth.random_problem(1, 64, 128, 1024)
    x, wq, s, b = to_device(p)
    y = bf16_from_bits(np.zeros((64, 128), dtype=np.uint16))
    L = lib.load()
    st = L.qmm_w4a16(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(), 64, 128, 1024, 128, 4,
                     None, 0, None)
    assert st == 5
    st = L.qmm_w4a16(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(), 64, 128, 1024, 128, 4,
                     ctypes.c_void_p(x.data_ptr()), 16, None)
    assert st == 5


def test_policy_split_without_workspace_falls_back(lib):
    import torch
    p = synth.random_problem(2, 64, 128, 2048)     # few tiles: the policy would split
    assert lib.w4a16_plan(64, 128, 2048)["split_k"] > 1
    x, wq, s, b = to_device(p)
    y = bf16_from_bits(np.zeros((64, 128), dtype=np.uint16))
    st = lib.load().w4a16_linear(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                                 64, 128, 2048, 128, None, 0, None)
    assert st == 0
    torch.cuda.synchronize()
    assert_parity(bits(y), p)


# ---------------------------------------------------------------------------------- fused gate / up

def gate_up_problem(seed, M, N, K):
    """x, gate and up weights of one shape from the seeded recipe (gate and up differ)."""
    g = synth.random_problem(seed, M, N, K)
    u = synth.random_problem(seed + 1000, M, N, K)
    return g["x"], (g["wq"], g["scales"], g["biases"]), (u["wq"], u["scales"], u["biases"])


def run_gate_up(lib, x, gate, up, split_k=0, workspace="auto"):
    import torch
    announce(f"gate_up M={x.shape[0]} N={gate[0].shape[0]} K={x.shape[1]} split={split_k}")
    M, K = x.shape
    xd = to_device({"x": x, "wq": gate[0], "scales": gate[1], "biases": gate[2]})
    ud = to_device({"x": x, "wq": up[0], "scales": up[1], "biases": up[2]})
    if workspace == "auto":
        h = lib.w4a16_gate_up_swiglu(xd[0], xd[1:], ud[1:], split_k=split_k)
    else:   # call the C ABI directly with the given workspace (None = no workspace)
        N = gate[0].shape[0]
        h = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        st = lib.load().w4a16_gate_up_swiglu(xd[0].data_ptr(), xd[1].data_ptr(), xd[2].data_ptr(), xd[3].data_ptr(),
                                             ud[1].data_ptr(), ud[2].data_ptr(), ud[3].data_ptr(), h.data_ptr(),
                                             M, N, K, 128, split_k, None, 0, None)
        if st != 0:
            return st
    torch.cuda.synchronize()
    return bits(h)


def assert_swiglu_parity(h_bits, x, gate, up, rows=None):
    xs = x if rows is None else x[rows]
    h_ref, g_ref, A_g, u_ref, A_u = O.swiglu_reference(xs, gate, up)
    got = h_bits if rows is None else h_bits[rows]
    r = O.check_swiglu(got, g_ref, A_g, u_ref, A_u)
    assert r.ok, str(r)
    return r


@pytest.mark.parametrize("M,N,K,split", [
    (33, 96, 256, 0),          # ragged M and N, 64-row dequantizing tiles (one round)
    (1, 1000, 2560, 0),        # one row: 32-row tiles, policy split
    (20, 1000, 2560, 0),       # skinny rows, ragged N
    (128, 9728, 2560, 0),      # the 128-row gate / up shape (152 tiles: unsplit)
    (128, 2560, 4096, 0),      # 40 tiles of 32 groups: policy split (6 slices)
    (128, 2000, 1024, 1),      # forced: unsplit
    (70, 1100, 1024, 2),       # forced: two slices
    (70, 1100, 1024, 5),       # forced: five slices of 1 or 2 groups
    (35, 203, 1024, 3),        # forced: three slices, M x N odd
    (1500, 512, 384, 0),       # beyond 1024 rows, odd group count
    (250, 9728, 384, 0),       # 96-row dequantizing tiles (one round against two): ragged rows
    (90, 40000, 256, 0),       # 96-row tiles, ragged columns (40000 = 312 x 128 + 64)
])
def test_gate_up_swiglu_matches_oracle(lib, M, N, K, split):
    x, gate, up = gate_up_problem(21, M, N, K)
    h = run_gate_up(lib, x, gate, up, split)
    assert_swiglu_parity(h, x, gate, up)
    assert np.array_equal(run_gate_up(lib, x, gate, up, split), h), "repeat run differs"


def test_gate_up_swiglu_prefill512_sampled_rows(lib):
    # the 512-row layer shape (2560 -> 9728): every column of a row sample, rows across all tiles
    x, gate, up = gate_up_problem(22, 512, 9728, 2560)
    h = run_gate_up(lib, x, gate, up)
    assert_swiglu_parity(h, x, gate, up, rows=np.arange(0, 512, 37))


@pytest.mark.parametrize("M,N", [(3, 96),        # 32-row dequantizing tiles
                                 (40, 96),       # 64-row dequantizing tiles (one round)
                                 (640, 5472)])   # 64-row exact-code tiles
def test_gate_up_swiglu_saturation_closed_form(lib, M, N):
    # all-zero codes and x = 1: g[n] = 128 * sum_g b_gate[n, g], u[n] = 128 * sum_g b_up[n, g].
    # Gate sums of -256, 0 and +256 hit silu's exp overflow (silu -> -0), its zero and its
    # identity tail (silu(256) = 256 in fp32); every product is exact in bf16.
    K = 256
    G = K // 128
    x = synth.const_bf16(1.0, (M, K))
    bg_vals = np.array([-1.0, 0.0, 1.0])[np.arange(N) % 3]
    bg = np.repeat(bg_vals[:, None], G, axis=1).astype(np.float32)
    bu = synth.const_bf16(2.0 ** -7, (N, G))                  # u = 128 * 2^-7 * G = G
    zero = np.zeros((N, K // 8), dtype=np.uint32)
    gate = (zero, synth.const_bf16(1.0, (N, G)), synth.to_bf16_bits(bg))
    up = (zero, synth.const_bf16(1.0, (N, G)), bu)
    h = run_gate_up(lib, x, gate, up)
    g = 128.0 * G * bg_vals
    expect = np.where(g > 0, g * G, 0.0)
    got = synth.from_bf16_bits(h)
    assert np.array_equal(got, np.broadcast_to(expect, (M, N)).astype(got.dtype)), got[0, :6]
    assert_swiglu_parity(h, x, gate, up, rows=np.r_[0:M:max(1, M // 16), M - 1])


def test_gate_up_exact_code_and_dequantizing_forms(lib):
    # above 32 rows, with more than one 64-row tile per compute unit and no 96-row plan, the plan
    # runs the exact-code form; a call without workspace (no room for the activations' group
    # sums) runs the dequantizing tiles instead: both within the tolerance
    x, gate, up = gate_up_problem(25, 640, 5472, 512)
    assert lib.w4a16_gate_up_plan(640, 5472, 512, split_k=1)["variant"] >= 10
    assert lib.w4a16_gate_up_plan(128, 9728, 2560)["variant"] < 10          # one round: dequantizing
    h_codes = run_gate_up(lib, x, gate, up, split_k=1)
    h_deq = run_gate_up(lib, x, gate, up, split_k=1, workspace=None)
    rows = np.r_[0:640:7, 639]
    assert_swiglu_parity(h_codes, x, gate, up, rows=rows)
    assert_swiglu_parity(h_deq, x, gate, up, rows=rows)


def test_gate_up_long_prefill_sampled_rows(lib):
    # 4096 rows of the 2560 -> 9728 pair (exact-code tiles): every column of sampled rows
    x, gate, up = gate_up_problem(26, 4096, 9728, 2560)
    h = run_gate_up(lib, x, gate, up)
    assert_swiglu_parity(h, x, gate, up, rows=np.r_[0, 63, 64, 2047, 4032, 4095])


def test_gate_up_forced_split_without_workspace_is_rejected(lib):
    x, gate, up = gate_up_problem(23, 64, 256, 1024)
    assert run_gate_up(lib, x, gate, up, split_k=4, workspace=None) == 5      # W4A16_ERR_WORKSPACE


def test_gate_up_policy_split_without_workspace_falls_back(lib):
    # the policy splits this grid; without a workspace the unsplit plan runs and gives the
    # forced-unsplit result bit for bit
    x, gate, up = gate_up_problem(24, 32, 2048, 2560)
    assert lib.w4a16_gate_up_plan(32, 2048, 2560)["split_k"] > 1
    h = run_gate_up(lib, x, gate, up, split_k=0, workspace=None)
    assert np.array_equal(h, run_gate_up(lib, x, gate, up, split_k=1))
    assert_swiglu_parity(h, x, gate, up)


# ---------------------------------------------------------------------------------- exact-code mode
# Above 1024 rows the 128-row tiles multiply the raw codes on the matrix core and scale each
# group's fp32 product once (acc += s * P), adding sum_g b X from the activations' group sums;
# without workspace for those sums the plan falls back to dequantizing in registers.

def exact_code_plan(lib, M, N, K, split=0):
    p = lib.w4a16_plan(M, N, K, 128, lib.PATH_QMM if split else lib.PATH_AUTO, split)
    assert p["variant"] >= 10, "expected the exact-code mode"
    return p


def test_exact_code_mode_identity_is_bit_exact(lib):
    q, p = identity_problem(K=1152, N=96, seed=31)      # M = K = 1152 > 1024 rows
    exact_code_plan(lib, 1152, 96, 1152)
    y = run(lib, p, "linear")
    assert np.array_equal(y, synth.to_bf16_bits(q.T.astype(np.float32))), "exact-code unpack / indexing mismatch"


def test_exact_code_mode_power_of_two_affine_is_bit_exact(lib):
    # x = I, s = 2^-6, b = -8 * 2^-6: y[k, n] = (q[n, k] - 8) / 64 exactly (the bias term b * X
    # with X = 1 for the group holding k)
    K, N = 1280, 160
    q, p = identity_problem(K=K, N=N, seed=32)
    G = K // 128
    p["scales"], p["biases"] = synth.const_bf16(2.0 ** -6, (N, G)), synth.const_bf16(-8.0 * 2.0 ** -6, (N, G))
    exact_code_plan(lib, K, N, K)
    y = run(lib, p, "linear")
    assert np.array_equal(y, synth.to_bf16_bits(((q.T - 8) / 64.0).astype(np.float32)))


@pytest.mark.parametrize("split", [0, 2])
def test_exact_code_mode_bias_term_is_exact(lib, split):
    # s = 0 and small-integer activations: y = sum_g b[n, g] X[m, g] with exact group sums
    M, N, K = 1100, 130, 2560
    G = K // 128
    rng = np.random.default_rng(33)
    xv = rng.integers(-3, 4, (M, K)).astype(np.float32)
    bias = (((np.arange(N)[:, None] % 7) - 3) / 4.0 * np.where(np.arange(G)[None, :] % 2, -1.0, 1.0)).astype(np.float32)
    p = {"x": synth.to_bf16_bits(xv), "wq": synth.pack_codes(rng.integers(0, 16, (N, K))),
         "scales": synth.const_bf16(0.0, (N, G)), "biases": synth.to_bf16_bits(bias), "M": M, "N": N, "K": K}
    if split:
        exact_code_plan(lib, M, N, K, split)
    y = run(lib, p, "qmm" if split else "linear", split or None)
    X = xv.reshape(M, G, 128).sum(axis=2)
    assert np.array_equal(y, synth.to_bf16_bits((X @ bias.T).astype(np.float32)))


def test_exact_code_and_dequantizing_forms_match_the_oracle(lib):
    import torch
    p = synth.random_problem(34, 1500, 640, 2560)
    exact_code_plan(lib, 1500, 640, 2560)
    x, wq, s, b = to_device(p)
    announce("exact-code vs dequantizing form M=1500 N=640 K=2560")
    y_codes = lib.w4a16_linear(x, wq, s, b)
    y_deq = torch.empty_like(y_codes)
    st = lib.load().w4a16_linear(x.data_ptr(), wq.data_ptr(), s.data_ptr(), b.data_ptr(), y_deq.data_ptr(),
                                 1500, 640, 2560, 128, None, 0, None)   # no workspace: dequantizing form
    assert st == 0
    torch.cuda.synchronize()
    yc, yd = bits(y_codes), bits(y_deq)
    assert not np.array_equal(yc, yd), "both calls ran the same form"
    rows = sample_rows(1500, 16)
    rc, rd = assert_parity(yc, p, rows=rows), assert_parity(yd, p, rows=rows)
    announce(f"exact-code {rc}; dequantizing {rd}")
