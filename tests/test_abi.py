"""Host-side tests of the C ABI (``-m "not gpu"``): the library loads, exports every
declared symbol, and its policy and validation behave as documented.  Compute entry points
are only called with arguments that fail validation before any HIP call.
"""

import ctypes

import pytest

import w4a16_group_quantized_qmv_amd as w4

CUS = 256  # MI355X compute units; passed explicitly so no device is queried


@pytest.fixture(scope="module")
def lib():
    return w4.load()


def test_library_exports_every_declared_symbol(lib):
    names = w4.declared_symbols()
    assert set(names) >= {"w4a16_abi_version", "w4a16_status_string", "w4a16_plan", "w4a16_workspace_bytes",
                          "qmv_w4a16", "qmm_w4a16", "w4a16_linear", "w4a16_gate_up_plan", "w4a16_gate_up_swiglu"}
    for name in names:
        assert hasattr(lib, name), f"libw4a16.so does not export {name}"


def test_abi_version_and_status_strings():
    assert w4.w4a16_abi_version() == 1
    expect = ["W4A16_OK", "W4A16_ERR_NULL", "W4A16_ERR_SHAPE", "W4A16_ERR_GROUP", "W4A16_ERR_ALIGN",
              "W4A16_ERR_WORKSPACE", "W4A16_ERR_UNSUPPORTED", "W4A16_ERR_LAUNCH", "W4A16_ERR_DEVICE",
              "W4A16_ERR_OVERLAP"]
    assert [w4.w4a16_status_string(i) for i in range(10)] == expect
    assert w4.w4a16_status_string(99) == "unknown"


def test_time_next_launch_is_host_state_only(lib):
    """Arming and cancelling set only the calling thread's request (no HIP call, no device)."""
    import types
    try:
        assert lib.w4a16_time_next_launch(None, None) == w4.W4A16_OK
        assert lib.w4a16_time_next_launch(ctypes.c_void_p(0x1000), None) == w4.W4A16_OK
    finally:
        assert lib.w4a16_time_next_launch(None, None) == w4.W4A16_OK   # cancelled: nothing stays armed
    with pytest.raises(ValueError, match="record"):                     # an event never recorded has no handle
        w4.w4a16_time_next_launch(types.SimpleNamespace(cuda_event=0), None)


# ------------------------------------------------------------------------------ dispatch policy

def plan(M, N, K, path=0, split_k=0):
    return w4.w4a16_plan(M, N, K, 128, path, split_k, CUS)


def test_matvec_threshold_is_eight_rows():
    # "Week 2 Day 6: SIMD-Matrix Prefill", Task 1: M <= 8 -> matvec, M > 8 -> matrix kernels;
    # 8 < M <= 32 is the skinny regime (small-batch tiles with deterministic split-K)
    for M in range(1, 9):
        assert plan(M, 4096, 2560)["path"] == w4.PATH_QMV
    for M in (9, 16, 17, 32):
        assert plan(M, 4096, 2560)["path"] == w4.PATH_SKINNY
    for M in (33, 128, 512, 4096):
        assert plan(M, 4096, 2560)["path"] == w4.PATH_QMM


def test_skinny_plans():
    # up to 16 rows: the matvec kernels (tile_m = 16, no split); above: 32-row tiles
    for M in (9, 12, 16):
        p = plan(M, 4096, 2560)
        assert p["tile_m"] == 16 and p["split_k"] == 1 and p["workspace_bytes"] == 0
    for M in (17, 24, 32):
        p = plan(M, 4096, 2560)
        assert p["tile_m"] == 32 and p["grid_y"] == 1
    # skinny split: about one work unit per compute unit, at most 8 slices of >= 2 groups
    assert plan(32, 9728, 2560)["split_k"] == CUS // 76          # 76 tiles of 32 x 128
    assert plan(32, 2560, 9728)["split_k"] == 8                  # 20 tiles, K = 9728
    assert plan(32, 1024, 256)["split_k"] == 1                   # two groups: nothing to split
    assert plan(32, 151936, 2560)["split_k"] == 1                # 1187 tiles fill the GPU
    # a 16-row wide head would leave one workgroup per compute unit: 32-row tiles instead
    assert plan(16, 151936, 2560)["tile_m"] == 32
    assert plan(9, 151936, 2560)["tile_m"] == 16
    # the forced skinny path serves any M <= 32 and nothing above
    assert plan(4, 4096, 2560, path=w4.PATH_SKINNY)["path"] == w4.PATH_SKINNY
    with pytest.raises(NotImplementedError):
        plan(33, 4096, 2560, path=w4.PATH_SKINNY)
    # workspace sizing follows the skinny split
    p = plan(32, 2560, 9728)
    assert p["workspace_bytes"] == 8 * 32 * 2560 * 4
    assert w4.w4a16_workspace_bytes(32, 2560, 9728, 128, CUS) == p["workspace_bytes"]


def test_forced_paths():
    assert plan(4, 1024, 256, path=w4.PATH_QMM)["path"] == w4.PATH_QMM
    with pytest.raises(NotImplementedError):
        plan(9, 1024, 256, path=w4.PATH_QMV)
    with pytest.raises(NotImplementedError):
        plan(9, 1024, 256, path=7)


def test_grid_covers_the_output():
    for M, N, K in [(33, 96, 256), (509, 9728, 2560), (128, 1024, 2560), (4096, 151936, 2560), (1, 151936, 2560)]:
        p = plan(M, N, K)
        if p["path"] == w4.PATH_QMV and p["grid_x"] * p["tile_n"] < N:
            # persistent wide matvec: resident workgroups whose waves loop over 16-column blocks
            waves_per_wg = p["block_threads"] // 64
            assert waves_per_wg == (8 if M <= 4 else 4)      # eight-wave workgroups up to 4 rows
            assert p["tile_n"] == 16 and p["k_waves"] == 1
            assert p["grid_x"] == min(-(-N // (16 * waves_per_wg)), 32 // waves_per_wg * CUS)
            continue
        assert p["grid_x"] * p["tile_n"] >= N and (p["grid_x"] - 1) * p["tile_n"] < N
        if p["path"] == w4.PATH_QMM:
            assert p["grid_y"] * p["tile_m"] >= M and (p["grid_y"] - 1) * p["tile_m"] < M
        assert p["tile_k"] == 128 and p["num_cus"] == CUS


def test_burst_matvec_plans():
    # up to 4 rows below 2048 column blocks of 16, and 5 to 8 rows below 1024 blocks up to 64
    # groups (16 columns, 8 row slots, g = 2 groups per wave or ceil(G / 16)): the burst
    # kernel.  Packed form (4 columns per
    # workgroup, steps of 4 groups: one per wave below 1024 blocks up to 64 groups, two
    # otherwise) at 1 and 2 rows up to 128 groups, and at 3 and 4 rows up to 160 blocks and 64
    # groups; otherwise, at 3 and 4 rows up to 80 groups and not from 1024 blocks at 32 groups,
    # 16 columns per workgroup with g = 2 groups per wave (3 from 1024 blocks), at least
    # ceil(G / 16)
    for M, N, K, cols, waves, per_wave in [
            (1, 9728, 2560, 4, 5, 4), (2, 9728, 2560, 4, 5, 4), (4, 9728, 2560, 16, 10, 2),
            (1, 4096, 2560, 4, 5, 4), (1, 1024, 2560, 4, 5, 4), (4, 1024, 2560, 4, 5, 4),
            (1, 2560, 9728, 4, 10, 8), (3, 2560, 9728, 16, 16, 5), (3, 2600, 8192, 16, 16, 4),
            (3, 2560, 8192, 4, 16, 4), (2, 1000, 10240, 4, 10, 8), (1, 96, 128, 4, 1, 4),
            (4, 2560, 4096, 4, 8, 4), (1, 16400, 2560, 4, 3, 8), (2, 24600, 384, 4, 1, 8),
            (1, 26608, 2560, 4, 3, 8), (4, 16368, 4096, 16, 16, 2), (3, 16400, 2560, 16, 7, 3),
            (1, 32752, 4096, 4, 4, 8), (1, 30000, 384, 4, 1, 8),
            (1, 16400, 9728, 4, 10, 8), (2, 1000, 16384, 4, 16, 8), (1, 24600, 9728, 4, 10, 8),
            (5, 9728, 2560, 16, 10, 2), (8, 4096, 2560, 16, 10, 2), (6, 2600, 8192, 16, 16, 4),
            (8, 96, 128, 16, 1, 2), (7, 9728, 4096, 16, 16, 2)]:
        p = plan(M, N, K)
        G = K // 128
        assert p["variant"] == 4, (M, N, K)                  # the burst kernel's instance index
        assert (p["tile_n"], p["k_waves"], p["block_threads"]) == (cols, waves, 64 * waves), (M, N, K)
        assert (p["grid_x"], p["workspace_bytes"]) == (-(-N // cols), 0)
        assert waves * per_wave >= G and waves <= 16
    # more rows, 2048 blocks or more, more groups than the forms take, 1024 blocks at 32 groups
    # or more above 2 rows, and 1024 blocks at 5 to 8 rows keep the other families
    assert plan(8, 2560, 9728)["variant"] == 0          # 76 groups at 8 rows
    assert plan(8, 16400, 384)["variant"] == 1
    assert plan(9, 9728, 2560, path=w4.PATH_SKINNY)["variant"] == 3
    assert plan(1, 1000, 16512)["variant"] == 0          # 129 groups
    assert plan(3, 1000, 10368)["variant"] == 0          # 81 groups at 3 rows
    assert plan(5, 16400, 384)["variant"] == 1
    assert plan(1, 32768, 2560)["variant"] == 2          # 2048 blocks
    assert plan(1, 26624, 2560)["variant"] == 2          # 1664 blocks under 32 groups
    assert plan(4, 16400, 4096)["variant"] == 2          # 1025 blocks at 32 groups, 4 rows
    assert plan(3, 24600, 9728)["variant"] == 2
    assert plan(1, 151936, 2560)["variant"] == 2


def test_k_split_waves_for_small_grids():
    # at most one work unit per compute unit: the 64 x 128 tiles run with two waves per column
    # strip (k_waves = 2, 8-wave workgroups); larger grids keep four waves
    q = plan(512, 4096, 2560)                      # 256 tiles, unsplit
    assert (q["tile_m"], q["tile_n"], q["k_waves"], q["block_threads"]) == (64, 128, 2, 512)
    k = plan(512, 1024, 2560)                      # 64 tiles x 4 slices
    assert k["k_waves"] == 2 and k["grid_x"] * k["grid_y"] * k["split_k"] <= CUS
    for M, N, K in [(512, 2560, 4096), (2048, 9728, 2560), (32, 9728, 2560), (384, 9728, 2560)]:
        p = plan(M, N, K)
        assert p["k_waves"] == 1 and p["block_threads"] == 256, (M, N, K)


def test_96_row_tiles_when_they_need_fewer_rounds():
    # unsplit grids: 96 x 128 tiles with two waves per strip (two resident per compute unit) when
    # their rounds of tiles per compute unit are fewer than the 64-row tiles' and at most two
    def rounds(M, N, bm):
        return -(-(-(-M // bm) * -(-N // 128)) // CUS)

    for M, N in [(512, 9728), (509, 9728), (256, 9728), (192, 16384)]:
        p = plan(M, N, 2560)
        assert rounds(M, N, 96) < rounds(M, N, 64) and rounds(M, N, 96) <= 2, (M, N)
        assert (p["tile_m"], p["tile_n"], p["k_waves"], p["block_threads"], p["split_k"]) == (96, 128, 2, 512, 1)
        assert p["grid_y"] == -(-M // 96) and p["grid_x"] == -(-N // 128)
    # as many rounds (384 rows), more than two (1024 rows), split grids and one tile per unit: 64 rows
    for M, N, K in [(384, 9728, 2560), (1024, 9728, 2560), (512, 12288, 2560), (512, 2560, 9728),
                    (512, 4096, 2560), (128, 9728, 2560)]:
        assert plan(M, N, K)["tile_m"] == 64, (M, N, K)


def test_split_k_only_for_under_filled_grids():
    # "Benchmark Analysis: Identify Under-Filled Prefill Shapes": the short, narrow K/V
    # projection (32 rows, N = 1024) has too few tiles and gains from split-K ...
    short = plan(32, 1024, 2560)
    assert short["split_k"] > 1
    # ... while a long, occupied grid (2048 rows) is left unsplit (split-K "neutral" at long M)
    assert plan(2048, 9728, 2560)["split_k"] == 1
    assert plan(2048, 2560, 9728)["split_k"] == 1
    # the pages' own geometry: 32 x 32 tiles give the unsplit 32-row K projection 32 groups
    assert -(-32 // 32) * -(-1024 // 32) == 32


def test_split_k_slices_keep_several_groups():
    for M, N, K in [(128, 1024, 2560), (128, 2560, 9728), (512, 2560, 9728), (64, 96, 1024), (16, 128, 4096)]:
        p = plan(M, N, K)
        G = K // 128
        tiles = p["grid_x"] * p["grid_y"]
        assert p["grid_z"] == p["split_k"]
        if p["split_k"] > 1:
            assert tiles < CUS
            assert G // p["split_k"] >= 4
            assert p["workspace_bytes"] == p["split_k"] * M * N * 4
        else:
            assert p["workspace_bytes"] == 0


def test_forced_split_is_clamped_to_the_group_count():
    assert plan(128, 1024, 256, path=w4.PATH_QMM, split_k=64)["split_k"] == 2
    assert plan(128, 1024, 2560, path=w4.PATH_QMM, split_k=3)["split_k"] == 3
    assert plan(128, 1024, 2560, path=w4.PATH_QMM, split_k=1)["split_k"] == 1


def test_long_k_down_projection_splits_at_512_rows():
    # 512-row down projection (K = 9728, 76 groups) has fewer tiles than compute units
    p = plan(512, 2560, 9728)
    assert p["split_k"] > 1 and p["grid_x"] * p["grid_y"] * p["split_k"] >= CUS


def test_workspace_bytes_matches_plan():
    for M, N, K in [(1, 9728, 2560), (128, 1024, 2560), (512, 2560, 9728), (4096, 9728, 2560)]:
        assert w4.w4a16_workspace_bytes(M, N, K, 128, CUS) == plan(M, N, K)["workspace_bytes"]
    assert w4.w4a16_workspace_bytes(0, 10, 128, 128, CUS) == 0
    assert w4.w4a16_workspace_bytes(4, 10, 100, 128, CUS) == 0


@pytest.mark.parametrize("args,err", [
    ((0, 10, 128, 128), ValueError), ((4, 0, 128, 128), ValueError), ((4, 10, 0, 128), ValueError),
    ((4, 10, 100, 128), ValueError), ((4, 10, 256, 64), ValueError), ((4, 10, 2 ** 31, 128), ValueError),
    ((4, 10, 2 ** 20 + 128, 128), ValueError),
])
def test_plan_rejects_invalid_shapes(args, err):
    with pytest.raises(err):
        w4.w4a16_plan(*args, 0, 0, CUS)


def test_plan_rejects_null_output(lib):
    assert lib.w4a16_plan(4, 10, 128, 128, 0, 0, CUS, None) == 1
    assert lib.w4a16_plan(4, 10, 128, 128, 0, -1, CUS, ctypes.byref(w4.Plan())) == 2


# ------------------------------------------------------------------------------ validation before launch

# fake, 16-byte aligned addresses 16 MiB apart (one per buffer, so no two overlap): validation
# fails before they could be used
X, WQ, S, B, Y, WS = (i << 24 for i in range(1, 7))
WU, SU, BU = (i << 24 for i in range(7, 10))
ODD = X + 8


@pytest.mark.parametrize("fn", ["qmv", "qmm", "linear"])
def test_compute_entry_points_validate_before_launch(lib, fn):
    def call(x=X, wq=WQ, s=S, b=B, y=Y, M=4, N=16, K=256, group=128):
        if fn == "qmv":
            return lib.qmv_w4a16(x, wq, s, b, y, M, N, K, group, None)
        if fn == "qmm":
            return lib.qmm_w4a16(x, wq, s, b, y, M, N, K, group, 1, None, 0, None)
        return lib.w4a16_linear(x, wq, s, b, y, M, N, K, group, None, 0, None)

    assert call(x=None) == 1 and call(wq=None) == 1 and call(s=None) == 1 and call(b=None) == 1 and call(y=None) == 1
    assert call(M=0) == 2 and call(N=-1) == 2 and call(K=100) == 2 and call(K=0) == 2
    assert call(group=64) == 3
    assert call(x=ODD) == 4 and call(wq=WQ + 8) == 4
    assert call(s=S + 1) == 4 and call(y=Y + 1) == 4
    # the output may not share a byte with an input (x is 4 x 256 bf16 = 2 KiB; wq 16 x 128 B)
    assert call(y=X) == 9 and call(y=X + 2046) == 9 and call(y=WQ + 1024) == 9 and call(y=S) == 9 and call(y=B) == 9


def test_qmv_rejects_more_than_eight_rows(lib):
    assert lib.qmv_w4a16(X, WQ, S, B, Y, 9, 16, 256, 128, None) == 6


def test_negative_split_is_a_shape_error(lib):
    assert lib.qmm_w4a16(X, WQ, S, B, Y, 16, 16, 256, 128, -2, None, 0, None) == 2


# ------------------------------------------------------------------------------ fused gate / up + SwiGLU

def gate_up_plan(M, N, K, split_k=0):
    return w4.w4a16_gate_up_plan(M, N, K, 128, split_k, CUS)


def test_gate_up_plan_tiles_and_workspace():
    # 32-row tiles up to 32 rows (dequantizing); above, 64-row tiles in the exact-code form, except
    # unsplit grids that dequantizing 96-row tiles cover in fewer rounds per compute unit (<= 2)
    r256 = lambda v: -(-v // 256) * 256
    for M, tile_m in [(1, 32), (32, 32), (33, 64), (256, 96), (384, 64), (512, 96), (1024, 64), (1025, 64),
                      (4096, 64)]:
        p = gate_up_plan(M, 9728, 2560)
        assert p["path"] == w4.PATH_GATE_UP and p["tile_m"] == tile_m and p["tile_n"] == 128, M
        assert p["grid_x"] == -(-9728 // 128) and p["grid_y"] == -(-M // tile_m)
        codes = M > 32 and tile_m == 64 and p["grid_x"] * p["grid_y"] * p["split_k"] > CUS
        assert (p["variant"] >= 10) == codes
        # the workspace holds the group sums (exact-code form), then gate and up partials
        sums = r256(M * w4.w4a8_xsum_cols(2560) * 2) if codes else 0
        assert p["workspace_bytes"] == sums + (2 * p["split_k"] * M * 9728 * 4 if p["split_k"] > 1 else 0)
        if tile_m == 96:
            assert p["variant"] == 3 and p["split_k"] == 1
    # the split follows the projection's rule on the same tile grid
    for M, N, K in [(128, 9728, 2560), (512, 9728, 2560), (512, 2560, 9728), (16, 1024, 2560)]:
        g, q = gate_up_plan(M, N, K), plan(M, N, K, path=w4.PATH_QMM if M > 32 else w4.PATH_SKINNY)
        assert g["split_k"] == q["split_k"] or M <= 16       # 9..16 rows: the skinny plan is a matvec
    assert gate_up_plan(128, 1024, 2560, split_k=3)["split_k"] == 3
    assert gate_up_plan(128, 1024, 256, split_k=64)["split_k"] == 2


def test_gate_up_validates_before_launch(lib):
    def call(x=X, wg=WQ, sg=S, bg=B, wu=WU, su=SU, bu=BU, h=Y, M=4, N=16, K=256, group=128, split=1):
        return lib.w4a16_gate_up_swiglu(x, wg, sg, bg, wu, su, bu, h, M, N, K, group, split, None, 0, None)

    for kw in ("x", "wg", "sg", "bg", "wu", "su", "bu", "h"):
        assert call(**{kw: None}) == 1, kw
    assert call(M=0) == 2 and call(K=100) == 2 and call(split=-1) == 2
    assert call(group=64) == 3
    assert call(wu=WU + 8) == 4 and call(su=SU + 1) == 4 and call(h=Y + 1) == 4
    for kw, base in (("x", X), ("wg", WQ), ("sg", S), ("bg", B), ("wu", WU), ("su", SU), ("bu", BU)):
        assert call(h=base) == 9, kw                                # h may not overlap any input
    with pytest.raises(ValueError):
        w4.w4a16_gate_up_plan(4, 16, 100, 128, 0, CUS)


# ------------------------------------------------------------------------------ width-generic matvec

def test_qmv_affine_plans():
    # measured routing: qmv_w4a16's policy at 4 bits; at 1, 2, 3 and 8 bits the burst forms where
    # they apply (packed: at most 4 rows, below 2048 column blocks of 16 and 128 groups, beyond
    # 160 blocks or 64 groups only up to 2 rows; 16 columns: 3 to 8 rows below 1024 blocks, up
    # to 80 groups at 3-4 rows and 64 at 5-8), the row-amortized kernel elsewhere
    for bits in w4.BITS:
        for M in range(1, 9):
            for N, K in [(4000, 2560), (151936, 2560), (2560, 9728), (1000, 16384), (2000, 8192), (20000, 4096)]:
                p = w4.qmv_affine_plan(M, N, K, bits, w4.QMV_POLICY, 128, CUS)
                assert p["path"] == w4.PATH_QMV and p["workspace_bytes"] == 0
                blocks, G = -(-N // 16), K // 128
                packed = M <= 4 and blocks < 2048 and G <= 128 and (M <= 2 or (blocks <= 160 and G <= 64))
                wide16 = not packed and 3 <= M <= 8 and blocks < 1024 and G <= (80 if M <= 4 else 64)
                burst = packed or wide16
                if bits == 4:
                    q = plan(M, N, K, path=w4.PATH_QMV) if G <= 8192 else None
                    assert p["variant"] == w4.QMV_FAMILIES
                    assert (p["tile_n"], p["grid_x"], p["k_waves"]) == (q["tile_n"], q["grid_x"], q["k_waves"])
                elif packed:
                    steps = 2 if G > 64 or blocks >= 1024 else 1
                    assert p["variant"] == w4.QMV_BURST, (bits, M, N, K)
                    assert (p["tile_n"], p["grid_x"]) == (4, -(-N // 4))
                    assert p["k_waves"] == -(-G // (4 * steps)) and p["block_threads"] == 64 * p["k_waves"]
                    assert p["tile_m"] == (1 if M == 1 else 2 if M == 2 else 4)
                elif wide16:
                    per_wave = max(2, -(-G // 16))
                    assert p["variant"] == w4.QMV_BURST, (bits, M, N, K)
                    assert (p["tile_n"], p["grid_x"], p["tile_m"]) == (16, -(-N // 16), 4 if M <= 4 else 8)
                    assert p["k_waves"] == -(-G // per_wave) and p["block_threads"] == 64 * p["k_waves"]
                else:
                    assert p["variant"] == w4.QMV_AMORTIZED, (bits, M, N, K)
                    assert p["tile_n"] == 16 and p["grid_x"] == -(-N // 16)
        for mode in (w4.QMV_AMORTIZED, w4.QMV_PER_ROW, w4.QMV_BURST):
            assert w4.qmv_affine_plan(2, 4000, 2560, bits, mode, 128, CUS)["variant"] == mode
        # the forced burst form outside its shapes
        for M, N, K in [(5, 20000, 2560), (1, 32768, 2560), (3, 4000, 10368), (6, 1000, 8320), (1, 1000, 16512)]:
            with pytest.raises(NotImplementedError):
                w4.qmv_affine_plan(M, N, K, bits, w4.QMV_BURST, 128, CUS)


@pytest.mark.parametrize("args", [
    (1, 16, 256, 5, 0), (1, 16, 256, 16, 0), (1, 16, 256, 0, 0),   # widths outside {1, 2, 3, 4, 8}
    (9, 16, 256, 4, 0),                                            # more than eight rows
    (3, 16, 256, 4, w4.QMV_PER_ROW),                               # per-row kernel: M <= 2
    (1, 16, 256, 2, w4.QMV_FAMILIES),                              # the 4-bit families: bits = 4
    (3, 16, 10368, 2, w4.QMV_BURST),                               # burst forms: at most 80 groups at 3 rows
    (1, 16, 256, 4, 5), (1, 16, 256, 4, -1),                       # unknown mode
])
def test_qmv_affine_rejects_unsupported(lib, args):
    M, N, K, bits, mode = args
    with pytest.raises(NotImplementedError):
        w4.qmv_affine_plan(M, N, K, bits, mode, 128, CUS)
    assert lib.qmv_affine(X, WQ, S, B, Y, M, N, K, 128, bits, mode, None) == 6


def test_qmv_affine_validates_before_launch(lib):
    def call(x=X, wq=WQ, s=S, b=B, y=Y, M=2, N=16, K=256, group=128, bits=2, mode=0):
        return lib.qmv_affine(x, wq, s, b, y, M, N, K, group, bits, mode, None)

    assert call(x=None) == 1 and call(wq=None) == 1 and call(s=None) == 1 and call(b=None) == 1 and call(y=None) == 1
    assert call(M=0) == 2 and call(N=-1) == 2 and call(K=100) == 2 and call(K=2 ** 20 + 128) == 2
    assert call(group=64) == 3
    assert call(x=ODD) == 4 and call(wq=WQ + 8) == 4 and call(s=S + 1) == 4 and call(y=Y + 1) == 4
    # 2-bit codes: wq is 16 x 64 bytes, so an output at +1000 overlaps it
    assert call(y=WQ + 1000) == 9
    assert lib.qmv_affine_plan(1, 16, 256, 128, 4, 0, CUS, None) == 1


# ------------------------------------------------------------------------------ W4A8

def test_w4a8_plan_tiles_split_and_workspace():
    for M, tile_m in [(1, 32), (32, 32), (33, 64), (512, 64), (1024, 64), (1025, 128), (4096, 128)]:
        p = w4.w4a8_plan(M, 9728, 2560, 128, 0, CUS)
        assert p["path"] == w4.PATH_W4A8 and p["tile_m"] == tile_m and p["tile_n"] == 128
        assert p["grid_x"] == -(-9728 // 128) and p["grid_y"] == -(-M // tile_m)
        assert p["workspace_bytes"] == (p["split_k"] * M * 9728 * 4 if p["split_k"] > 1 else 0)
    # the split rule of the W4A16 tiles: only under-filled grids with enough groups
    assert w4.w4a8_plan(4096, 9728, 2560, 128, 0, CUS)["split_k"] == 1
    assert w4.w4a8_plan(512, 2560, 9728, 128, 0, CUS)["split_k"] > 1
    assert w4.w4a8_plan(33, 96, 256, 128, 0, CUS)["split_k"] == 1          # G = 2: never split
    assert w4.w4a8_plan(128, 1024, 2560, 128, 3, CUS)["split_k"] == 3
    assert w4.w4a8_plan(128, 1024, 256, 128, 64, CUS)["split_k"] == 2       # clamped to G


def test_w4a8_k_split_waves_for_small_grids():
    # at most one work unit per compute unit: 64-row tiles with two waves per column block
    q = w4.w4a8_plan(512, 4096, 2560, 128, 0, CUS)                 # 256 tiles, unsplit
    assert (q["tile_m"], q["tile_n"], q["k_waves"], q["block_threads"]) == (64, 128, 2, 512)
    for M, N in [(512, 9728), (2048, 9728), (32, 9728)]:
        p = w4.w4a8_plan(M, N, 2560, 128, 0, CUS)
        assert p["k_waves"] == 1 and p["block_threads"] == 256, (M, N)


def test_w4a8_xsum_columns_and_linear_workspace():
    # two bf16 halves per group, rounded up to the 16-value MFMA step
    for K, cols in [(128, 16), (256, 16), (1024, 16), (1152, 32), (2560, 48), (4096, 64), (9728, 160)]:
        assert w4.w4a8_xsum_cols(K) == cols
    assert w4.w4a8_xsum_cols(100) == 0 and w4.w4a8_xsum_cols(0) == 0
    r256 = lambda v: -(-v // 256) * 256
    for M, N, K in [(33, 96, 256), (512, 9728, 2560), (512, 2560, 9728)]:
        act = r256(M * K) + r256(M * 4) + r256(M * w4.w4a8_xsum_cols(K) * 2)
        assert w4.w4a8_linear_workspace_bytes(M, N, K, 128, CUS) == act + w4.w4a8_plan(M, N, K, 128, 0, CUS)[
            "workspace_bytes"]


def test_w4a8_entry_points_validate_before_launch(lib):
    def quant(x=X, xq=WQ, sx=S, xs=B, M=4, K=256, group=128):
        return lib.w4a8_quantize_rows(x, xq, sx, xs, M, K, group, None)

    assert quant(x=None) == 1 and quant(xq=None) == 1 and quant(sx=None) == 1 and quant(xs=None) == 1
    assert quant(M=0) == 2 and quant(K=100) == 2 and quant(group=64) == 3
    assert quant(x=ODD) == 4 and quant(xq=WQ + 8) == 4 and quant(xs=B + 8) == 4 and quant(sx=S + 2) == 4
    assert quant(xq=X + 1024) == 9 and quant(sx=X) == 9 and quant(xs=WQ + 16) == 9 and quant(sx=WQ + 1020) == 9

    def qmm(xq=X, sx=WS, xs=WU, wq=WQ, s=S, b=B, y=Y, M=4, N=16, K=256, group=128, split=1):
        return lib.qmm_w4a8(xq, sx, xs, wq, s, b, y, M, N, K, group, split, None, 0, None)

    for kw in ("xq", "sx", "xs", "wq", "s", "b", "y"):
        assert qmm(**{kw: None}) == 1, kw
    assert qmm(M=0) == 2 and qmm(K=100) == 2 and qmm(split=-1) == 2 and qmm(group=64) == 3
    assert qmm(xq=ODD) == 4 and qmm(wq=WQ + 8) == 4 and qmm(y=Y + 1) == 4
    for kw, base in (("xq", X), ("sx", WS), ("xs", WU), ("wq", WQ), ("s", S), ("b", B)):
        assert qmm(y=base) == 9, kw

    def linear(x=X, wq=WQ, s=S, b=B, y=Y, M=4, N=16, K=256, ws=WS, nbytes=1 << 20):
        return lib.w4a8_linear(x, wq, s, b, y, M, N, K, 128, ws, nbytes, None)

    assert linear(x=None) == 1 and linear(M=0) == 2 and linear(x=ODD) == 4
    assert linear(ws=None) == 5 and linear(nbytes=100) == 5 and linear(ws=WS + 16) == 4
    assert linear(y=X + 512) == 9


def test_exact_code_mode_plans():
    # above 1024 rows the 128-row tiles run the exact-code mode: the plan reports the tile
    # variant + 10 and the workspace starts with the activations' group sums (bf16 [M, KB])
    r256 = lambda v: -(-v // 256) * 256
    for M, N, K in [(1025, 9728, 2560), (4096, 2560, 9728), (4096, 151936, 2560), (2048, 1024, 256)]:
        p = plan(M, N, K)
        assert p["path"] == w4.PATH_QMM and p["tile_m"] == 128 and p["variant"] >= 10
        sums = r256(M * w4.w4a8_xsum_cols(K) * 2)
        parts = p["split_k"] * M * N * 4 if p["split_k"] > 1 else 0
        assert p["workspace_bytes"] == sums + parts
        assert w4.w4a16_workspace_bytes(M, N, K, 128, CUS) == p["workspace_bytes"]
    # 1024 rows and fewer dequantize in registers (no group sums)
    for M in (33, 512, 1024):
        p = plan(M, 9728, 2560)
        assert p["variant"] < 10
        assert p["workspace_bytes"] == (p["split_k"] * M * 9728 * 4 if p["split_k"] > 1 else 0)
    # the fused gate / up pair runs the exact-code form on its 64-row tiles above 32 rows
    assert gate_up_plan(4096, 9728, 2560)["variant"] == 11 and gate_up_plan(1024, 9728, 2560)["variant"] == 11
    assert gate_up_plan(512, 9728, 2560)["variant"] == 3                 # 96-row dequantizing tiles
    assert gate_up_plan(32, 9728, 2560)["variant"] < 10


# ------------------------------------------------------------------------------ grouped projections of one input

def grouped_plan(N, M, K):
    return w4.w4a16_grouped_plan(N, M, K, 128, CUS)


def test_grouped_plan_one_launch_over_the_column_tiles():
    # "Week 2 Day 6: SIMD-Matrix Prefill", Benchmark Analysis: the short key / value projections
    # under-fill the GPU alone; grouped with the query projection their tiles share one grid
    qkv = [4096, 1024, 1024]
    for M in (33, 128, 509, 512, 1024, 4096):
        p = grouped_plan(qkv, M, 2560)
        alone = plan(M, 6144, 2560)        # the tile form and split of one 6144-column projection
        assert p["path"] == w4.PATH_GROUPED and p["grid_z"] == p["split_k"]
        assert p["grid_x"] == 48 and p["grid_y"] == -(-M // p["tile_m"])
        assert (p["tile_m"], p["tile_n"], p["variant"], p["block_threads"], p["split_k"]) == \
            (alone["tile_m"], alone["tile_n"], alone["variant"], alone["block_threads"], alone["split_k"])
        # the partials of every projection in one [S][M][48 * 128] array
        assert p["workspace_bytes"] == alone["workspace_bytes"]
    # an under-filled grid splits (96 tiles at 128 rows), a filled one does not
    assert grouped_plan(qkv, 128, 2560)["split_k"] > 1 and grouped_plan(qkv, 512, 2560)["split_k"] == 1
    # ragged projections: each owns ceil(N / 128) column tiles
    assert grouped_plan([200, 96, 1000], 509, 256)["grid_x"] == 2 + 1 + 8
    # the exact-code form above 1024 rows: the group sums of the shared x, once
    p = grouped_plan(qkv, 4096, 2560)
    assert p["variant"] >= 10 and p["workspace_bytes"] == -(-4096 * w4.w4a8_xsum_cols(2560) * 2 // 256) * 256


def test_grouped_plan_per_projection_for_few_rows():
    # at most 32 rows (matvec and skinny paths) and for one projection: each projection's own dispatch
    for M in (1, 8, 16, 32):
        p = grouped_plan([4096, 1024, 1024], M, 2560)
        assert p["path"] == w4.PATH_PER_PROJECTION
        assert p["workspace_bytes"] == max(plan(M, n, 2560)["workspace_bytes"] for n in (4096, 1024, 1024))
        first = plan(M, 4096, 2560)
        assert p["variant"] == first["variant"] and p["tile_m"] == first["tile_m"]
    assert grouped_plan([2560], 512, 9728) == plan(512, 2560, 9728)


@pytest.mark.parametrize("N,err", [([], 2), ([64] * 5, 2), ([64, 0], 2), ([64, 64], 0)])
def test_grouped_plan_counts(N, err, lib):
    arr = (ctypes.c_int64 * max(1, len(N)))(*N)
    assert lib.w4a16_grouped_plan(len(N), arr, 64, 256, 128, CUS, ctypes.byref(w4.Plan())) == err
    assert lib.w4a16_grouped_plan(2, None, 64, 256, 128, CUS, ctypes.byref(w4.Plan())) == 1
    assert lib.w4a16_grouped_plan(2, arr, 64, 256, 64, CUS, ctypes.byref(w4.Plan())) in (2, 3)


def test_grouped_call_validates_before_launch(lib):
    # two projections at fake addresses: x, then per projection wq / s / b / y (16 MiB apart)
    P = ctypes.c_void_p * 2
    wq2, s2, b2, y2 = (i << 24 for i in range(10, 14))

    def call(x=X, wq=(WQ, wq2), s=(S, s2), b=(B, b2), y=(Y, y2), N=(64, 32), M=40, K=256, group=128, count=2):
        arrs = [None if v is None else P(*v) for v in (wq, s, b, y)]
        n = None if N is None else (ctypes.c_int64 * 2)(*N)
        return lib.w4a16_linear_grouped(x, count, *arrs, n, M, K, group, None, 0, None)

    assert call(wq=None) == 1 and call(y=None) == 1 and call(N=None) == 1
    assert call(x=None) == 1 and call(wq=(WQ, None)) == 1 and call(y=(None, y2)) == 1
    assert call(count=0) == 2 and call(count=5) == 2
    assert call(N=(64, 0)) == 2 and call(K=100) == 2 and call(group=64) == 3
    assert call(x=ODD) == 4 and call(s=(S, s2 + 1)) == 4
    # an output may share no byte with an input of its own projection or another one, nor with
    # another output (y0 is 40 x 64 bf16 = 5 KiB, y1 40 x 32 bf16 = 2.5 KiB)
    assert call(y=(X, y2)) == 9
    assert call(y=(Y, wq2)) == 9 and call(y=(Y, s2 + 2)) == 9 and call(y=(b2, y2)) == 9
    assert call(y=(Y, Y + 4096)) == 9 and call(y=(Y + 2048, Y)) == 9
