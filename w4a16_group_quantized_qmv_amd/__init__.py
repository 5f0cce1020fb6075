"""MI355X-native W4A16 group-quantized projection: Python binding of ``libw4a16.so``.

The functions below have the names of the C ABI (``include/w4a16.h``) and only marshal
arguments: tensor checks, pointers, the current HIP stream, and output / workspace
allocation through torch.  Every step of the projection runs in the library's HIP kernels.
There is no fallback: if the library is not built, every compute call raises.

Tensor conventions (all on the GPU, contiguous):
    x        torch.bfloat16 [M, K]
    wq       torch.int32    [N, K/8]   packed codes, read as uint32 (low nibble first)
    scales   torch.bfloat16 [N, K/128]
    biases   torch.bfloat16 [N, K/128]
    y        torch.bfloat16 [M, N]

``qmv_affine`` takes codes of 1, 2, 3, 4 or 8 bits: ``wq`` int32 [N, K*bits/32], a row's words one
bit stream, lowest bits first.

``linear(..., logits_to_keep=k)`` is the model-level entry: it projects only the last ``k``
rows (a view, no copy) before the projection, as tiny-llm's "Week 2 Day 6: SIMD-Matrix
Prefill", Task 4 does before the vocabulary head; ``k = 0`` projects every row.
"""

from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "W4A16_OK", "PATH_AUTO", "PATH_QMV", "PATH_QMM", "PATH_SKINNY", "PATH_GATE_UP", "GROUP",
    "load", "lib_path", "w4a16_abi_version", "w4a16_status_string", "w4a16_plan", "w4a16_workspace_bytes",
    "qmv_w4a16", "qmm_w4a16", "w4a16_linear", "w4a16_linear_noalloc", "NOALLOC_SCRATCH_BYTES", "linear", "W4A16Error", "declared_symbols", "PreparedLinear",
    "w4a16_gate_up_plan", "w4a16_gate_up_swiglu", "PreparedGateUp",
    "qmv_affine", "qmv_affine_plan", "QMV_POLICY", "QMV_AMORTIZED", "QMV_PER_ROW", "QMV_FAMILIES", "QMV_BURST", "BITS",
    "PATH_W4A8", "w4a8_xsum_cols", "w4a8_quantize_rows", "w4a8_plan", "qmm_w4a8", "w4a8_linear_workspace_bytes",
    "w4a8_linear", "PreparedW4A8",
    "PATH_GROUPED", "PATH_PER_PROJECTION", "MAX_GROUPED", "w4a16_grouped_plan", "w4a16_linear_grouped",
    "PreparedGrouped",
]

GROUP = 128
W4A16_OK = 0
PATH_AUTO, PATH_QMV, PATH_QMM, PATH_SKINNY, PATH_GATE_UP, PATH_W4A8 = 0, 1, 2, 3, 4, 5
PATH_GROUPED, PATH_PER_PROJECTION = 6, 7
MAX_GROUPED = 4
QMV_POLICY, QMV_AMORTIZED, QMV_PER_ROW, QMV_FAMILIES, QMV_BURST = 0, 1, 2, 3, 4
BITS = (1, 2, 3, 4, 8)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG_DIR), "include", "w4a16.h")
_LIB = None


class W4A16Error(RuntimeError):
    pass


class Plan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "path", "tile_m", "tile_n", "tile_k", "grid_x", "grid_y", "grid_z", "block_threads",
        "split_k", "k_waves", "num_cus", "variant")] + [("workspace_bytes", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


def lib_path() -> str:
    return os.environ.get("W4A16_LIB", os.path.join(_PKG_DIR, "libw4a16.so"))


def load():
    """Load ``libw4a16.so`` (built in-tree) and declare its C signatures; raises if missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise W4A16Error(f"{path} is not built; run `python -m w4a16_group_quantized_qmv_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, u16p, u32p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.w4a16_abi_version.restype = ctypes.c_int
    lib.w4a16_abi_version.argtypes = []
    lib.w4a16_status_string.restype = ctypes.c_char_p
    lib.w4a16_status_string.argtypes = [ctypes.c_int]
    lib.w4a16_plan.restype = ctypes.c_int
    lib.w4a16_plan.argtypes = [i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.w4a16_workspace_bytes.restype = ctypes.c_uint64
    lib.w4a16_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    lib.qmv_w4a16.restype = ctypes.c_int
    lib.qmv_w4a16.argtypes = [u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, vp]
    lib.qmm_w4a16.restype = ctypes.c_int
    lib.qmm_w4a16.argtypes = [u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, i32, vp, ctypes.c_size_t, vp]
    lib.w4a16_linear.restype = ctypes.c_int
    lib.w4a16_linear.argtypes = [u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, vp, ctypes.c_size_t, vp]
    lib.w4a16_linear_noalloc.restype = ctypes.c_int
    lib.w4a16_linear_noalloc.argtypes = [u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, i32, vp]
    lib.w4a16_gate_up_plan.restype = ctypes.c_int
    lib.w4a16_gate_up_plan.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.w4a16_gate_up_swiglu.restype = ctypes.c_int
    lib.w4a16_gate_up_swiglu.argtypes = [u16p, u32p, u16p, u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, i32,
                                         vp, ctypes.c_size_t, vp]
    lib.qmv_affine_plan.restype = ctypes.c_int
    lib.qmv_affine_plan.argtypes = [i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.qmv_affine.restype = ctypes.c_int
    lib.qmv_affine.argtypes = [u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, i32, i32, vp]
    lib.w4a8_xsum_cols.restype = i64
    lib.w4a8_xsum_cols.argtypes = [i64]
    lib.w4a8_quantize_rows.restype = ctypes.c_int
    lib.w4a8_quantize_rows.argtypes = [u16p, vp, vp, u16p, i64, i64, i32, vp]
    lib.w4a8_plan.restype = ctypes.c_int
    lib.w4a8_plan.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.qmm_w4a8.restype = ctypes.c_int
    lib.qmm_w4a8.argtypes = [vp, vp, u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, i32, vp, ctypes.c_size_t, vp]
    lib.w4a8_linear_workspace_bytes.restype = ctypes.c_uint64
    lib.w4a8_linear_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    lib.w4a8_linear.restype = ctypes.c_int
    lib.w4a8_linear.argtypes = [u16p, u32p, u16p, u16p, u16p, i64, i64, i64, i32, vp, ctypes.c_size_t, vp]
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.w4a16_grouped_plan.restype = ctypes.c_int
    lib.w4a16_grouped_plan.argtypes = [i32, ctypes.POINTER(i64), i64, i64, i32, i32, ctypes.POINTER(Plan)]
    lib.w4a16_linear_grouped.restype = ctypes.c_int
    lib.w4a16_linear_grouped.argtypes = [u16p, i32, pp, pp, pp, pp, ctypes.POINTER(i64), i64, i64, i32, vp,
                                         ctypes.c_size_t, vp]
    lib.w4a16_time_next_launch.restype = ctypes.c_int
    lib.w4a16_time_next_launch.argtypes = [vp, vp]
    _LIB = lib
    return lib


def declared_symbols() -> list[str]:
    """Function names declared in include/w4a16.h."""
    with open(_HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


# ------------------------------------------------------------------------------------ status


def w4a16_abi_version() -> int:
    return load().w4a16_abi_version()


def w4a16_status_string(status: int) -> str:
    return load().w4a16_status_string(status).decode()


def _event_handle(event) -> int | None:
    """The hipEvent_t of a torch.cuda.Event (created by its first record()), an int handle, or None."""
    if event is None or isinstance(event, int):
        return event or None
    handle = int(event.cuda_event)
    if handle == 0:
        raise ValueError("the event has no HIP event yet: record() it once before passing it")
    return handle


def w4a16_time_next_launch(start_event=None, stop_event=None):
    """Arm the calling thread's kernel-timestamp request: the next contraction kernel launched
    through the library records its own execution start and end on the two events."""
    _raise_for(load().w4a16_time_next_launch(_event_handle(start_event), _event_handle(stop_event)),
               "w4a16_time_next_launch")


def _raise_for(status: int, what: str):
    if status == W4A16_OK:
        return
    msg = f"{what}: {w4a16_status_string(status)}"
    if status in (1, 2, 3, 4, 5, 9):
        raise ValueError(msg)
    if status == 6:
        raise NotImplementedError(msg)
    raise W4A16Error(msg)


# ------------------------------------------------------------------------------------ planning


def w4a16_plan(M: int, N: int, K: int, group: int = GROUP, path: int = PATH_AUTO, split_k: int = 0,
               num_cus: int = 0) -> dict:
    p = Plan()
    _raise_for(load().w4a16_plan(M, N, K, group, path, split_k, num_cus, ctypes.byref(p)), "w4a16_plan")
    return p.as_dict()


def w4a16_workspace_bytes(M: int, N: int, K: int, group: int = GROUP, num_cus: int = 0) -> int:
    return int(load().w4a16_workspace_bytes(M, N, K, group, num_cus))


def w4a16_gate_up_plan(M: int, N: int, K: int, group: int = GROUP, split_k: int = 0, num_cus: int = 0) -> dict:
    p = Plan()
    _raise_for(load().w4a16_gate_up_plan(M, N, K, group, split_k, num_cus, ctypes.byref(p)), "w4a16_gate_up_plan")
    return p.as_dict()


def qmv_affine_plan(M: int, N: int, K: int, bits: int, mode: int = QMV_POLICY, group: int = GROUP,
                    num_cus: int = 0) -> dict:
    p = Plan()
    _raise_for(load().qmv_affine_plan(M, N, K, group, bits, mode, num_cus, ctypes.byref(p)), "qmv_affine_plan")
    return p.as_dict()


def w4a8_plan(M: int, N: int, K: int, group: int = GROUP, split_k: int = 0, num_cus: int = 0) -> dict:
    p = Plan()
    _raise_for(load().w4a8_plan(M, N, K, group, split_k, num_cus, ctypes.byref(p)), "w4a8_plan")
    return p.as_dict()


def w4a8_xsum_cols(K: int) -> int:
    return int(load().w4a8_xsum_cols(K))


def w4a8_linear_workspace_bytes(M: int, N: int, K: int, group: int = GROUP, num_cus: int = 0) -> int:
    return int(load().w4a8_linear_workspace_bytes(M, N, K, group, num_cus))


# ------------------------------------------------------------------------------------ tensors


def _torch():
    import torch
    return torch


def _check(t, name, dtype, shape):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _operands(x, wq, scales, biases, y, bits: int = 4):
    torch = _torch()
    if x.dim() != 2 or wq.dim() != 2:
        raise ValueError("x and wq must be 2-D")
    M, K = x.shape
    N = wq.shape[0]
    if K % GROUP:
        raise ValueError(f"K={K} must be a multiple of {GROUP}")
    _check(x, "x", torch.bfloat16, (M, K))
    _check(wq, "wq", torch.int32, (N, K * bits // 32))
    _check(scales, "scales", torch.bfloat16, (N, K // GROUP))
    _check(biases, "biases", torch.bfloat16, (N, K // GROUP))
    devs = {t.device for t in (x, wq, scales, biases)}
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, (M, N))
    devs.add(y.device)
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    return M, N, K, y


def _stream_handle(stream) -> int:
    """A HIP stream handle from a ``torch.cuda.Stream`` or an integer handle."""
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _stream(stream, device):
    if stream is not None:
        return ctypes.c_void_p(_stream_handle(stream))
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _keep_for_stream(stream, device, *tensors):
    """Tensors allocated here (on torch's current stream) but used by kernels on the caller's
    ``stream``: record that stream on them, so torch's caching allocator does not hand their
    memory to another allocation before the kernels queued there have finished with it."""
    if stream is None:
        return
    torch = _torch()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream_handle(stream),
                                                                                      device=device)
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _workspace(workspace, nbytes, device):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace, workspace.numel() * workspace.element_size()


def qmv_w4a16(x, wq, scales, biases, y=None, stream=None):
    """Decode-row matvec (1 <= M <= 8); returns y."""
    own_y = y is None
    M, N, K, y = _operands(x, wq, scales, biases, y)
    _keep_for_stream(stream, x.device, y if own_y else None)
    st = load().qmv_w4a16(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(),
                          M, N, K, GROUP, _stream(stream, x.device))
    _raise_for(st, "qmv_w4a16")
    return y


def qmv_affine(x, wq, scales, biases, bits: int, y=None, mode: int = QMV_POLICY, stream=None):
    """Decode-row matvec (1 <= M <= 8) over ``bits``-bit affine codes (1, 2, 3, 4 or 8; ``wq`` int32
    ``[N, K * bits / 32]``, lowest bits first), routed by (bits, M) unless ``mode`` forces the
    row-amortized, the per-row kernel or the burst form.  Returns y."""
    if bits not in BITS:
        raise ValueError(f"bits={bits} must be one of {BITS}")
    own_y = y is None
    M, N, K, y = _operands(x, wq, scales, biases, y, bits)
    _keep_for_stream(stream, x.device, y if own_y else None)
    st = load().qmv_affine(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(),
                           M, N, K, GROUP, bits, mode, _stream(stream, x.device))
    _raise_for(st, "qmv_affine")
    return y


def qmm_w4a16(x, wq, scales, biases, y=None, split_k: int = 0, workspace=None, stream=None):
    """Tiled matrix path for any M; split_k 0 = policy, 1 = off, S > 1 forced.  Returns y."""
    own_y, own_ws = y is None, workspace is None
    M, N, K, y = _operands(x, wq, scales, biases, y)
    need = w4a16_plan(M, N, K, GROUP, PATH_QMM, split_k)["workspace_bytes"]
    ws, ws_bytes = _workspace(workspace, need, x.device)
    _keep_for_stream(stream, x.device, y if own_y else None, ws if own_ws else None)
    st = load().qmm_w4a16(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(),
                          M, N, K, GROUP, split_k, None if ws is None else ws.data_ptr(), ws_bytes,
                          _stream(stream, x.device))
    _raise_for(st, "qmm_w4a16")
    return y


def w4a16_linear(x, wq, scales, biases, y=None, workspace=None, stream=None):
    """Dispatching entry point (qmv for M <= 8, the skinny path for 8 < M <= 32, qmm beyond, each
    with the policy's split).  Returns y."""
    own_y, own_ws = y is None, workspace is None
    M, N, K, y = _operands(x, wq, scales, biases, y)
    ws, ws_bytes = _workspace(workspace, w4a16_workspace_bytes(M, N, K), x.device)
    _keep_for_stream(stream, x.device, y if own_y else None, ws if own_ws else None)
    st = load().w4a16_linear(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(),
                             M, N, K, GROUP, None if ws is None else ws.data_ptr(), ws_bytes,
                             _stream(stream, x.device))
    _raise_for(st, "w4a16_linear")
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20


def w4a16_linear_noalloc(x, wq, scales, biases, y, split_k: int = 0, stream=None):
    """``w4a16_linear`` with its workspace in the library's own device scratch (no allocation in
    the call; ``y`` must be given).  ``split_k`` as for ``qmm_w4a16``.  Calls that overlap on one
    GPU share the scratch and must be ordered by the caller.  Returns y."""
    if y is None:
        raise ValueError("w4a16_linear_noalloc writes into a caller-provided y")
    M, N, K, y = _operands(x, wq, scales, biases, y)
    st = load().w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                     y.data_ptr(), M, N, K, GROUP, split_k, _stream(stream, x.device))
    _raise_for(st, "w4a16_linear_noalloc")
    return y


def w4a16_gate_up_swiglu(x, gate, up, h=None, split_k: int = 0, workspace=None, stream=None):
    """Fused gate / up projections with SwiGLU: ``h = silu(x . Wg^T) * (x . Wu^T)`` in one tile
    kernel.  ``gate`` and ``up`` are ``(wq, scales, biases)`` triples of one shape.  Returns h."""
    (wg, sg, bg), (wu, su, bu) = gate, up
    own_h, own_ws = h is None, workspace is None
    M, N, K, h = _operands(x, wg, sg, bg, h)
    if tuple(wu.shape) != tuple(wg.shape) or tuple(su.shape) != tuple(sg.shape) or tuple(bu.shape) != tuple(bg.shape):
        raise ValueError("gate and up weights must have the same shapes")
    _operands(x, wu, su, bu, h)                      # same dtype / device / contiguity checks for up
    need = w4a16_gate_up_plan(M, N, K, GROUP, split_k)["workspace_bytes"]
    ws, ws_bytes = _workspace(workspace, need, x.device)
    _keep_for_stream(stream, x.device, h if own_h else None, ws if own_ws else None)
    st = load().w4a16_gate_up_swiglu(x.data_ptr(), wg.data_ptr(), sg.data_ptr(), bg.data_ptr(), wu.data_ptr(),
                                     su.data_ptr(), bu.data_ptr(), h.data_ptr(), M, N, K, GROUP, split_k,
                                     None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream, x.device))
    _raise_for(st, "w4a16_gate_up_swiglu")
    return h


def w4a8_quantize_rows(x, xq=None, sx=None, xsum=None, stream=None):
    """Per-row int8 quantization of bf16 ``x [M, K]`` for the W4A8 path; returns ``(xq, sx, xsum)``:
    ``xq`` int8 ``[M, K]`` (each run of 8 values stored as k0 k2 k4 k6 k1 k3 k5 k7), ``sx`` fp32
    ``[M]`` and ``xsum`` bf16 ``[M, w4a8_xsum_cols(K)]`` (exact per-group code sums as hi / lo)."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    KB = w4a8_xsum_cols(K)
    if KB == 0:
        raise ValueError(f"K={K} must be a positive multiple of {GROUP}")
    own = [t is None for t in (xq, sx, xsum)]
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device) if xq is None else xq
    sx = torch.empty((M,), dtype=torch.float32, device=x.device) if sx is None else sx
    xsum = torch.empty((M, KB), dtype=torch.bfloat16, device=x.device) if xsum is None else xsum
    _check(xq, "xq", torch.int8, (M, K))
    _check(sx, "sx", torch.float32, (M,))
    _check(xsum, "xsum", torch.bfloat16, (M, KB))
    _keep_for_stream(stream, x.device, *[t for t, o in zip((xq, sx, xsum), own) if o])
    st = load().w4a8_quantize_rows(x.data_ptr(), xq.data_ptr(), sx.data_ptr(), xsum.data_ptr(), M, K, GROUP,
                                   _stream(stream, x.device))
    _raise_for(st, "w4a8_quantize_rows")
    return xq, sx, xsum


def qmm_w4a8(xq, sx, xsum, wq, scales, biases, y=None, split_k: int = 0, workspace=None, stream=None):
    """int8-activation tile path over the buffers of ``w4a8_quantize_rows``; split_k as for
    ``qmm_w4a16``.  Returns y (bf16 ``[M, N]``)."""
    torch = _torch()
    if xq.dim() != 2 or wq.dim() != 2:
        raise ValueError("xq and wq must be 2-D")
    M, K = xq.shape
    N = wq.shape[0]
    if K % GROUP:
        raise ValueError(f"K={K} must be a multiple of {GROUP}")
    _check(xq, "xq", torch.int8, (M, K))
    _check(sx, "sx", torch.float32, (M,))
    _check(xsum, "xsum", torch.bfloat16, (M, w4a8_xsum_cols(K)))
    _check(wq, "wq", torch.int32, (N, K // 8))
    _check(scales, "scales", torch.bfloat16, (N, K // GROUP))
    _check(biases, "biases", torch.bfloat16, (N, K // GROUP))
    own_y, own_ws = y is None, workspace is None
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check(y, "y", torch.bfloat16, (M, N))
    need = w4a8_plan(M, N, K, GROUP, split_k)["workspace_bytes"]
    ws, ws_bytes = _workspace(workspace, need, xq.device)
    _keep_for_stream(stream, xq.device, y if own_y else None, ws if own_ws else None)
    st = load().qmm_w4a8(xq.data_ptr(), sx.data_ptr(), xsum.data_ptr(), wq.data_ptr(), scales.data_ptr(),
                         biases.data_ptr(), y.data_ptr(), M, N, K, GROUP, split_k,
                         None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream, xq.device))
    _raise_for(st, "qmm_w4a8")
    return y


def w4a8_linear(x, wq, scales, biases, y=None, workspace=None, stream=None):
    """One-call W4A8 projection of bf16 ``x``: per-row int8 quantization into the workspace, then
    the int8 tile path under the policy.  Returns y."""
    own_y, own_ws = y is None, workspace is None
    M, N, K, y = _operands(x, wq, scales, biases, y)
    ws, ws_bytes = _workspace(workspace, w4a8_linear_workspace_bytes(M, N, K), x.device)
    _keep_for_stream(stream, x.device, y if own_y else None, ws if own_ws else None)
    st = load().w4a8_linear(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(),
                            M, N, K, GROUP, None if ws is None else ws.data_ptr(), ws_bytes,
                            _stream(stream, x.device))
    _raise_for(st, "w4a8_linear")
    return y


def linear(x, wq, scales, biases, logits_to_keep: int = 0, path: str | None = None, split_k: int | None = None):
    """Quantized linear layer ``y = x · dequant(Wq)ᵀ`` with the ``logits_to_keep`` row slice.

    ``logits_to_keep = k > 0`` projects only the last ``k`` rows (for generation, the final
    prompt row before the vocabulary head); ``0`` projects every row (prompt scoring).
    ``path`` ("qmv" / "qmm") and ``split_k`` force a path or split for tests and benchmarks.
    """
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M = x.shape[0]
    if logits_to_keep < 0 or logits_to_keep > M:
        raise ValueError(f"logits_to_keep={logits_to_keep} must be in [0, M={M}]")
    if logits_to_keep:
        x = x[M - logits_to_keep:]          # trailing rows of a row-major matrix: still contiguous
    if path is None and split_k is None:
        return w4a16_linear(x, wq, scales, biases)
    if path == "qmv":
        return qmv_w4a16(x, wq, scales, biases)
    if path in (None, "qmm"):
        return qmm_w4a16(x, wq, scales, biases, split_k=split_k or 0)
    raise ValueError(f"unknown path {path!r}")


def w4a16_grouped_plan(N, M: int, K: int, group: int = GROUP, num_cus: int = 0) -> dict:
    """Plan of ``w4a16_linear_grouped`` for projections of ``N[p]`` columns (one list entry each)."""
    arr = (ctypes.c_int64 * len(N))(*N)
    plan = Plan()
    st = load().w4a16_grouped_plan(len(N), arr, M, K, group, num_cus, ctypes.byref(plan))
    _raise_for(st, "w4a16_grouped_plan")
    return plan.as_dict()


def _grouped_args(x, weights, ys):
    if not 1 <= len(weights) <= MAX_GROUPED:
        raise ValueError(f"{len(weights)} projections: 1 .. {MAX_GROUPED} are supported")
    if ys is None:
        ys = [None] * len(weights)
    if len(ys) != len(weights):
        raise ValueError("one output per projection")
    out, Ns = [], []
    for (wq, s, b), y in zip(weights, ys):
        M, N, K, y = _operands(x, wq, s, b, y)
        out.append(y)
        Ns.append(N)
    vp = ctypes.c_void_p
    arrays = tuple((vp * len(weights))(*[t.data_ptr() for t in col])
                   for col in ([w[0] for w in weights], [w[1] for w in weights], [w[2] for w in weights], out))
    return M, K, out, Ns, arrays


def w4a16_linear_grouped(x, weights, ys=None, workspace=None, stream=None):
    """Projections of one input in one call: ``weights`` is a list of ``(wq, scales, biases)``
    triples (1 .. MAX_GROUPED), e.g. the query, key and value projections; returns the list of
    outputs ``y_p = x . dequant(wq_p)^T``."""
    own_y, own_ws = ys is None, workspace is None
    M, K, out, Ns, (wqa, sa, ba, ya) = _grouped_args(x, weights, ys)
    need = w4a16_grouped_plan(Ns, M, K)["workspace_bytes"]
    ws, ws_bytes = _workspace(workspace, need, x.device)
    _keep_for_stream(stream, x.device, *(out if own_y else []), ws if own_ws else None)
    st = load().w4a16_linear_grouped(x.data_ptr(), len(weights), wqa, sa, ba, ya, (ctypes.c_int64 * len(Ns))(*Ns),
                                     M, K, GROUP, None if ws is None else ws.data_ptr(), ws_bytes,
                                     _stream(stream, x.device))
    _raise_for(st, "w4a16_linear_grouped")
    return out


class PreparedLinear:
    """One projection with fixed tensors, validated once; calling it only enqueues the kernels.

    For timing loops and graph capture: the output ``y`` and any workspace are allocated here
    (or passed in: ``y`` and ``workspace`` may be shared by calls that do not overlap), and
    ``__call__`` issues a single C-ABI call (``w4a16_linear``, or
    ``qmv_w4a16`` / ``qmm_w4a16`` when ``path`` forces one) on the stream current at
    construction.
    """

    def __init__(self, x, wq, scales, biases, y=None, path: str | None = None, split_k: int = 0, workspace=None):
        M, N, K, y = _operands(x, wq, scales, biases, y)
        self.M, self.N, self.K, self.y = M, N, K, y
        lib = load()
        stream = _stream(None, x.device)
        ptrs = (x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(), M, N, K, GROUP)
        if path == "qmv":
            self.plan = w4a16_plan(M, N, K, GROUP, PATH_QMV, 1)
            self._fn, self._args, self._name = lib.qmv_w4a16, ptrs + (stream,), "qmv_w4a16"
            self.workspace = None
        else:
            forced = path == "qmm" or split_k != 0
            self.plan = w4a16_plan(M, N, K, GROUP, PATH_QMM if forced else PATH_AUTO, split_k)
            ws, ws_bytes = _workspace(workspace, self.plan["workspace_bytes"], x.device)
            self.workspace = ws
            wsp = None if ws is None else ws.data_ptr()
            if forced:
                self._fn, self._name = lib.qmm_w4a16, "qmm_w4a16"
                self._args = ptrs + (split_k, wsp, ws_bytes, stream)
            else:
                self._fn, self._name = lib.w4a16_linear, "w4a16_linear"
                self._args = ptrs + (wsp, ws_bytes, stream)

    def __call__(self):
        st = self._fn(*self._args)
        if st != W4A16_OK:
            _raise_for(st, self._name)
        return self.y


class PreparedGateUp:
    """The fused gate / up + SwiGLU call with fixed tensors, validated once (see PreparedLinear):
    ``h`` and any split-K workspace are allocated here; ``__call__`` issues one C-ABI call
    (``w4a16_gate_up_swiglu``) on the stream current at construction."""

    def __init__(self, x, gate, up, h=None, split_k: int = 0, workspace=None):
        (wg, sg, bg), (wu, su, bu) = gate, up
        M, N, K, h = _operands(x, wg, sg, bg, h)
        if tuple(wu.shape) != tuple(wg.shape):
            raise ValueError("gate and up weights must have the same shapes")
        _operands(x, wu, su, bu, h)
        self.M, self.N, self.K, self.h = M, N, K, h
        lib = load()
        self.plan = w4a16_gate_up_plan(M, N, K, GROUP, split_k)
        ws, ws_bytes = _workspace(workspace, self.plan["workspace_bytes"], x.device)
        self.workspace = ws
        self._fn = lib.w4a16_gate_up_swiglu
        self._args = (x.data_ptr(), wg.data_ptr(), sg.data_ptr(), bg.data_ptr(), wu.data_ptr(), su.data_ptr(),
                      bu.data_ptr(), h.data_ptr(), M, N, K, GROUP, split_k, None if ws is None else ws.data_ptr(),
                      ws_bytes, _stream(None, x.device))

    def __call__(self):
        st = self._fn(*self._args)
        if st != W4A16_OK:
            _raise_for(st, "w4a16_gate_up_swiglu")
        return self.h


class PreparedGrouped:
    """Grouped projections of one input with fixed tensors, validated once (see PreparedLinear):
    the outputs and any workspace are allocated here (or passed in); ``__call__`` issues one
    C-ABI call (``w4a16_linear_grouped``) on the stream current at construction."""

    def __init__(self, x, weights, ys=None, workspace=None):
        M, K, out, Ns, arrays = _grouped_args(x, weights, ys)
        self.M, self.K, self.N, self.ys = M, K, Ns, out
        self.plan = w4a16_grouped_plan(Ns, M, K)
        ws, ws_bytes = _workspace(workspace, self.plan["workspace_bytes"], x.device)
        self.workspace = ws
        self._keep = (arrays, (ctypes.c_int64 * len(Ns))(*Ns))
        self._fn = load().w4a16_linear_grouped
        self._args = (x.data_ptr(), len(weights), *arrays, self._keep[1], M, K, GROUP,
                      None if ws is None else ws.data_ptr(), ws_bytes, _stream(None, x.device))

    def __call__(self):
        st = self._fn(*self._args)
        if st != W4A16_OK:
            _raise_for(st, "w4a16_linear_grouped")
        return self.ys


class PreparedW4A8:
    """The one-call W4A8 projection with fixed tensors, validated once (see PreparedLinear): ``y``
    and the workspace (activation buffers plus partials) are allocated here; ``__call__`` issues
    one C-ABI call (``w4a8_linear``) on the stream current at construction."""

    def __init__(self, x, wq, scales, biases, y=None, workspace=None):
        M, N, K, y = _operands(x, wq, scales, biases, y)
        self.M, self.N, self.K, self.y = M, N, K, y
        lib = load()
        self.plan = w4a8_plan(M, N, K, GROUP, 0)
        ws, ws_bytes = _workspace(workspace, w4a8_linear_workspace_bytes(M, N, K), x.device)
        self.workspace = ws
        self._fn = lib.w4a8_linear
        self._args = (x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), y.data_ptr(), M, N, K,
                      GROUP, ws.data_ptr(), ws_bytes, _stream(None, x.device))

    def __call__(self):
        st = self._fn(*self._args)
        if st != W4A16_OK:
            _raise_for(st, "w4a8_linear")
        return self.y
