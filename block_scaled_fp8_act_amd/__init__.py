"""Python binding of libfp8blk: block-scaled ("fine-grained") FP8 linear
layers on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libfp8blk.so; torch provides device memory and the current
stream.  There is no fallback: if the library is missing or the device is
not a gfx950, calls raise.

Low-level entry points carry the C names and take torch tensors for every
buffer (inputs and preallocated outputs):

    fp8_weight_block_quant(w, w_q, w_scale)
    fp8_act_quant_group(x, x_q, x_scale)
    fp8_block_gemm(x_q, x_scale, w_q, w_scale, y)
    fp8_grouped_block_gemm(x_q, x_scale, w_q, w_scale, offsets, y)

their power-of-two-scale twins (scales as E8M0 bytes, uint8 or
torch.float8_e8m0fnu tensors): fp8_weight_block_quant_ue8m0,
fp8_act_quant_group_ue8m0, fp8_block_gemm_ue8m0, fp8_grouped_block_gemm_ue8m0,
and the static-activation-scale pair (one fp32 scale in a 1-element device
tensor): fp8_act_quant_static(x, x_scale, x_q),
fp8_block_gemm_static(x_q, x_scale, w_q, w_scale, y); the batched expert
layout fp8_batched_block_gemm(x_q, x_scale, w_q, w_scale, counts, y) with
x_q [E, C, K]; row-wise scales fp8_rowwise_quant(x, q, scale),
fp8_rowwise_gemm(x_q, x_scale, w_q, w_scale, y); and SwiGLU ahead of the
activation quantizer fp8_swiglu_act_quant(gate_up, x_q, x_scale) (the
input of a mixture-of-experts down projection, gate_up [M, 2I] with the
gate first).

Convenience wrappers allocate the outputs; ``scale_fmt`` is "float" (fp32
scales) or "ue8m0" (E8M0 bytes), and the GEMMs pick the path from the scale
tensors' dtype:

    weight_block_quant(w, scale_fmt) -> (w_q uint8 [N,K], w_scale [ceil(N/128), K/128])
    act_quant_group(x, scale_fmt)    -> (x_q uint8 [M,K], x_scale [M, K/128])
    block_gemm(x_q, x_scale, w_q, w_scale) -> y bf16 [M,N]
    grouped_block_gemm(x_q, x_scale, w_q, w_scale, offsets) -> y bf16 [sum M_e, N]
    linear(x, w_q, w_scale) -> y bf16 [M,N]   (dynamic act quant, then GEMM)
    act_quant_static(x, x_scale) -> x_q uint8 [M,K]
    block_gemm_static(x_q, x_scale, w_q, w_scale) -> y bf16 [M,N]
    linear_static(x, x_scale, w_q, w_scale) -> y bf16 [M,N]
    batched_block_gemm(x_q, x_scale, w_q, w_scale, counts) -> y bf16 [E,C,N]
    rowwise_quant(x) -> (q uint8 [R,K], scale fp32 [R])
    rowwise_gemm(x_q, x_scale, w_q, w_scale) -> y bf16 [M,N]
    linear_rowwise(x, w_q, w_scale) -> y bf16 [M,N]
    swiglu_act_quant(gate_up, scale_fmt) -> (x_q uint8 [M,I], x_scale [M, I/128])
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Fp8BlkError", "BLOCK", "lib_path", "load_library", "status_string",
    "fp8_weight_block_quant", "fp8_act_quant_group", "fp8_block_gemm",
    "fp8_grouped_block_gemm", "fp8_block_gemm_ws", "fp8_block_gemm_workspace_bytes",
    "fp8_block_gemm_ue8m0_ws", "fp8_block_gemm_noalloc", "SCRATCH_BYTES",
    "fp8_weight_block_quant_ue8m0", "fp8_act_quant_group_ue8m0",
    "fp8_block_gemm_ue8m0", "fp8_grouped_block_gemm_ue8m0", "fp8_act_quant_static",
    "fp8_block_gemm_static", "act_quant_static", "block_gemm_static", "linear_static",
    "fp8_linear", "fp8_batched_block_gemm", "batched_block_gemm", "fp8_rowwise_quant", "fp8_rowwise_gemm",
    "rowwise_quant", "rowwise_gemm", "linear_rowwise", "fp8_swiglu_act_quant",
    "fp8_swiglu_act_quant_ue8m0", "swiglu_act_quant",
    "weight_block_quant",
    "act_quant_group", "block_gemm", "grouped_block_gemm", "linear", "SCALE_FMTS",
]

BLOCK = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libfp8blk.so")
_lib = None

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_LAUNCH, ERR_SCRATCH = range(7)
SCRATCH_BYTES = 16 * 1024 * 1024 + 64 * 1024     # FP8BLK_SCRATCH_BYTES


class Fp8BlkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Fp8BlkValueError(Fp8BlkError, ValueError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libfp8blk.so (built in-tree by block_scaled_fp8_act_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libfp8blk.so not found at {_LIB_PATH}; build it with "
            "`python -m block_scaled_fp8_act_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sigs = {
        "fp8_weight_block_quant": [vp, i64, i64, vp, vp, vp],
        "fp8_act_quant_group": [vp, i64, i64, vp, vp, vp],
        "fp8_block_gemm": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8_block_gemm_ws": [vp, vp, vp, vp, i64, i64, i64, vp, vp, ctypes.c_size_t, vp],
        "fp8_block_gemm_noalloc": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8_grouped_block_gemm": [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, vp],
        "fp8_linear": [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp],
        "fp8_batched_block_gemm": [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, vp],
        "fp8_rowwise_quant": [vp, i64, i64, vp, vp, vp],
        "fp8_swiglu_act_quant": [vp, i64, i64, vp, vp, vp],
        "fp8_swiglu_act_quant_ue8m0": [vp, i64, i64, vp, vp, vp],
        "fp8_rowwise_gemm": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8_act_quant_static": [vp, i64, i64, vp, vp, vp],
        "fp8_block_gemm_static": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8_weight_block_quant_ue8m0": [vp, i64, i64, vp, vp, vp],
        "fp8_act_quant_group_ue8m0": [vp, i64, i64, vp, vp, vp],
        "fp8_block_gemm_ue8m0": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8_block_gemm_ue8m0_ws": [vp, vp, vp, vp, i64, i64, i64, vp, vp, ctypes.c_size_t, vp],
        "fp8_grouped_block_gemm_ue8m0": [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    for name in ("fp8_block_gemm_workspace_bytes", "fp8_block_gemm_ue8m0_workspace_bytes"):
        getattr(lib, name).argtypes = [i64, i64, i64]
        getattr(lib, name).restype = ctypes.c_size_t
    lib.fp8blk_status_string.argtypes = [ctypes.c_int]
    lib.fp8blk_status_string.restype = ctypes.c_char_p
    lib.fp8blk_abi_version.argtypes = []
    lib.fp8blk_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fp8blk_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status == OK:
        return
    msg = f"{what}: {status_string(status)}"
    if status in (ERR_SHAPE, ERR_DEVICE):
        raise Fp8BlkValueError(status, msg)
    raise Fp8BlkError(status, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


_CODES = (torch.uint8, torch.float8_e4m3fn)


def _shape_eq(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# --------------------------------------------------------------------------
# low-level entry points (same names as the C ABI)

_F32 = (torch.float32,)
_E8M0 = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
SCALE_FMTS = ("float", "ue8m0")


def _weight_quant(cname, sdt, w, w_q, w_scale):
    _need(w, "w", (torch.bfloat16,), 2)
    N, K = w.shape
    _need(w_q, "w_q", _CODES); _need(w_scale, "w_scale", sdt)
    _shape_eq(w_q, (N, K), "w_q")
    if K % BLOCK == 0:
        _shape_eq(w_scale, (-(-N // BLOCK), K // BLOCK), "w_scale")
    _check(getattr(load_library(), cname)(_ptr(w), N, K, _ptr(w_q), _ptr(w_scale), _stream()),
           cname)


def _act_quant(cname, sdt, x, x_q, x_scale):
    _need(x, "x", (torch.bfloat16,), 2)
    M, K = x.shape
    _need(x_q, "x_q", _CODES); _need(x_scale, "x_scale", sdt)
    _shape_eq(x_q, (M, K), "x_q")
    if K % BLOCK == 0:
        _shape_eq(x_scale, (M, K // BLOCK), "x_scale")
    _check(getattr(load_library(), cname)(_ptr(x), M, K, _ptr(x_q), _ptr(x_scale), _stream()),
           cname)


def _gemm(cname, sdt, x_q, x_scale, w_q, w_scale, y):
    _need(x_q, "x_q", _CODES, 2); _need(w_q, "w_q", _CODES, 2)
    _need(x_scale, "x_scale", sdt, 2); _need(w_scale, "w_scale", sdt, 2)
    _need(y, "y", (torch.bfloat16,), 2)
    M, K = x_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("x_q and w_q disagree on K")
    if K % BLOCK == 0:
        _shape_eq(x_scale, (M, K // BLOCK), "x_scale")
        _shape_eq(w_scale, (-(-N // BLOCK), K // BLOCK), "w_scale")
    _shape_eq(y, (M, N), "y")
    _check(getattr(load_library(), cname)(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale),
                                          M, N, K, _ptr(y), _stream()), cname)


def _grouped(cname, sdt, x_q, x_scale, w_q, w_scale, offsets, y):
    _need(x_q, "x_q", _CODES, 2); _need(w_q, "w_q", _CODES, 3)
    _need(x_scale, "x_scale", sdt, 2); _need(w_scale, "w_scale", sdt, 3)
    _need(offsets, "offsets", (torch.int32,), 1); _need(y, "y", (torch.bfloat16,), 2)
    total, K = x_q.shape
    E, N, K2 = w_q.shape
    if K2 != K:
        raise ValueError("x_q and w_q disagree on K")
    if offsets.numel() != E + 1:
        raise ValueError("offsets must have E+1 entries")
    if K % BLOCK == 0:
        _shape_eq(x_scale, (total, K // BLOCK), "x_scale")
        _shape_eq(w_scale, (E, -(-N // BLOCK), K // BLOCK), "w_scale")
    _shape_eq(y, (total, N), "y")
    _check(getattr(load_library(), cname)(
        _ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale), _ptr(offsets), E, total, N, K,
        _ptr(y), _stream()), cname)


def fp8_weight_block_quant(w, w_q, w_scale):
    _weight_quant("fp8_weight_block_quant", _F32, w, w_q, w_scale)


def fp8_act_quant_group(x, x_q, x_scale):
    _act_quant("fp8_act_quant_group", _F32, x, x_q, x_scale)


def fp8_block_gemm(x_q, x_scale, w_q, w_scale, y):
    _gemm("fp8_block_gemm", _F32, x_q, x_scale, w_q, w_scale, y)


def fp8_block_gemm_noalloc(x_q, x_scale, w_q, w_scale, y):
    """fp8_block_gemm_ws with the library's own device scratch: no
    workspace, no allocation (callers that cannot allocate)."""
    _gemm("fp8_block_gemm_noalloc", _F32, x_q, x_scale, w_q, w_scale, y)


def fp8_block_gemm_workspace_bytes(M, N, K, scale_fmt="float"):
    """Workspace bytes fp8_block_gemm_ws (scale_fmt "ue8m0":
    fp8_block_gemm_ue8m0_ws) splits K with for these sizes (0: no split; the
    call is then the plain GEMM)."""
    name = ("fp8_block_gemm_ue8m0_workspace_bytes" if scale_fmt == "ue8m0"
            else "fp8_block_gemm_workspace_bytes")
    return int(getattr(load_library(), name)(int(M), int(N), int(K)))


def fp8_block_gemm_ws(x_q, x_scale, w_q, w_scale, y, workspace=None):
    """fp8_block_gemm with K split over workgroups through ``workspace`` (a
    device tensor of at least fp8_block_gemm_workspace_bytes bytes) for
    grids that would leave most CUs idle; without a large enough workspace
    it is fp8_block_gemm."""
    _gemm_ws("fp8_block_gemm_ws", _F32, x_q, x_scale, w_q, w_scale, y, workspace)


def fp8_block_gemm_ue8m0_ws(x_q, x_scale, w_q, w_scale, y, workspace=None):
    """fp8_block_gemm_ue8m0 with K split over workgroups (as fp8_block_gemm_ws)."""
    _gemm_ws("fp8_block_gemm_ue8m0_ws", _E8M0, x_q, x_scale, w_q, w_scale, y, workspace)


def _gemm_ws(cname, sdt, x_q, x_scale, w_q, w_scale, y, workspace):
    _need(x_q, "x_q", _CODES, 2); _need(w_q, "w_q", _CODES, 2)
    _need(x_scale, "x_scale", sdt, 2); _need(w_scale, "w_scale", sdt, 2)
    _need(y, "y", (torch.bfloat16,), 2)
    M, K = x_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("x_q and w_q disagree on K")
    if K % BLOCK == 0:
        _shape_eq(x_scale, (M, K // BLOCK), "x_scale")
        _shape_eq(w_scale, (-(-N // BLOCK), K // BLOCK), "w_scale")
    _shape_eq(y, (M, N), "y")
    wbytes = 0
    if workspace is not None:
        _need(workspace, "workspace", (workspace.dtype,))
        wbytes = workspace.numel() * workspace.element_size()
    _check(getattr(load_library(), cname)(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale),
                                          M, N, K, _ptr(y), _ptr(workspace), wbytes, _stream()),
           cname)


def fp8_grouped_block_gemm(x_q, x_scale, w_q, w_scale, offsets, y):
    _grouped("fp8_grouped_block_gemm", _F32, x_q, x_scale, w_q, w_scale, offsets, y)


def _static_scale(x_scale):
    _need(x_scale, "x_scale", _F32)
    if x_scale.numel() != 1:
        raise ValueError("the static activation scale is one fp32 value")


def fp8_act_quant_static(x, x_scale, x_q):
    _need(x, "x", (torch.bfloat16,), 2)
    M, K = x.shape
    _static_scale(x_scale)
    _need(x_q, "x_q", _CODES)
    _shape_eq(x_q, (M, K), "x_q")
    _check(load_library().fp8_act_quant_static(_ptr(x), M, K, _ptr(x_scale), _ptr(x_q), _stream()),
           "fp8_act_quant_static")


def fp8_block_gemm_static(x_q, x_scale, w_q, w_scale, y):
    _need(x_q, "x_q", _CODES, 2); _need(w_q, "w_q", _CODES, 2)
    _static_scale(x_scale); _need(w_scale, "w_scale", _F32, 2)
    _need(y, "y", (torch.bfloat16,), 2)
    M, K = x_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("x_q and w_q disagree on K")
    if K % BLOCK == 0:
        _shape_eq(w_scale, (-(-N // BLOCK), K // BLOCK), "w_scale")
    _shape_eq(y, (M, N), "y")
    _check(load_library().fp8_block_gemm_static(_ptr(x_q), _ptr(x_scale), _ptr(w_q),
                                                _ptr(w_scale), M, N, K, _ptr(y), _stream()),
           "fp8_block_gemm_static")


FUSED_MAX_M = 64


def fp8_linear(x, w_q, w_scale, y, x_q_ws=None, x_scale_ws=None):
    """One C call for the linear layer: fused in one kernel for M <= 64 when
    no workspaces are given, and with workspaces where that is faster (M <= 16
    with N * K <= 2^25 or with several 16-column slabs per workgroup at
    K <= 8192; 16 < M <= 32 with N * K <= 2^24); else quantization into the
    workspaces (required for M > 64) and the GEMM."""
    _need(x, "x", (torch.bfloat16,), 2); _need(w_q, "w_q", _CODES, 2)
    _need(w_scale, "w_scale", _F32, 2); _need(y, "y", (torch.bfloat16,), 2)
    M, K = x.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("x and w_q disagree on K")
    if K % BLOCK == 0:
        _shape_eq(w_scale, (-(-N // BLOCK), K // BLOCK), "w_scale")
    _shape_eq(y, (M, N), "y")
    if M > FUSED_MAX_M:
        if x_q_ws is None or x_scale_ws is None:
            raise ValueError("M > 64 needs the x_q_ws / x_scale_ws workspaces")
        _need(x_q_ws, "x_q_ws", _CODES); _need(x_scale_ws, "x_scale_ws", _F32)
        _shape_eq(x_q_ws, (M, K), "x_q_ws")
        if K % BLOCK == 0:
            _shape_eq(x_scale_ws, (M, K // BLOCK), "x_scale_ws")
    _check(load_library().fp8_linear(_ptr(x), M, N, K, _ptr(w_q), _ptr(w_scale), _ptr(x_q_ws),
                                     _ptr(x_scale_ws), _ptr(y), _stream()), "fp8_linear")


def fp8_batched_block_gemm(x_q, x_scale, w_q, w_scale, counts, y):
    _need(x_q, "x_q", _CODES, 3); _need(w_q, "w_q", _CODES, 3)
    _need(x_scale, "x_scale", _F32, 3); _need(w_scale, "w_scale", _F32, 3)
    _need(counts, "counts", (torch.int32,), 1); _need(y, "y", (torch.bfloat16,), 3)
    E, C, K = x_q.shape
    E2, N, K2 = w_q.shape
    if E2 != E or K2 != K:
        raise ValueError("x_q [E,C,K] and w_q [E,N,K] disagree")
    if counts.numel() != E:
        raise ValueError("counts must have E entries")
    if K % BLOCK == 0:
        _shape_eq(x_scale, (E, C, K // BLOCK), "x_scale")
        _shape_eq(w_scale, (E, -(-N // BLOCK), K // BLOCK), "w_scale")
    _shape_eq(y, (E, C, N), "y")
    _check(load_library().fp8_batched_block_gemm(
        _ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale), _ptr(counts), E, C, N, K, _ptr(y),
        _stream()), "fp8_batched_block_gemm")


def fp8_rowwise_quant(x, q, scale):
    _need(x, "x", (torch.bfloat16,), 2)
    R, K = x.shape
    _need(q, "q", _CODES); _need(scale, "scale", _F32)
    _shape_eq(q, (R, K), "q")
    _shape_eq(scale, (R,), "scale")
    _check(load_library().fp8_rowwise_quant(_ptr(x), R, K, _ptr(q), _ptr(scale), _stream()),
           "fp8_rowwise_quant")


def _swiglu(cname, sdt, gate_up, x_q, x_scale):
    _need(gate_up, "gate_up", (torch.bfloat16,), 2)
    M, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up must hold 2I columns")
    I = two_i // 2
    _need(x_q, "x_q", _CODES); _need(x_scale, "x_scale", sdt)
    _shape_eq(x_q, (M, I), "x_q")
    if I % BLOCK == 0:
        _shape_eq(x_scale, (M, I // BLOCK), "x_scale")
    _check(getattr(load_library(), cname)(_ptr(gate_up), M, I, _ptr(x_q), _ptr(x_scale),
                                          _stream()), cname)


def fp8_swiglu_act_quant(gate_up, x_q, x_scale):
    """gate_up bf16 [M, 2I] (gate in columns [0, I), up in [I, 2I)) ->
    codes of h = bf16(SiLU(gate) * up) in x_q [M, I] and fp32 group scales
    in x_scale [M, I/128]."""
    _swiglu("fp8_swiglu_act_quant", _F32, gate_up, x_q, x_scale)


def fp8_swiglu_act_quant_ue8m0(gate_up, x_q, x_scale):
    """As fp8_swiglu_act_quant with E8M0 scale bytes (uint8 or float8_e8m0fnu)."""
    _swiglu("fp8_swiglu_act_quant_ue8m0", _E8M0, gate_up, x_q, x_scale)


def fp8_rowwise_gemm(x_q, x_scale, w_q, w_scale, y):
    _need(x_q, "x_q", _CODES, 2); _need(w_q, "w_q", _CODES, 2)
    _need(x_scale, "x_scale", _F32, 1); _need(w_scale, "w_scale", _F32, 1)
    _need(y, "y", (torch.bfloat16,), 2)
    M, K = x_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("x_q and w_q disagree on K")
    _shape_eq(x_scale, (M,), "x_scale"); _shape_eq(w_scale, (N,), "w_scale")
    _shape_eq(y, (M, N), "y")
    _check(load_library().fp8_rowwise_gemm(_ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale),
                                           M, N, K, _ptr(y), _stream()), "fp8_rowwise_gemm")


def fp8_weight_block_quant_ue8m0(w, w_q, w_scale):
    _weight_quant("fp8_weight_block_quant_ue8m0", _E8M0, w, w_q, w_scale)


def fp8_act_quant_group_ue8m0(x, x_q, x_scale):
    _act_quant("fp8_act_quant_group_ue8m0", _E8M0, x, x_q, x_scale)


def fp8_block_gemm_ue8m0(x_q, x_scale, w_q, w_scale, y):
    _gemm("fp8_block_gemm_ue8m0", _E8M0, x_q, x_scale, w_q, w_scale, y)


def fp8_grouped_block_gemm_ue8m0(x_q, x_scale, w_q, w_scale, offsets, y):
    _grouped("fp8_grouped_block_gemm_ue8m0", _E8M0, x_q, x_scale, w_q, w_scale, offsets, y)


# --------------------------------------------------------------------------
# convenience wrappers (allocate outputs with torch.empty)

def _scale_dtype(scale_fmt):
    if scale_fmt not in SCALE_FMTS:
        raise ValueError(f"scale_fmt must be one of {SCALE_FMTS}, got {scale_fmt!r}")
    return torch.float32 if scale_fmt == "float" else torch.uint8


def _is_e8m0(t):
    return t.dtype in _E8M0


def weight_block_quant(w, scale_fmt="float"):
    N, K = w.shape
    w_q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    w_s = torch.empty((-(-N // BLOCK), max(K // BLOCK, 0)), dtype=_scale_dtype(scale_fmt),
                      device=w.device)
    (fp8_weight_block_quant if scale_fmt == "float" else fp8_weight_block_quant_ue8m0)(w, w_q, w_s)
    return w_q, w_s


def act_quant_group(x, scale_fmt="float"):
    M, K = x.shape
    x_q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    x_s = torch.empty((M, max(K // BLOCK, 0)), dtype=_scale_dtype(scale_fmt), device=x.device)
    (fp8_act_quant_group if scale_fmt == "float" else fp8_act_quant_group_ue8m0)(x, x_q, x_s)
    return x_q, x_s


def block_gemm(x_q, x_scale, w_q, w_scale):
    """y = x * W^T in bf16.  fp32 scales: with K split over workgroups (and a
    workspace from torch's allocator) when the library asks for one."""
    M, N, K = x_q.shape[0], w_q.shape[0], x_q.shape[1]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x_q.device)
    e8m0 = _is_e8m0(w_scale)
    need = fp8_block_gemm_workspace_bytes(M, N, K, "ue8m0" if e8m0 else "float")
    if need:
        work = torch.empty(need, dtype=torch.uint8, device=x_q.device)
        (fp8_block_gemm_ue8m0_ws if e8m0 else fp8_block_gemm_ws)(x_q, x_scale, w_q, w_scale, y, work)
    else:
        (fp8_block_gemm_ue8m0 if e8m0 else fp8_block_gemm)(x_q, x_scale, w_q, w_scale, y)
    return y


def grouped_block_gemm(x_q, x_scale, w_q, w_scale, offsets):
    y = torch.empty((x_q.shape[0], w_q.shape[1]), dtype=torch.bfloat16, device=x_q.device)
    fn = fp8_grouped_block_gemm_ue8m0 if _is_e8m0(w_scale) else fp8_grouped_block_gemm
    fn(x_q, x_scale, w_q, w_scale, offsets, y)
    return y


def linear(x, w_q, w_scale):
    """The FP8 linear layer: dynamic per-token-group quantization of x, then
    the block-scaled GEMM on the current stream (fp32 scales: one C call,
    fused into one kernel where the library finds that faster, M <= 32; the
    quantizer then the GEMM with a workspace when the library asks for one:
    output grids too small to fill the chip (K split over workgroups, or
    stream-K with long K), a partly empty last round of tiles, and 9 <= M <=
    16 or 33 <= M <= 64 with long K, where re-reading x per column slab costs
    more than the separate quantizer and the split).  E8M0 weight scales
    select power-of-two activation scales as well."""
    if _is_e8m0(w_scale):
        x_q, x_s = act_quant_group(x, "ue8m0")
        return block_gemm(x_q, x_s, w_q, w_scale)
    M, K = x.shape
    if fp8_block_gemm_workspace_bytes(M, w_q.shape[0], K):
        x_q, x_s = act_quant_group(x)
        return block_gemm(x_q, x_s, w_q, w_scale)
    y = torch.empty((M, w_q.shape[0]), dtype=torch.bfloat16, device=x.device)
    x_q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    x_s = torch.empty((M, max(K // BLOCK, 0)), dtype=torch.float32, device=x.device)
    fp8_linear(x, w_q, w_scale, y, x_q, x_s)   # the library picks fused or two kernels
    return y


def act_quant_static(x, x_scale):
    x_q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    fp8_act_quant_static(x, x_scale, x_q)
    return x_q


def block_gemm_static(x_q, x_scale, w_q, w_scale):
    y = torch.empty((x_q.shape[0], w_q.shape[0]), dtype=torch.bfloat16, device=x_q.device)
    fp8_block_gemm_static(x_q, x_scale, w_q, w_scale, y)
    return y


def linear_static(x, x_scale, w_q, w_scale):
    """The FP8 linear layer with a static (calibrated, per-tensor) activation
    scale: quantization of x, then the block-scaled GEMM."""
    return block_gemm_static(act_quant_static(x, x_scale), x_scale, w_q, w_scale)


def batched_block_gemm(x_q, x_scale, w_q, w_scale, counts):
    """Rows past an expert's count are left as torch.empty returned them."""
    y = torch.empty((x_q.shape[0], x_q.shape[1], w_q.shape[1]), dtype=torch.bfloat16,
                    device=x_q.device)
    fp8_batched_block_gemm(x_q, x_scale, w_q, w_scale, counts, y)
    return y


def rowwise_quant(x):
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty((x.shape[0],), dtype=torch.float32, device=x.device)
    fp8_rowwise_quant(x, q, s)
    return q, s


def swiglu_act_quant(gate_up, scale_fmt="float"):
    M, I = gate_up.shape[0], gate_up.shape[1] // 2
    q = torch.empty((M, I), dtype=torch.uint8, device=gate_up.device)
    s = torch.empty((M, I // BLOCK), dtype=_scale_dtype(scale_fmt), device=gate_up.device)
    (fp8_swiglu_act_quant if scale_fmt == "float" else fp8_swiglu_act_quant_ue8m0)(gate_up, q, s)
    return q, s


def rowwise_gemm(x_q, x_scale, w_q, w_scale):
    y = torch.empty((x_q.shape[0], w_q.shape[0]), dtype=torch.bfloat16, device=x_q.device)
    fp8_rowwise_gemm(x_q, x_scale, w_q, w_scale, y)
    return y


def linear_rowwise(x, w_q, w_scale):
    """Row-wise ("fp8r") linear layer: per-token quantization of x, then the
    row-scaled GEMM."""
    x_q, x_s = rowwise_quant(x)
    return rowwise_gemm(x_q, x_s, w_q, w_scale)
