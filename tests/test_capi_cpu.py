"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments with the documented status codes
before touching the HIP runtime.  No compute call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")


@pytest.fixture(scope="module")
def lib():
    from block_scaled_fp8_act_amd import build
    import block_scaled_fp8_act_amd as fb
    if not os.path.exists(fb.lib_path()):
        build.build()
    return fb.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*FP8BLK_API\s+(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("fp8_weight_block_quant", "fp8_act_quant_group", "fp8_block_gemm",
              "fp8_grouped_block_gemm", "fp8blk_status_string", "fp8blk_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_internal_symbols_hidden(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions()), exported


def test_status_strings(lib):
    import block_scaled_fp8_act_amd as fb
    for code in range(7):
        assert fb.status_string(code).startswith("FP8BLK_")
    assert fb.status_string(99) == "FP8BLK_ERR_UNKNOWN"
    assert lib.fp8blk_abi_version() == 1


A = 0x10000          # fake, 16-byte aligned addresses: never dereferenced
B = 0x20000
C = 0x30000
D = 0x40000
E_ = 0x50000
MIS = 0x10008        # 8-byte aligned only
NULL = None


def call(lib, name, *args):
    return getattr(lib, name)(*args)


@pytest.mark.parametrize("args,want", [
    ((NULL, 4, 128, B, C, NULL), 1),            # null input
    ((A, 4, 128, NULL, C, NULL), 1),            # null codes
    ((A, 4, 128, B, NULL, NULL), 1),            # null scales
    ((A, -1, 128, B, C, NULL), 2),              # negative rows
    ((A, 4, 0, B, C, NULL), 2),                 # K = 0
    ((A, 4, 100, B, C, NULL), 2),               # K % 128 != 0
    ((A, 4, 1 << 25, B, C, NULL), 2),           # K over the limit
    ((A, 1 << 31, 128, B, C, NULL), 2),         # rows over the limit
    ((MIS, 4, 128, B, C, NULL), 3),             # misaligned input
    ((A, 4, 128, MIS, C, NULL), 3),             # misaligned output
])
@pytest.mark.parametrize("name", ["fp8_act_quant_group", "fp8_weight_block_quant"])
def test_quant_validation(lib, name, args, want):
    assert call(lib, name, *args) == want


@pytest.mark.parametrize("args,want", [
    ((NULL, B, C, D, 4, 256, 128, E_, NULL), 1),
    ((A, NULL, C, D, 4, 256, 128, E_, NULL), 1),
    ((A, B, C, D, 4, 256, 128, NULL, NULL), 1),
    ((A, B, C, D, -4, 256, 128, E_, NULL), 2),
    ((A, B, C, D, 4, -1, 128, E_, NULL), 2),
    ((A, B, C, D, 4, 256, 192, E_, NULL), 2),
    ((A, B, C, D, 4, 256, 128, MIS, NULL), 3),
    ((A, MIS, C, D, 4, 256, 128, E_, NULL), 3),
])
def test_gemm_validation(lib, args, want):
    assert call(lib, "fp8_block_gemm", *args) == want


@pytest.mark.parametrize("M,N,K,want", [
    (512, 1536, 7168, 5 * 512 * 1536 * 4),      # DeepSeek-V3 q_a: 48 tiles, 5 ranges of 12 K blocks
    (512, 576, 7168, 10 * 512 * 576 * 4),       # kv_a: 20 tiles, 10 ranges of 6 (the last of 2)
    (1024, 1024, 4096, 4 * 1024 * 1024 * 4),    # 64 tiles, 4 ranges of 8
    (65, 1, 5120, 10 * 68 * 4),                 # slices padded to a multiple of 4 floats
    (256, 7168, 2048, 0),                       # the model gains too little (measured slower)
    (300, 576, 2048, 0),
    (32, 1536, 7168, 0),                        # 17 <= M <= 32: the decode kernel, whole
    # 33 <= M <= 64 with K >= 6144: one row tile of 128 (rows padded), K split
    (64, 1536, 7168, 14 * 64 * 1536 * 4),       # DeepSeek-V3 q_a: 14 ranges of 4 K blocks
    (33, 4096, 14336, 8 * 33 * 4096 * 4),       # Llama down: 8 ranges of 14
    (33, 4096, 6144, 8 * 33 * 4096 * 4),        # K = 6144: the smallest K split at this M
    (33, 4096, 6016, 0),                        # K < 6144: the decode kernel
    (48, 4096, 4096, 0),
    (64, 14336, 4096, 0),                       # 112 tiles, K = 4096: the model gains too little
    (64, 7168, 18432, 7340032),                 # DeepSeek-V3 MLP down
    (4096, 1024, 4096, 0),                      # 256 tiles: the chip is full
    # 9 <= M <= 16: decode with four 16-column slabs per workgroup, K split
    # so that (N/64 column groups) x (splits) fills the chip
    (16, 4096, 14336, 4 * 16 * 4096 * 4),       # Llama down: 64 groups x 4 ranges of 28
    (9, 4096, 14336, 4 * 9 * 4096 * 4),         # M = 9: slices of 9 x 4096 floats
    (9, 4095, 14336, 4 * (9 * 4095 + 1) * 4),   # slices padded to a multiple of 4 floats
    (8, 4096, 14336, 0),                        # M <= 8: x is too small to be worth a split
    (1, 4096, 14336, 0),
    (16, 7168, 16384, 2 * 16 * 7168 * 4),       # DeepSeek-V3 o_proj: 112 groups x 2
    (16, 4000, 8192, 4 * 16 * 4000 * 4),        # ragged last group (250 slabs)
    (16, 4004, 8192, 4 * 16 * 4004 * 4),        # ragged last slab
    (16, 4096, 4096, 0),                        # 16 K blocks per range would leave 128 groups
    (16, 14336, 4096, 0),                       # four slabs already fill the chip
    (16, 1024, 4096, 0),                        # 16 groups: too few to split
    (17, 4096, 14336, 0),                       # two row fragments: not split
    (16, 4096, 128 * 600, 0),                   # past the scale-staging limit of the decode kernel
    (-1, 1536, 7168, 0), (512, 1536, 100, 0), (512, 0, 7168, 0),
    ((1 << 63) - 1, 1536, 7168, 0), (512, (1 << 63) - 1, 7168, 0), (512, 1536, (1 << 62), 0),
])
def test_gemm_workspace_bytes(lib, M, N, K, want):
    """The split plan is host arithmetic only (a time model picks the number
    of K ranges, then evens the ranges out); slices of M*N floats rounded up
    to a multiple of 4."""
    lib.fp8_block_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.fp8_block_gemm_workspace_bytes.argtypes = [ctypes.c_int64] * 3
    assert lib.fp8_block_gemm_workspace_bytes(M, N, K) == want


@pytest.mark.parametrize("M,N,K,want", [
    (512, 1536, 7168, 5 * 512 * 1536 * 4),      # even K-block ranges: 5 of 12
    (1000, 700, 5632, 5 * 1000 * 700 * 4),      # 44 blocks: ranges of 10 (9 rounded up), last 4
    (512, 1536, 7040, 0),                       # 55 K blocks: odd, never split
    (64, 1536, 7168, 0),
    (16, 4096, 14336, 0),                       # the decode split is fp32-scale only
])
def test_gemm_ue8m0_workspace_bytes(lib, M, N, K, want):
    lib.fp8_block_gemm_ue8m0_workspace_bytes.restype = ctypes.c_size_t
    lib.fp8_block_gemm_ue8m0_workspace_bytes.argtypes = [ctypes.c_int64] * 3
    assert lib.fp8_block_gemm_ue8m0_workspace_bytes(M, N, K) == want


@pytest.mark.parametrize("args,want", [
    ((NULL, B, C, D, 512, 1536, 7168, E_, A, 1 << 26, NULL), 1),
    ((A, B, C, D, 512, 1536, 7100, E_, A, 1 << 26, NULL), 2),
    ((A, B, C, D, 512, 1536, 7168, E_, MIS, 1 << 26, NULL), 3),   # the workspace would be used
    ((A, B, C, D, 512, 1536, 7168, MIS, A, 1 << 26, NULL), 3),
    ((A, B, C, D, (1 << 63) - 1, 1536, 7168, E_, A, 1 << 26, NULL), 2),
])
def test_gemm_ws_validation(lib, args, want):
    f = lib.fp8_block_gemm_ws
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    assert f(*args) == want


def test_gemm_ws_unused_workspace_is_not_checked(lib):
    """A workspace too small to be used (or for a shape that needs none) is
    ignored, misaligned or not: the call is fp8_block_gemm (here without a
    GPU: FP8BLK_ERR_DEVICE after the argument checks)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    f = lib.fp8_block_gemm_ws
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    assert f(A, B, C, D, 512, 1536, 7168, E_, MIS, 1024, NULL) == 4
    assert f(A, B, C, D, 4096, 1024, 4096, E_, MIS, 1 << 30, NULL) == 4


@pytest.mark.parametrize("args,want", [
    ((NULL, B, C, D, A, 4, 64, 256, 128, E_, NULL), 1),
    ((A, B, C, D, NULL, 4, 64, 256, 128, E_, NULL), 1),
    ((A, B, C, D, A, -1, 64, 256, 128, E_, NULL), 2),
    ((A, B, C, D, A, 4, 64, 256, 130, E_, NULL), 2),
    ((A, B, C, D, A, 4, -64, 256, 128, E_, NULL), 2),
    ((A, B, C, MIS, A, 4, 64, 256, 128, E_, NULL), 3),
])
def test_grouped_validation(lib, args, want):
    assert call(lib, "fp8_grouped_block_gemm", *args) == want


def test_valid_arguments_without_gpu_report_device(lib):
    """With valid arguments the next check is the device: in a container
    with no GPU it must answer FP8BLK_ERR_DEVICE, never crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call(lib, "fp8_act_quant_group", A, 4, 128, B, C, NULL) == 4
    assert call(lib, "fp8_block_gemm", A, B, C, D, 4, 256, 128, E_, NULL) == 4


@pytest.mark.parametrize("name", ["fp8_block_gemm", "fp8_block_gemm_static", "fp8_rowwise_gemm"])
def test_gemm_with_zero_columns_is_empty_work(lib, name):
    """N == 0 with M > 0 is empty work (no division by the zero size in the
    size checks): OK with a GPU, FP8BLK_ERR_DEVICE without."""
    import torch
    want = 0 if torch.cuda.is_available() else 4
    assert call(lib, name, NULL, NULL, NULL, NULL, 16, 0, 128, NULL, NULL) == want


def test_grouped_with_zero_columns_is_empty_work(lib):
    import torch
    want = 0 if torch.cuda.is_available() else 4
    assert call(lib, "fp8_grouped_block_gemm", NULL, NULL, NULL, NULL, NULL, 4, 64, 0, 128, NULL,
                NULL) == want


def test_empty_work_is_validated_then_ok_or_device(lib):
    """M == 0 skips the pointer checks but still checks shape and device."""
    import torch
    want = 0 if torch.cuda.is_available() else 4
    assert call(lib, "fp8_act_quant_group", NULL, 0, 128, NULL, NULL, NULL) == want
    assert call(lib, "fp8_act_quant_group", NULL, 0, 100, NULL, NULL, NULL) == 2
    assert call(lib, "fp8_block_gemm", NULL, NULL, NULL, NULL, 0, 16, 128, NULL, NULL) == want


def test_binding_raises_without_device():
    import torch
    import block_scaled_fp8_act_amd as fb
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fb.act_quant_group(x)  # CPU tensor: refused, no fallback


MIS1 = 0x10001       # odd address
MIS4 = 0x10004       # 4-byte aligned only


@pytest.mark.parametrize("name", ["fp8_act_quant_group_ue8m0", "fp8_weight_block_quant_ue8m0"])
def test_ue8m0_quant_validation(lib, name):
    assert call(lib, name, NULL, 4, 128, B, C, NULL) == 1
    assert call(lib, name, A, 4, 100, B, C, NULL) == 2
    assert call(lib, name, MIS, 4, 128, B, C, NULL) == 3
    # E8M0 byte arrays may sit at any address: the next check is the device
    import torch
    if not torch.cuda.is_available():
        assert call(lib, name, A, 4, 128, B, MIS1, NULL) == 4


def test_ue8m0_gemm_validation(lib):
    assert call(lib, "fp8_block_gemm_ue8m0", NULL, B, C, D, 4, 256, 128, E_, NULL) == 1
    assert call(lib, "fp8_block_gemm_ue8m0", A, B, C, D, 4, 256, 192, E_, NULL) == 2
    assert call(lib, "fp8_block_gemm_ue8m0", A, B, C, D, 4, 256, 128, MIS, NULL) == 3
    assert call(lib, "fp8_grouped_block_gemm_ue8m0", A, B, C, D, NULL, 4, 64, 256, 128, E_, NULL) == 1
    assert call(lib, "fp8_grouped_block_gemm_ue8m0", A, B, MIS, D, A, 4, 64, 256, 128, E_, NULL) == 3
    import torch
    if not torch.cuda.is_available():
        assert call(lib, "fp8_block_gemm_ue8m0", A, MIS1, C, MIS1, 4, 256, 128, E_, NULL) == 4


def test_static_validation(lib):
    # fp8_act_quant_static(x, M, K, x_scale, x_q, stream)
    assert call(lib, "fp8_act_quant_static", NULL, 4, 128, B, C, NULL) == 1
    assert call(lib, "fp8_act_quant_static", A, 4, 128, NULL, C, NULL) == 1
    assert call(lib, "fp8_act_quant_static", A, 4, 96, B, C, NULL) == 2
    assert call(lib, "fp8_act_quant_static", A, 4, 128, MIS1, C, NULL) == 3   # scale: 4-byte
    assert call(lib, "fp8_act_quant_static", A, 4, 128, B, MIS, NULL) == 3
    # fp8_block_gemm_static(x_q, x_scale, w_q, w_scale, M, N, K, y, stream)
    assert call(lib, "fp8_block_gemm_static", A, NULL, C, D, 4, 256, 128, E_, NULL) == 1
    assert call(lib, "fp8_block_gemm_static", A, B, C, D, 4, 256, 64, E_, NULL) == 2
    assert call(lib, "fp8_block_gemm_static", A, MIS1, C, D, 4, 256, 128, E_, NULL) == 3
    assert call(lib, "fp8_block_gemm_static", A, B, C, MIS, 4, 256, 128, E_, NULL) == 3
    import torch
    if not torch.cuda.is_available():
        assert call(lib, "fp8_act_quant_static", A, 4, 128, MIS4, C, NULL) == 4
        assert call(lib, "fp8_block_gemm_static", A, MIS4, C, D, 4, 256, 128, E_, NULL) == 4
        # empty shapes validate fully, then the device check still comes first
        assert call(lib, "fp8_block_gemm_static", A, B, C, D, 0, 256, 128, E_, NULL) == 4


def test_batched_and_rowwise_validation(lib):
    # fp8_batched_block_gemm(x_q, x_s, w_q, w_s, counts, E, C, N, K, y, stream)
    f = "fp8_batched_block_gemm"
    assert call(lib, f, A, B, C, D, NULL, 4, 64, 256, 128, E_, NULL) == 1
    assert call(lib, f, A, B, C, D, A, -1, 64, 256, 128, E_, NULL) == 2
    assert call(lib, f, A, B, C, D, A, 4, -64, 256, 128, E_, NULL) == 2
    assert call(lib, f, A, B, C, D, A, 4, 64, 256, 96, E_, NULL) == 2
    assert call(lib, f, A, B, C, D, A, 1 << 20, 1 << 20, 256, 128, E_, NULL) == 2   # E*C over 2^31
    assert call(lib, f, A, B, C, D, MIS1, 4, 64, 256, 128, E_, NULL) == 3       # counts: 4-byte
    assert call(lib, f, A, MIS, C, D, A, 4, 64, 256, 128, E_, NULL) == 3
    # fp8_rowwise_quant(in, R, K, q, scale, stream), fp8_rowwise_gemm(x_q, x_s, w_q, w_s, M, N, K, y, stream)
    assert call(lib, "fp8_rowwise_quant", NULL, 4, 128, B, C, NULL) == 1
    assert call(lib, "fp8_rowwise_quant", A, 4, 130, B, C, NULL) == 2
    assert call(lib, "fp8_rowwise_quant", A, 4, 128, B, MIS, NULL) == 3
    assert call(lib, "fp8_rowwise_gemm", A, B, C, NULL, 4, 256, 128, E_, NULL) == 1
    assert call(lib, "fp8_rowwise_gemm", A, B, C, D, 4, 256, 100, E_, NULL) == 2
    assert call(lib, "fp8_rowwise_gemm", A, B, C, MIS, 4, 256, 128, E_, NULL) == 3
    import torch
    if not torch.cuda.is_available():
        assert call(lib, f, A, B, C, D, MIS4, 4, 64, 256, 128, E_, NULL) == 4
        assert call(lib, "fp8_rowwise_quant", A, 4, 128, B, C, NULL) == 4
        assert call(lib, "fp8_rowwise_gemm", A, B, C, D, 4, 256, 128, E_, NULL) == 4


def test_swiglu_validation(lib):
    # fp8_swiglu_act_quant(gate_up, M, I, x_q, x_scale, stream)
    f = "fp8_swiglu_act_quant"
    assert call(lib, f, NULL, 4, 128, B, C, NULL) == 1
    assert call(lib, f, A, 4, 128, NULL, C, NULL) == 1
    assert call(lib, f, A, 4, 128, B, NULL, NULL) == 1
    assert call(lib, f, A, -1, 128, B, C, NULL) == 2
    assert call(lib, f, A, 4, 0, B, C, NULL) == 2
    assert call(lib, f, A, 4, 192, B, C, NULL) == 2
    assert call(lib, f, A, 1 << 30, 1 << 10, B, C, NULL) == 2     # 2^31 groups
    assert call(lib, f, MIS, 4, 128, B, C, NULL) == 3
    assert call(lib, f, A, 4, 128, MIS, C, NULL) == 3
    assert call(lib, f, A, 4, 128, B, MIS, NULL) == 3
    assert call(lib, f, NULL, 0, 128, NULL, NULL, NULL) in (0, 4)   # empty: no pointers needed
    g = "fp8_swiglu_act_quant_ue8m0"
    assert call(lib, g, NULL, 4, 128, B, C, NULL) == 1
    assert call(lib, g, A, 4, 192, B, C, NULL) == 2
    assert call(lib, g, A, 4, 128, MIS, C, NULL) == 3
    assert call(lib, g, A, 4, 128, B, MIS1, NULL) in (0, 4)          # byte scales: no alignment
    import torch
    if not torch.cuda.is_available():
        assert call(lib, f, A, 4, 128, B, C, NULL) == 4
        assert call(lib, g, A, 4, 128, B, MIS1, NULL) == 4


def test_linear_validation(lib):
    # fp8_linear(x, M, N, K, w_q, w_scale, x_q_ws, x_scale_ws, y, stream)
    f = "fp8_linear"
    assert call(lib, f, NULL, 16, 256, 128, C, D, NULL, NULL, E_, NULL) == 1
    assert call(lib, f, A, 65, 256, 128, C, D, NULL, NULL, E_, NULL) == 1      # workspaces needed
    assert call(lib, f, A, 65, 256, 128, C, D, B, NULL, E_, NULL) == 1
    assert call(lib, f, A, 16, 256, 100, C, D, NULL, NULL, E_, NULL) == 2
    assert call(lib, f, MIS, 16, 256, 128, C, D, NULL, NULL, E_, NULL) == 3
    assert call(lib, f, A, 65, 256, 128, C, D, MIS, B, E_, NULL) == 3
    import torch
    if not torch.cuda.is_available():
        # M <= 64 needs no workspace; a misaligned unused workspace is ignored
        assert call(lib, f, A, 64, 256, 128, C, D, NULL, NULL, E_, NULL) == 4
        assert call(lib, f, A, 16, 256, 128, C, D, MIS, MIS, E_, NULL) == 4


def test_ceiling_library_exports_and_checks_arguments():
    """libfp8ceil.so (the measurement-only matrix-core ceiling kernels timed
    by bench.py) exports exactly its two entry points and refuses bad
    arguments before any HIP call."""
    import subprocess
    from block_scaled_fp8_act_amd import build
    if not os.path.exists(build.CEIL_LIB):
        build.build()
    out = subprocess.run(["nm", "-D", "--defined-only", build.CEIL_LIB], capture_output=True,
                         text=True).stdout
    assert {l.split()[-1] for l in out.splitlines() if " T " in l} == {
        "fp8ceil_mfma", "fp8ceil_wall_clock_khz"}
    f = ctypes.CDLL(build.CEIL_LIB).fp8ceil_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    assert f(0, None, None, 8, 8, None) == -1
    assert f(1, A, None, 0, 8, None) == -1
    assert f(1, A, None, 8, 0, None) == -1
    assert f(-1, A, None, 8, 8, None) == -1
    assert f(4, A, A, 8, 8, None) == -1


def test_noalloc_scratch_covers_every_split_plan(lib):
    """fp8_block_gemm_noalloc keeps the K split's partial sums in a device
    array of FP8BLK_SCRATCH_BYTES: no split over workgroups may need more
    (tiled plans over M > 64 and decode plans over 9 <= M <= 16, scanned
    over sizes)."""
    import block_scaled_fp8_act_amd as fb
    header = open(HEADER).read()
    m = re.search(r"#define FP8BLK_SCRATCH_BYTES \(\(size_t\)16 \* 1024 \* 1024 \+ \(size_t\)64 \* 1024\)", header)
    assert m and fb.SCRATCH_BYTES == 16 * 1024 * 1024 + 64 * 1024
    worst = 0
    for K in (512, 1024, 2048, 4096, 7168, 14336, 18432, 32768, 65536):
        for M in list(range(9, 17)) + list(range(33, 65, 5)) + list(range(65, 2100, 37)):
            for N in list(range(1, 4200, 97)) + [576, 1536, 7168, 16384]:
                # past 128 output tiles of 128x128 (M > 64) the plan can only
                # be stream-K, which fp8_block_gemm_noalloc never runs
                if M > 64 and -(-M // 128) * -(-N // 128) > 128:
                    continue
                worst = max(worst, lib.fp8_block_gemm_workspace_bytes(M, N, K))
    assert 0 < worst <= fb.SCRATCH_BYTES, worst


def test_noalloc_validates_before_the_device(lib):
    st = lib.fp8_block_gemm_noalloc(A, B, C, D, -1, 64, 128, E_, None)
    assert st == 2
    st = lib.fp8_block_gemm_noalloc(A, B, C, D, 64, 64, 100, E_, None)
    assert st == 2
    st = lib.fp8_block_gemm_noalloc(A + 4, B, C, D, 64, 64, 128, E_, None)
    assert st == 3
    st = lib.fp8_block_gemm_noalloc(None, B, C, D, 64, 64, 128, E_, None)
    assert st == 1
    assert lib.fp8_block_gemm_noalloc(A, B, C, D, 0, 64, 128, E_, None) in (0, 4)


def test_stream_k_small_grid_plan(lib):
    """Grids of 32-191 256x256 tiles with K >= 7168 and more than 128
    128x128 tiles run wholly as stream-K when the model beats the 128x128
    kernels' estimate by 10 %: DeepSeek-V3 o_proj, MLP up and MLP down at
    M = 512, Llama down at M = 768; not MLP up at M = 384 (one round of
    128x128 tiles), short K, or the split-over-workgroups regime."""
    slot = 256 * 256 * 4
    lib.fp8_block_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.fp8_block_gemm_workspace_bytes.argtypes = [ctypes.c_int64] * 3
    assert lib.fp8_block_gemm_workspace_bytes(512, 7168, 16384) == 312 * slot
    assert lib.fp8_block_gemm_workspace_bytes(512, 18432, 7168) == 396 * slot
    assert lib.fp8_block_gemm_workspace_bytes(512, 7168, 18432) == 308 * slot
    assert lib.fp8_block_gemm_workspace_bytes(768, 4096, 14336) == 304 * slot
    assert lib.fp8_block_gemm_workspace_bytes(700, 4000, 14336) == 304 * slot
    for M, N, K in ((384, 18432, 7168), (512, 4096, 4096), (1536, 4096, 4096),
                    (1024, 4096, 14336), (512, 24576, 1536), (768, 18432, 7168)):
        assert lib.fp8_block_gemm_workspace_bytes(M, N, K) == 0, (M, N, K)


def test_stream_k_tail_plan(lib):
    """The stream-K tail: planned for 3.5 rounds of 256x256 tiles with long
    K (DeepSeek-V3 o_proj and MLP down at M = 8192: 128 tail tiles, 256
    ranges, slots for 384 pieces of 256 KB), not for full rounds (MLP up,
    q_b) nor for a short-K tail (Llama gate/up)."""
    slot = 256 * 256 * 4
    assert lib.fp8_block_gemm_workspace_bytes(8192, 7168, 16384) == 384 * slot
    assert lib.fp8_block_gemm_workspace_bytes(8192, 7168, 18432) == 384 * slot
    for M, N, K in ((8192, 18432, 7168), (8192, 24576, 1536), (4096, 14336, 4096),
                    (4096, 4096, 14336)):
        assert lib.fp8_block_gemm_workspace_bytes(M, N, K) == 0, (M, N, K)
