"""GPU parity of the block-scaled GEMM, the grouped GEMM and the linear
layer against the CPU oracle (fp64 dequantize-then-matmul).

Tolerance (from the library's acceptance rule): relative Frobenius error
<= 2e-3 and, for every element, |y - y_hat| <= 2^-8 |y_hat| + 2^-13 S with
S = sum_k |A||B| the magnitude of the summed terms, against the unrounded
fp64 y_hat (bf16 output rounding plus the fp8 matrix instruction's own
truncating summation, pinned by test_gpu_mfma_accum.py).  Exact pins (integer operands with
power-of-two scales; unit codes with distinct power-of-two scales) must be
bit-exact against bf16_RNE of the exact value."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import quant as oq
from gpu_helpers import assert_codes_equal, bf16_to_host, dev, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def gpu_gemm(xq, xs, wq, ws):
    y = fb.block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    return bf16_to_host(y)


def check_tol(y_bits, y_hat, S, what):
    rep = og.tolerance_report(y_bits, y_hat, S)
    say(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], (what, rep)
    return rep


def quantized_operands(x_bits, w_bits):
    xq, xs = oq.act_quant_group(x_bits)
    wq, ws = oq.weight_block_quant(w_bits)
    return xq, xs, wq, ws


# ----------------------------------------------------------------------------
# exact pins

@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (64, 192, 1024), (130, 576, 4096), (1, 300, 512),
                                   (40, 12300, 256), (64, 12288, 384), (3900, 3300, 4096),
                                   (4000, 3200, 640)])
def test_gemm_exact_integer_operands(M, N, K):
    """|codes| <= 8 integers, scales in {1/2, 1, 2}: every partial sum and
    every promotion is exact in fp32, so y must equal bf16_RNE(exact).
    (40, 12300) and (64, 12288): 33-64 rows with N >= 12288 take the tiled
    kernel (one padded row tile) instead of the decode kernel.  The last
    two run 256x256 tiles with ragged last row and column tiles: at
    K = 4096 the activation scales load four K blocks at a time, at
    K = 640 one block per step."""
    rng = np.random.default_rng(M + N + K)
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    y = gpu_gemm(xq, xs, wq, ws)
    exact = og.block_gemm(xq, xs, wq, ws)          # exact in fp64 here
    want = og.bf16_rne_bits(exact)
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(65, 128, 256), (130, 576, 384), (257, 1000, 640),
                                   (1024, 1024, 1152), (300, 2000, 2048)])
def test_gemm_split_k_tiles_exact(M, N, K):
    """Grids of at most 320 128x128 tiles run with K split over two wave
    groups inside the workgroup (odd K-block counts included: the second
    group's extra step must add nothing).  Integer operands with
    power-of-two scales keep every sum exact, so the order of the two
    partial sums cannot matter: bit-exact against bf16_RNE(exact)."""
    rng = np.random.default_rng(M * 7 + N + K)
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    y = gpu_gemm(xq, xs, wq, ws)
    want = og.bf16_rne_bits(og.block_gemm(xq, xs, wq, ws))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(100, 300, 384), (520, 1100, 1408), (4096, 1024, 640)])
def test_gemm_split_k_tiles_tolerance(M, N, K):
    x = synth.dsv3_activations(M + 5 * K, M, K, N)
    w = synth.normal_bf16(N + 3 * K, (N, K), 0.01)
    xq, xs, wq, ws = quantized_operands(x, w)
    rows = np.arange(M) if M <= 600 else np.sort(np.concatenate(
        [[0, M - 1], np.random.default_rng(1).choice(np.arange(1, M - 1), 126, replace=False)]))
    y = gpu_gemm(xq, xs, wq, ws)
    check_tol(y[rows], og.block_gemm(xq[rows], xs[rows], wq, ws),
              og.term_magnitude(xq[rows], xs[rows], wq, ws), f"split-K {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 14380, 256), (7, 7176, 384), (16, 14380, 512),
                                   (16, 14336, 1024), (3, 4100, 768),
                                   (17, 14380, 256), (32, 7176, 384), (24, 14336, 640),
                                   (33, 14380, 256), (64, 7176, 512), (48, 4100, 768),
                                   (64, 4096, 1024), (20, 8192, 384), (32, 8191, 256)])
def test_gemm_decode_multi_slab_exact(M, N, K):
    """Decode shapes for which the launcher packs four (N = 14380, 14336 at
    M <= 32) or two (N = 7176 and 4100, and every packed shape at M = 33-64)
    16-column slabs per workgroup, with a partly empty last workgroup and a
    ragged last slab, and one unpacked shape (N = 4096 at M = 64): integer
    operands, power-of-two scales, bit-exact against bf16_RNE(exact).  At
    17-32 rows N >= 8192 runs 8 waves per workgroup (14380, 14336, and
    8192 against 8191 at the boundary), narrower N 16."""
    rng = np.random.default_rng(M * 5 + N + K)
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    y = gpu_gemm(xq, xs, wq, ws)
    want = og.bf16_rne_bits(og.block_gemm(xq, xs, wq, ws))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(8, 256, 1536), (33, 200, 1280)])
def test_gemm_scale_indexing(M, N, K):
    """All codes 1.0; x_s[m,kb] = 2^((kb+m) % KB), w_s[nb,kb] = 2^(KB*((kb+nb)%2)):
    each output is 128 * a sum of distinct powers of two, exact in fp32,
    so a wrong or transposed scale index changes its bits."""
    KB, NB = K // 128, -(-N // 128)
    xq = np.full((M, K), 0x38, np.uint8); wq = np.full((N, K), 0x38, np.uint8)
    xs = np.array([[2.0 ** ((kb + m) % KB) for kb in range(KB)] for m in range(M)], np.float32)
    ws = np.array([[2.0 ** (KB * ((kb + nb) % 2) - 20) for kb in range(KB)] for nb in range(NB)],
                  np.float32)
    y = gpu_gemm(xq, xs, wq, ws)
    want = og.bf16_rne_bits(og.block_gemm(xq, xs, wq, ws))
    assert np.array_equal(y, want)


# ----------------------------------------------------------------------------
# tolerance parity

def test_gemm_tiny():
    x, w = synth.tiny_inputs()
    xq, xs, wq, ws = quantized_operands(x, w)
    check_tol(gpu_gemm(xq, xs, wq, ws), og.block_gemm(xq, xs, wq, ws),
              og.term_magnitude(xq, xs, wq, ws), "tiny")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (15, 100, 256), (17, 576, 384),
                                   (130, 300, 1024), (257, 1000, 512), (16, 4096, 4096),
                                   (200, 129, 7168), (129, 257, 128), (33, 4096, 4096),
                                   (40, 300, 512), (64, 1024, 2048), (65, 256, 256),
                                   (2, 24576, 1536), (3, 576, 18432), (520, 3000, 1280)])
def test_gemm_ragged(M, N, K):
    x = synth.dsv3_activations(M + 11 * K, M, K, N)
    w = synth.normal_bf16(N + 13 * K, (N, K), 0.02)
    xq, xs, wq, ws = quantized_operands(x, w)
    check_tol(gpu_gemm(xq, xs, wq, ws), og.block_gemm(xq, xs, wq, ws),
              og.term_magnitude(xq, xs, wq, ws), f"ragged {M}x{N}x{K}")


@pytest.mark.parametrize("shape_index", range(4))
@pytest.mark.parametrize("M", [1, 4, 16, 32, 64])
def test_gemm_llama_decode(shape_index, M):
    x, w = synth.llama_inputs(shape_index, M, config=2)
    xq, xs, wq, ws = quantized_operands(x, w)
    check_tol(gpu_gemm(xq, xs, wq, ws), og.block_gemm(xq, xs, wq, ws),
              og.term_magnitude(xq, xs, wq, ws), f"llama decode {synth.LLAMA_SHAPES[shape_index][0]} M={M}")


def _sampled_rows_check(x, w, rows, what):
    """Full GEMM on the GPU from bf16 x (the GPU quantizes it), oracle on
    sampled rows: the oracle quantizes those rows of x itself (row-local),
    the GPU's codes and scales of those rows must equal the oracle's, and
    the GEMM outputs of those rows are checked against the oracle's GEMM of
    the oracle's operands."""
    xd = to_dev_bf16(x)
    xq, xs = fb.act_quant_group(xd)
    wq, ws = oq.weight_block_quant(w)
    y = fb.block_gemm(xq, xs, to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    y = bf16_to_host(y)
    oxq, oxs = oq.act_quant_group(x[rows])
    assert_codes_equal(host(xq)[rows], host(xs)[rows], oxq, oxs, what)
    want = og.block_gemm(oxq, oxs, wq, ws)
    return check_tol(y[rows], want, og.term_magnitude(oxq, oxs, wq, ws), what)


@pytest.mark.parametrize("shape_index", range(4))
def test_gemm_llama_prefill_sampled(shape_index):
    x, w = synth.llama_inputs(shape_index, 4096, config=3)
    rows = np.concatenate([[0, 4095], np.random.default_rng(shape_index).choice(4096, 62, replace=False)])
    _sampled_rows_check(x, w, np.sort(rows), f"llama prefill {synth.LLAMA_SHAPES[shape_index][0]}")


@pytest.mark.parametrize("shape_index", range(6))
@pytest.mark.parametrize("M", [512, 8192])
def test_gemm_dsv3_sampled(shape_index, M):
    x, w = synth.dsv3_inputs(shape_index, M)
    rows = np.concatenate([[0, M - 1], np.random.default_rng(M + shape_index).choice(M, 30, replace=False)])
    _sampled_rows_check(x, w, np.sort(rows), f"dsv3 {synth.DSV3_SHAPES[shape_index][0]} M={M}")


def test_linear_matches_oracle_linear():
    x, w = synth.llama_inputs(1, 64, config=3)
    wq, ws = oq.weight_block_quant(w)
    y = fb.linear(to_dev_bf16(x), to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    xq, xs = oq.act_quant_group(x)
    check_tol(bf16_to_host(y), og.linear(x, wq, ws), og.term_magnitude(xq, xs, wq, ws), "linear")


def test_gemm_empty_and_errors():
    d = dev()
    xq = torch.zeros((0, 256), dtype=torch.uint8, device=d)
    xs = torch.zeros((0, 2), dtype=torch.float32, device=d)
    wq = torch.zeros((64, 256), dtype=torch.uint8, device=d)
    ws = torch.zeros((1, 2), dtype=torch.float32, device=d)
    assert fb.block_gemm(xq, xs, wq, ws).shape == (0, 64)
    with pytest.raises(TypeError):
        fb.block_gemm(xq.float(), xs, wq, ws)


# ----------------------------------------------------------------------------
# K split over workgroups (fp8_block_gemm_ws): grids of at most 128 tiles of
# 128x128 and at least 8 K blocks

def gpu_gemm_ws(xq, xs, wq, ws, work_bytes=None, fill=0xFF):
    """fp8_block_gemm_ws with a workspace of work_bytes (default: what the
    library asks for) pre-filled with `fill` bytes (0xFF: fp32 NaN, so any
    partial sum the kernels leave unwritten would show).  Returns y and the
    workspace."""
    M, K = xq.shape
    N = wq.shape[0]
    nbytes = fb.fp8_block_gemm_workspace_bytes(M, N, K) if work_bytes is None else work_bytes
    work = torch.full((max(nbytes, 1),), fill, dtype=torch.uint8, device=dev())
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm_ws(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), y,
                         work if nbytes else None)
    torch.cuda.synchronize()
    return bf16_to_host(y), work


def gpu_gemm_plain(xq, xs, wq, ws):
    M, N = xq.shape[0], wq.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), y)
    torch.cuda.synchronize()
    return bf16_to_host(y)


@pytest.mark.parametrize("M,N,K", [(65, 1536, 7168), (130, 100, 3072), (77, 333, 5760),
                                   (1000, 700, 5632), (512, 1536, 7168), (257, 129, 4096),
                                   (40, 1000, 8192), (48, 576, 7168), (33, 300, 6144)])
def test_gemm_split_over_workgroups_exact(M, N, K):
    """Integer operands with power-of-two scales: every partial sum of every
    K range, and their sum, is exact in fp32, so the split result must equal
    bf16_RNE(exact) bit for bit (ranges, scale offsets and the reduction
    indexing are all checked).  The shapes cover ragged M and N, ranges of
    an odd number of K blocks (77x333x5760: 9 ranges of 5), a shorter
    last range (1000x700x5632: 5 ranges of 9, the last of 8), and 33-64
    rows with K >= 6144 (one row tile of 128, most of it padding)."""
    assert fb.fp8_block_gemm_workspace_bytes(M, N, K) > 0, "shape must take the split path"
    rng = np.random.default_rng(M * 13 + N + K)
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    say("split", M, N, K, "workspace", fb.fp8_block_gemm_workspace_bytes(M, N, K))
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    want = og.bf16_rne_bits(og.block_gemm(xq, xs, wq, ws))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("shape_index", [0, 2])
def test_gemm_split_over_workgroups_dsv3_m512(shape_index):
    """DeepSeek-V3 q_a (7168 -> 1536) and kv_a (7168 -> 576) at M = 512:
    48 and 20 tiles, split 5 and 12 ways; every row against the oracle."""
    x, w = synth.dsv3_inputs(shape_index, 512)
    xq, xs, wq, ws = quantized_operands(x, w)
    M, K = xq.shape
    assert fb.fp8_block_gemm_workspace_bytes(M, wq.shape[0], K) > 0
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    check_tol(y, og.block_gemm(xq, xs, wq, ws), og.term_magnitude(xq, xs, wq, ws),
              f"split dsv3 {synth.DSV3_SHAPES[shape_index][0]} M=512")


@pytest.mark.parametrize("M,N,K", [(77, 333, 5760), (300, 576, 4096)])
def test_gemm_split_over_workgroups_tolerance_ragged(M, N, K):
    x = synth.dsv3_activations(M + 3 * K, M, K, N)
    w = synth.normal_bf16(N + 5 * K, (N, K), 0.01)
    xq, xs, wq, ws = quantized_operands(x, w)
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    check_tol(y, og.block_gemm(xq, xs, wq, ws), og.term_magnitude(xq, xs, wq, ws),
              f"split {M}x{N}x{K}")


# Decode (9 <= M <= 16) with long K: four 16-column slabs per workgroup and the K
# blocks split over workgroups (fp8_block_gemm_ws)

@pytest.mark.parametrize("M,N,K", [(16, 4096, 8192), (16, 4096, 128 * 71), (9, 4000, 8192),
                                   (11, 4004, 8192), (13, 4040, 8320), (16, 3072, 8192)])
def test_decode_split_exact(M, N, K):
    """Integer operands with power-of-two scales (every partial sum exact in
    fp32): the split decode GEMM must equal bf16_RNE(exact) bit for bit.
    Ranges of 16 K blocks (4096x8192), a shorter last range (71 blocks:
    18, 18, 18, 17), a partial last 64-column group (N = 4000) and a
    partial last slab (N = 4004, 4040), M = 9, 11 and 13 (rows past M
    masked)."""
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    assert need > 0, "shape must take the split decode path"
    rng = np.random.default_rng(M * 7 + N + K)
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    say("decode split", M, N, K, "workspace", need)
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    want = og.bf16_rne_bits(og.block_gemm(xq, xs, wq, ws))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K,seed", [(16, 4096, 14336, 1), (12, 7168, 16384, 2)])
def test_decode_split_tolerance(M, N, K, seed):
    """Llama-3-8B down (4096 x 14336) at M = 16 and DeepSeek-V3 o_proj
    (7168 x 16384) at M = 12 on synthetic activations: the split decode GEMM
    against the oracle within the GEMM tolerance, and two calls give the
    same bits (fixed reduction order)."""
    x = synth.dsv3_activations(seed, M, K, N)
    w = synth.normal_bf16(seed + 100, (N, K), 0.01)
    xq, xs, wq, ws = quantized_operands(x, w)
    assert fb.fp8_block_gemm_workspace_bytes(M, N, K) > 0
    say("decode split", M, N, K)
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    y2, _ = gpu_gemm_ws(xq, xs, wq, ws, fill=0x00)
    assert np.array_equal(y, y2)
    check_tol(y, og.block_gemm(xq, xs, wq, ws), og.term_magnitude(xq, xs, wq, ws),
              f"decode split {M}x{N}x{K}")


def test_gemm_ws_without_usable_workspace_is_fp8_block_gemm():
    """No workspace, or one byte too small: the call is fp8_block_gemm (same
    bits) and a too-small workspace is left untouched."""
    M, N, K = 300, 576, 4096
    x = synth.dsv3_activations(11, M, K, 12)
    w = synth.normal_bf16(13, (N, K), 0.01)
    xq, xs, wq, ws = quantized_operands(x, w)
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    assert need > 0
    plain = gpu_gemm_plain(xq, xs, wq, ws)
    y0, _ = gpu_gemm_ws(xq, xs, wq, ws, work_bytes=0)
    y1, work = gpu_gemm_ws(xq, xs, wq, ws, work_bytes=need - 1, fill=0x5A)
    assert np.array_equal(y0, plain) and np.array_equal(y1, plain)
    assert bool((work == 0x5A).all()), "a workspace that is not used was written"


def test_gemm_ws_large_grid_ignores_workspace():
    """4096x1024 outputs fill the chip (256 tiles of 128x128): no split, the
    same bits as fp8_block_gemm even with a workspace given, which stays
    untouched."""
    M, N, K = 4096, 1024, 1024
    assert fb.fp8_block_gemm_workspace_bytes(M, N, K) == 0
    rng = np.random.default_rng(5)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    xs = np.exp2(rng.integers(-3, 3, (M, K // 128))).astype(np.float32)
    ws = np.exp2(rng.integers(-3, 3, (N // 128, K // 128))).astype(np.float32)
    plain = gpu_gemm_plain(xq, xs, wq, ws)
    y, work = gpu_gemm_ws(xq, xs, wq, ws, work_bytes=1 << 20, fill=0x5A)
    assert np.array_equal(y, plain)
    assert bool((work == 0x5A).all())


def test_gemm_ws_misaligned_workspace_raises():
    M, N, K = 512, 1536, 7168
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    d = dev()
    xq = torch.zeros((M, K), dtype=torch.uint8, device=d)
    xs = torch.zeros((M, K // 128), dtype=torch.float32, device=d)
    wq = torch.zeros((N, K), dtype=torch.uint8, device=d)
    ws = torch.zeros((N // 128, K // 128), dtype=torch.float32, device=d)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    work = torch.empty(need + 16, dtype=torch.uint8, device=d)[1:]
    with pytest.raises(fb.Fp8BlkError) as e:
        fb.fp8_block_gemm_ws(xq, xs, wq, ws, y, work)
    assert e.value.status == 3


# ----------------------------------------------------------------------------
# stream-K tail (fp8_block_gemm_ws on 3.5 rounds of 256x256 tiles, long K)

def test_stream_k_tail_exact_ragged():
    """8000 x 7000 x 16384: 32 x 28 tiles of 256x256, the last 128 (8-row
    group 3, columns 12..27, incl. the ragged last row and column tiles)
    split over 256 ranges of 64 K blocks.  Integer operands with
    power-of-two scales keep every partial sum exact, so the rows checked --
    all in the tail's row range or in the whole tiles -- must equal
    bf16_RNE(exact) bit for bit; a second call gives the same bits."""
    M, N, K = 8000, 7000, 16384
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    assert need == 384 * 256 * 256 * 4
    rng = np.random.default_rng(17)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    y2, _ = gpu_gemm_ws(xq, xs, wq, ws, fill=0x00)
    assert np.array_equal(y, y2)
    rows = np.sort(np.concatenate([[0, 255, 6143, 6144, 7935, 7936, M - 1],
                                   rng.choice(np.arange(6144, M), 40, replace=False),
                                   rng.choice(np.arange(0, 6144), 16, replace=False)]))
    want = og.bf16_rne_bits(og.block_gemm(xq[rows], xs[rows], wq, ws))
    bad = np.argwhere(y[rows] != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N", [(768, 4096), (700, 4000)])
def test_stream_k_small_grid_exact(M, N):
    """A grid of 48 256x256 tiles with K = 14336 (112 blocks) runs entirely
    as stream-K: 256 ranges of 21 K blocks over the linearized (tile, block)
    space, every range spanning one or two tiles, no data-parallel part.
    700 x 4000 makes the last row and column tiles ragged.  Integer
    operands with power-of-two scales keep every partial sum exact, so the
    sampled rows (from every row tile) must equal bf16_RNE(exact) in every
    column; a second call into a zero-filled workspace gives the same
    bits."""
    K = 14336
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    assert need == 304 * 256 * 256 * 4
    rng = np.random.default_rng(M + N)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (NB, KB))).astype(np.float32)
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    y2, _ = gpu_gemm_ws(xq, xs, wq, ws, fill=0x00)
    assert np.array_equal(y, y2)
    rows = np.unique(np.concatenate([[0, 255, 256, 511, 512, M - 1],
                                     rng.choice(M, 26, replace=False)]))
    want = og.bf16_rne_bits(og.block_gemm(xq[rows], xs[rows], wq, ws))
    bad = np.argwhere(y[rows] != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


def test_stream_k_small_grid_dsv3_m512_tolerance():
    """DeepSeek-V3 o_proj at M = 512 (56 tiles of 256x256, K = 16384) on the
    small-grid stream-K path, data-like operands quantized by the oracle:
    every row within the GEMM tolerance."""
    M, N, K = 512, 7168, 16384
    assert fb.fp8_block_gemm_workspace_bytes(M, N, K) == 312 * 256 * 256 * 4
    x = synth.dsv3_activations(77, M, K, 78)
    w = synth.normal_bf16(79, (N, K), 0.01)
    xq, xs, wq, ws = quantized_operands(x, w)
    y, _ = gpu_gemm_ws(xq, xs, wq, ws)
    check_tol(y, og.block_gemm(xq, xs, wq, ws), og.term_magnitude(xq, xs, wq, ws),
              "stream-K small grid o_proj M=512")


def test_stream_k_tail_without_workspace_is_plain():
    """Without a large enough workspace the stream-K shape runs
    fp8_block_gemm (same bits) and leaves the workspace alone."""
    M, N, K = 8000, 7000, 16384
    rng = np.random.default_rng(18)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    xs = np.ones((M, K // 128), np.float32)
    ws = np.ones((-(-N // 128), K // 128), np.float32)
    plain = gpu_gemm_plain(xq, xs, wq, ws)
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    y, work = gpu_gemm_ws(xq, xs, wq, ws, work_bytes=need - 16, fill=0x5A)
    assert np.array_equal(y, plain)
    assert bool((work == 0x5A).all())


# ----------------------------------------------------------------------------
# grouped GEMM

def _grouped_case(sizes, N, K, seed):
    E = len(sizes)
    off = synth.random_offsets(0, E, sizes=sizes)
    total = int(off[-1])
    x = synth.dsv3_activations(seed, total, K, seed + 1)
    w = synth.normal_bf16(seed + 2, (E, N, K), 0.01)
    xq, xs = oq.act_quant_group(x)
    NB = -(-N // 128)
    wq = np.empty((E, N, K), np.uint8); ws = np.empty((E, NB, K // 128), np.float32)
    for e in range(E):
        wq[e], ws[e] = oq.weight_block_quant(w[e])
    return xq, xs, wq, ws, off


@pytest.mark.parametrize("sizes,N,K", [
    ([0, 1, 15, 16, 17, 0, 130, 3], 256, 512),
    ([5], 576, 384),
    ([0, 0, 0, 40], 128, 128),
    ([129, 255, 1, 0, 64], 300, 1024),
])
def test_grouped_matches_oracle_and_per_expert_gemm(sizes, N, K):
    xq, xs, wq, ws, off = _grouped_case(sizes, N, K, sum(sizes) + N)
    total = int(off[-1])
    y = fb.grouped_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(off))
    torch.cuda.synchronize()
    y = bf16_to_host(y)
    check_tol(y, og.grouped_block_gemm(xq, xs, wq, ws, off),
              og.grouped_term_magnitude(xq, xs, wq, ws, off), f"grouped {sizes}")
    # each expert's rows also agree with the plain GEMM on that expert (the two
    # may pick different tile configurations, so only to the tolerance)
    for e in range(len(sizes)):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            ye = gpu_gemm(xq[r0:r1], xs[r0:r1], wq[e], ws[e])
            check_tol(ye, og.block_gemm(xq[r0:r1], xs[r0:r1], wq[e], ws[e]),
                      og.term_magnitude(xq[r0:r1], xs[r0:r1], wq[e], ws[e]), f"plain expert {e}")
            diff = np.abs(og.bf16_bits_to_f64(ye) - og.bf16_bits_to_f64(y[r0:r1]))
            # both within the allowance of the same y_hat: at most twice it apart
            yh = og.block_gemm(xq[r0:r1], xs[r0:r1], wq[e], ws[e])
            allow = og.BF16_U * np.abs(yh) + og.ACC_TOL * og.term_magnitude(
                xq[r0:r1], xs[r0:r1], wq[e], ws[e])
            assert np.all(diff <= 2 * allow), f"expert {e}: grouped and plain GEMM disagree"


@pytest.mark.parametrize("sizes,N,K", [
    ([65, 300, 1, 129, 256, 0, 383, 128, 511], 300, 1024),
    ([7, 200, 120], 256, 2048),
])
def test_grouped_ragged_tiles_exact(sizes, N, K):
    """Integer operands with power-of-two scales: every sum is exact, so each
    expert's rows must equal bf16_RNE(exact) bit for bit.  The sizes put
    every kind of last row tile in play: at most 128 rows (its upper half
    of waves idle and its rows unstaged), 129-255 rows, exactly 128 and 256,
    single rows and empty experts."""
    E = len(sizes)
    off = synth.random_offsets(0, E, sizes=sizes)
    total = int(off[-1])
    rng = np.random.default_rng(sum(sizes) + N + K)
    xq = oe.encode(rng.integers(-8, 9, (total, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (E, N, K)).astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xs = np.exp2(rng.integers(-1, 2, (total, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(0, 2, (E, NB, KB))).astype(np.float32)
    y = fb.grouped_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(off))
    torch.cuda.synchronize()
    y = bf16_to_host(y)
    want = og.bf16_rne_bits(og.grouped_block_gemm(xq, xs, wq, ws, off))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


def test_grouped_rows_outside_experts_untouched():
    xq, xs, wq, ws, off = _grouped_case([3, 4], 128, 256, 77)
    total = int(off[-1]) + 5                            # 5 trailing rows of no expert
    xq = np.concatenate([xq, np.zeros((5, 256), np.uint8)])
    xs = np.concatenate([xs, np.ones((5, 2), np.float32)])
    y = torch.full((total, 128), 7.0, dtype=torch.bfloat16, device=dev())
    fb.fp8_grouped_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(off), y)
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy()
    assert np.all(yh[-5:] == 7.0)


@pytest.mark.parametrize("which", [0, 1])
def test_grouped_moe_sampled(which):
    """DeepSeek-V3 MoE share (32 experts, ragged Zipf loads) on the GPU from
    bf16 inputs (the GPU quantizes x and every expert's weights).  For every
    expert the oracle quantizes 3 of its rows of x and one random 128-row
    block row of its weights itself (both quantizers are local to a row
    group or a block, so these equal the full quantization's), the GPU's
    codes and scales there must equal the oracle's, and the GEMM outputs at
    those rows and 128 columns are checked against the oracle's GEMM of the
    oracle's operands."""
    x, w, off = synth.moe_inputs(which)
    E, N, K = w.shape
    say("moe", which, x.shape, w.shape, "sizes", np.diff(off).min(), np.diff(off).max())
    xd = to_dev_bf16(x)
    xq, xs = fb.act_quant_group(xd)
    wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev())
    ws = torch.empty((E, -(-N // 128), K // 128), dtype=torch.float32, device=dev())
    for e in range(E):
        fb.fp8_weight_block_quant(to_dev_bf16(w[e]), wq[e], ws[e])
    y = fb.grouped_block_gemm(xq, xs, wq, ws, to_dev(off))
    torch.cuda.synchronize()
    y = bf16_to_host(y)
    xq_h, xs_h, wq_h, ws_h = host(xq), host(xs), host(wq), host(ws)
    rng = np.random.default_rng(which)
    got, want, mag = [], [], []
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        pick = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, 1)]))
        oxq, oxs = oq.act_quant_group(x[pick])
        assert_codes_equal(xq_h[pick], xs_h[pick], oxq, oxs, f"moe {which} expert {e} rows")
        nb = int(rng.integers(0, -(-N // 128)))
        c0, c1 = 128 * nb, min(N, 128 * nb + 128)
        owq, ows = oq.weight_block_quant(w[e][c0:c1])
        assert_codes_equal(wq_h[e][c0:c1], ws_h[e][nb:nb + 1], owq, ows,
                           f"moe {which} expert {e} weight block row {nb}")
        got.append(y[pick][:, c0:c1])
        want.append(og.block_gemm(oxq, oxs, owq, ows))
        mag.append(og.term_magnitude(oxq, oxs, owq, ows))
    check_tol(np.concatenate(got), np.concatenate(want), np.concatenate(mag), f"moe {which}")
