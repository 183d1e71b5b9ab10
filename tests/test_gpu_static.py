"""GPU parity of the static-activation-scale path (one calibrated fp32 scale
per tensor) against the CPU oracle.

Quantizer: codes bit-exact on ragged and workload shapes, on every finite
bf16 value under 96 scales (powers of two, near-ties, tiny scales whose
quotients overflow, huge and subnormal scales), including saturation.
GEMM: bit-exact on exact-arithmetic pins, otherwise the block-scaled GEMM's
tolerance (relative Frobenius <= 2e-3, per element <= 1e-2 *
max(|y_hat|, 2^-6 * S)), in every tile configuration (decode, 128x128,
256x256)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import quant as oq
from oracle import static as ost
from gpu_helpers import bf16_to_host, dev, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def scale_dev(s):
    return torch.tensor([np.float32(s)], dtype=torch.float32, device=dev())


def gpu_static_quant(x_bits, s):
    q = fb.act_quant_static(to_dev_bf16(x_bits), scale_dev(s))
    torch.cuda.synchronize()
    return host(q)


def assert_codes(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[:3].tolist()}: " \
        f"{got[tuple(bad[0])]:#x} vs {want[tuple(bad[0])]:#x}"


def all_finite_bf16():
    """Every finite bf16 value (both signs, both zeros) as [N, 128]."""
    b = np.arange(0, 0x7F80, dtype=np.uint16)
    v = np.concatenate([b, b | 0x8000]).astype(np.uint16)
    pad = (-len(v)) % 128
    return np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(-1, 128)


def scale_set():
    rng = np.random.default_rng(5)
    s = [1.0, 0.5, 2.0, 3.0, 7.0, 0.37, 1 / 448, 2.0 ** -20, 2.0 ** 20, 1e-30, 1e30,
         1e-38, 1.5e-40, 3.4e38, 448.0, 0.1, 0.3, 1.1, 13.0]
    s += list(np.exp2(rng.uniform(-60, 60, 40)))
    s += list(rng.uniform(0.5, 2.0, 37))
    return [np.float32(v) for v in s]


@pytest.mark.parametrize("chunk", range(4))
def test_static_quant_every_bf16_value(chunk):
    x = all_finite_bf16()
    scales = scale_set()
    part = scales[chunk::4]
    say(f"static quant: {x.size} bf16 values x {len(part)} scales")
    for s in part:
        assert_codes(gpu_static_quant(x, s), ost.act_quant_static(x, s), f"scale {float(s)!r}")


@pytest.mark.parametrize("M,K,s", [(1, 128, 0.05), (3, 384, 1.0), (17, 512, 0.013),
                                   (5, 1536, 3.0), (33, 2048, 1e-3), (4, 14336, 0.2),
                                   (127, 7168, 0.02), (4096, 4096, 0.05)])
def test_static_quant_ragged(M, K, s):
    x = synth.dsv3_activations(M * 7 + K, M, K, M + 3)
    say("static quant", M, K, s)
    assert_codes(gpu_static_quant(x, s), ost.act_quant_static(x, s), f"{M}x{K}")


def test_static_scale_read_on_device():
    """The scale lives in device memory: changing it between calls changes
    the codes with no other argument touched."""
    x = synth.normal_bf16(3, (8, 256))
    xd = to_dev_bf16(x)
    sd = scale_dev(1.0)
    q = torch.empty((8, 256), dtype=torch.uint8, device=dev())
    fb.fp8_act_quant_static(xd, sd, q)
    torch.cuda.synchronize()
    assert_codes(host(q), ost.act_quant_static(x, 1.0), "s=1")
    sd.fill_(0.01)
    fb.fp8_act_quant_static(xd, sd, q)
    torch.cuda.synchronize()
    assert_codes(host(q), ost.act_quant_static(x, np.float32(0.01)), "s=0.01")


# ----------------------------------------------------------------------------
# GEMM

def gpu_gemm_static(xq, s, wq, ws):
    y = fb.block_gemm_static(to_dev(xq), scale_dev(s), to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    return bf16_to_host(y)


def check_tol(y_bits, y_hat, S, what):
    rep = og.tolerance_report(y_bits, y_hat, S)
    say(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], (what, rep)


@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (64, 192, 1024), (130, 576, 4096),
                                   (1, 300, 512), (300, 520, 768), (2048, 2048, 512),
                                   (32, 14380, 256), (64, 7176, 384), (40, 12300, 256)])
def test_static_gemm_exact_integer_operands(M, N, K):
    """Integer codes |c| <= 8, activation scale 0.5, weight scales in
    {1/2, 1, 2}: exact in fp32, so y must equal bf16_RNE(exact).  The last
    three take the decode kernel with four and two column slabs per
    workgroup (M = 32, 64) and the tiled kernel at M = 33-64 with
    N >= 12288."""
    rng = np.random.default_rng(M + N + K)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    ws = np.exp2(rng.integers(-1, 2, (-(-N // 128), K // 128))).astype(np.float32)
    y = gpu_gemm_static(xq, 0.5, wq, ws)
    want = og.bf16_rne_bits(ost.block_gemm_static(xq, 0.5, wq, ws))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (15, 100, 256), (17, 576, 384),
                                   (130, 300, 1024), (257, 1000, 512), (16, 4096, 4096),
                                   (64, 1024, 2048), (65, 256, 256), (520, 3000, 1280),
                                   (3, 576, 18432)])
def test_static_gemm_ragged(M, N, K):
    x = synth.dsv3_activations(M + 11 * K, M, K, N)
    w = synth.normal_bf16(N + 13 * K, (N, K), 0.02)
    s = np.float32(0.05)
    xq = ost.act_quant_static(x, s)
    wq, ws = oq.weight_block_quant(w)
    check_tol(gpu_gemm_static(xq, s, wq, ws), ost.block_gemm_static(xq, s, wq, ws),
              ost.term_magnitude_static(xq, s, wq, ws), f"static {M}x{N}x{K}")


@pytest.mark.parametrize("shape_index", range(4))
@pytest.mark.parametrize("M", [1, 16, 4096])
def test_static_linear_llama(shape_index, M):
    x, w = synth.llama_inputs(shape_index, M, config=3 if M > 16 else 2)
    s = np.float32(0.06)
    wq, ws = oq.weight_block_quant(w)
    y = bf16_to_host(fb.linear_static(to_dev_bf16(x), scale_dev(s), to_dev(wq), to_dev(ws)))
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 16 else np.sort(np.concatenate(
        [[0, M - 1], np.random.default_rng(shape_index).choice(np.arange(1, M - 1), 62, replace=False)]))
    xq = ost.act_quant_static(x[rows], s)
    check_tol(y[rows], ost.block_gemm_static(xq, s, wq, ws), ost.term_magnitude_static(xq, s, wq, ws),
              f"static linear {synth.LLAMA_SHAPES[shape_index][0]} M={M}")


def test_static_gemm_matches_dynamic_gemm_with_broadcast_scales():
    """The static GEMM is the dynamic GEMM with the scale broadcast to every
    (row, K block): same kernels, same order, identical bits."""
    x = synth.dsv3_activations(9, 300, 1024, 4)
    w = synth.normal_bf16(10, (700, 1024), 0.02)
    s = np.float32(0.04)
    xq = ost.act_quant_static(x, s)
    wq, ws = oq.weight_block_quant(w)
    y1 = gpu_gemm_static(xq, s, wq, ws)
    y2 = torch.empty((300, 700), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm(to_dev(xq), to_dev(np.full((300, 8), s, np.float32)), to_dev(wq),
                      to_dev(ws), y2)
    torch.cuda.synchronize()
    y2 = bf16_to_host(y2)
    assert np.array_equal(y1, y2)
