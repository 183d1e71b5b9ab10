"""GPU parity of the whole linear layer in one C call (fp8_linear): the
fused decode kernel (activation quantization inside the weight-streaming
GEMM, M <= 64) and the two-kernel path through workspaces (M > 64).

The fused result equals the two-launch result (fp8_act_quant_group then
fp8_block_gemm) bit for bit where the two-launch GEMM is the decode kernel
(same K split over the same number of waves, same order of sums) and is
within the GEMM tolerance of the oracle everywhere."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import gemm as og
from oracle import quant as oq
from gpu_helpers import bf16_to_host, dev, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def decode_gemm_runs(M, N, K):
    """Whether fp8_block_gemm takes the decode kernel at these sizes (as the
    fused kernel, 16 waves up to 32 rows and 8 waves above): at most 64
    rows, N under 12288 past 32 rows, and the activation scales of the row
    fragments within the kernel's 32 KB of LDS."""
    mf = 1 if M <= 16 else (2 if M <= 32 else 4)
    return M <= 64 and (M <= 32 or N < 12288) and (K // 128) * mf * 16 * 4 <= 32 * 1024


def two_launch(xd, wq, ws):
    """fp8_act_quant_group then fp8_block_gemm (never the split-K variant)."""
    xq, xs = fb.act_quant_group(xd)
    y = torch.empty((xd.shape[0], wq.shape[0]), dtype=torch.bfloat16, device=xd.device)
    fb.fp8_block_gemm(xq, xs, wq, ws, y)
    return y


def check(x, w, what, bit_identical, tol_rows=None):
    """The fused kernel proper (no workspaces given, so M <= 64 always fuses)."""
    xd = to_dev_bf16(x)
    wq, ws = oq.weight_block_quant(w)
    wqd, wsd = to_dev(wq), to_dev(ws)
    y = torch.empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16, device=dev())
    fb.fp8_linear(xd, wqd, wsd, y)
    y2 = two_launch(xd, wqd, wsd)
    torch.cuda.synchronize()
    y, y2 = bf16_to_host(y), bf16_to_host(y2)
    if bit_identical:
        bad = np.argwhere(y != y2)
        assert bad.size == 0, f"{what}: {len(bad)} outputs differ from the two-launch path"
    xq, xs = oq.act_quant_group(x)
    rows = np.arange(x.shape[0]) if tol_rows is None else np.asarray(tol_rows)
    rep = og.tolerance_report(y[rows], og.block_gemm(xq[rows], xs[rows], wq, ws),
                              og.term_magnitude(xq[rows], xs[rows], wq, ws))
    say(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], (what, rep)


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 64])
@pytest.mark.parametrize("shape_index", range(4))
def test_fused_decode_llama(M, shape_index):
    x, w = synth.llama_inputs(shape_index, M, config=2)
    N, K = w.shape
    check(x, w, f"fused {synth.LLAMA_SHAPES[shape_index][0]} M={M}",
          bit_identical=decode_gemm_runs(M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 100, 256), (16, 300, 384), (31, 576, 18432),
                                   (40, 1000, 1280), (64, 24576, 1536), (7, 7168, 16384),
                                   (20, 7176, 512), (32, 14380, 256), (48, 4100, 384),
                                   (33, 14336, 640)])
def test_fused_decode_ragged(M, N, K):
    """Ragged shapes, including two 16-column slabs per workgroup at
    M = 17-64 (N = 7176, 14380, 4100, 14336, 24576), some with a last
    workgroup holding one slab and a last slab of 4-12 columns."""
    x = synth.dsv3_activations(M + K, M, K, N)
    w = synth.normal_bf16(N + K, (N, K), 0.02)
    check(x, w, f"fused {M}x{N}x{K}", bit_identical=decode_gemm_runs(M, N, K))


def test_fused_decode_edge_values():
    """Groups that are all zero, hold bf16 subnormals or reach bf16's
    largest values: the fused quantizer must take the general path exactly
    like the standalone one (bit-identical outputs on every row).  Rows 1
    and 2 hold bf16-subnormal groups: their scales (~2e-43, ~3e-41) make the
    promotion factor x_s * w_s fall below fp32's normal range (to 0 or to a
    subnormal with a few significant bits), so any fp32-promoting GEMM
    loses those outputs' precision while the fp64 oracle does not; those
    rows are left out of the oracle tolerance."""
    K = 512
    x = np.zeros((8, K), np.uint16)
    x[1, :128] = 0x0001                              # subnormal amax group
    x[2, 128:256] = np.arange(128, dtype=np.uint16) | 0x0040
    x[3, :] = synth.normal_bf16(1, (1, K))[0]
    x[4, 256] = 0x7F7F                                 # largest bf16
    x[5, 300] = 0x8000                                 # negative zero
    x[6, :] = 0x3F80
    w = synth.normal_bf16(2, (256, K), 0.02)
    check(x, w, "fused edges", bit_identical=True, tol_rows=[0, 3, 4, 5, 6, 7])


@pytest.mark.parametrize("M", [65, 300])
def test_linear_workspace_path(M):
    x, w = synth.llama_inputs(1, M, config=3)
    xd = to_dev_bf16(x)
    wq, ws = oq.weight_block_quant(w)
    wqd, wsd = to_dev(wq), to_dev(ws)
    K = x.shape[1]
    xq_ws = torch.empty((M, K), dtype=torch.uint8, device=dev())
    xs_ws = torch.empty((M, K // 128), dtype=torch.float32, device=dev())
    y = torch.empty((M, w.shape[0]), dtype=torch.bfloat16, device=dev())
    fb.fp8_linear(xd, wqd, wsd, y, xq_ws, xs_ws)
    y2 = two_launch(xd, wqd, wsd)
    torch.cuda.synchronize()
    oxq, oxs = oq.act_quant_group(x)
    assert np.array_equal(host(xq_ws), oxq)
    assert np.array_equal(host(xs_ws).view(np.uint32), oxs.view(np.uint32))
    assert np.array_equal(bf16_to_host(y), bf16_to_host(y2))
    with pytest.raises(ValueError):
        fb.fp8_linear(xd, wqd, wsd, y)


@pytest.mark.parametrize("M,N,K,fused", [(24, 4096, 4096, True), (32, 1536, 7168, True),
                                         (17, 14336, 4096, False), (48, 4096, 4096, False),
                                         (64, 1024, 4096, False), (40, 14336, 4096, False)])
def test_linear_with_workspaces_small_batch(M, N, K, fused):
    """fp8_linear with workspaces at M = 17-64: fused for 16 < M <= 32 with
    N * K <= 2^24, else the quantizer into the workspaces and the GEMM.
    Either way y equals the two-launch result bit for bit (the fused kernel
    sums in the decode kernel's order); the workspaces hold the oracle's
    codes and scales exactly when the two kernels ran and are untouched
    (still NaN-filled) when the fused kernel ran."""
    x = synth.llama_activations(M + N + K, M, K, 7)
    w = synth.normal_bf16(N + K, (N, K), 0.02)
    wq, ws = oq.weight_block_quant(w)
    xd, wqd, wsd = to_dev_bf16(x), to_dev(wq), to_dev(ws)
    xq_ws = torch.full((M, K), 0x7F, dtype=torch.uint8, device=dev())
    xs_ws = torch.full((M, K // 128), float("nan"), dtype=torch.float32, device=dev())
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_linear(xd, wqd, wsd, y, xq_ws, xs_ws)
    y2 = two_launch(xd, wqd, wsd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_host(y), bf16_to_host(y2))
    if fused:
        assert bool(torch.all(xq_ws == 0x7F)) and bool(torch.all(torch.isnan(xs_ws)))
    else:
        oxq, oxs = oq.act_quant_group(x)
        assert np.array_equal(host(xq_ws), oxq)
        assert np.array_equal(host(xs_ws).view(np.uint32), oxs.view(np.uint32))


@pytest.mark.parametrize("N,K", [(4096, 4096), (14336, 4096), (4096, 14336), (24576, 1536),
                                 (7168, 16384)])
def test_linear_picks_a_path_and_agrees(N, K):
    """fb.linear passes workspaces; the library fuses for N * K <= 2^25 and
    for wide N with K <= 8192 (several slabs per workgroup: 14336 x 4096,
    24576 x 1536): bit for bit the two-launch path at M = 16.  For
    4096 x 14336 and 7168 x 16384 the library plans a K split at M = 16, and
    fb.linear runs the quantizer then fp8_block_gemm_ws: bit for bit that
    pair of calls (the split itself is checked against the oracle in the
    GEMM tests)."""
    x = synth.llama_activations(N + K, 16, K, 7)
    w = synth.normal_bf16(N, (N, K), 0.02)
    wq, ws = oq.weight_block_quant(w)
    xd, wqd, wsd = to_dev_bf16(x), to_dev(wq), to_dev(ws)
    y = fb.linear(xd, wqd, wsd)
    need = fb.fp8_block_gemm_workspace_bytes(16, N, K)
    assert (need > 0) == ((N, K) in ((4096, 14336), (7168, 16384)))
    if need:
        xq, xs = fb.act_quant_group(xd)
        y2 = torch.empty_like(y)
        work = torch.empty(need, dtype=torch.uint8, device=xd.device)
        fb.fp8_block_gemm_ws(xq, xs, wqd, wsd, y2, work)
    else:
        y2 = two_launch(xd, wqd, wsd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_host(y), bf16_to_host(y2))
