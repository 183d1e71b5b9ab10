"""fp8_block_gemm_noalloc (the K-split GEMM on the library's own device
scratch, for callers that cannot allocate) against fp8_block_gemm_ws with a
caller workspace: the same kernels and plan, so the outputs must be equal
bit for bit.  Two calls in a row on the shared scratch, the second smaller,
then shapes that take the decode split and no split at all."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import gemm as og
from oracle import quant as oq
from gpu_helpers import bf16_to_host, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    x = synth.dsv3_activations(seed, M, K, seed + 1)
    w = synth.normal_bf16(seed + 2, (N, K), 0.01)
    xq, xs = oq.act_quant_group(x)
    wq, ws = oq.weight_block_quant(w)
    return xq, xs, wq, ws


def _both(xq, xs, wq, ws):
    M, K = xq.shape
    N = wq.shape[0]
    d = dev()
    a, b, c, e = to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws)
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    work = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device=d)
    y_ws = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    fb.fp8_block_gemm_ws(a, b, c, e, y_ws, work if need else None)
    y_na = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=d)
    fb.fp8_block_gemm_noalloc(a, b, c, e, y_na)
    torch.cuda.synchronize()
    return bf16_to_host(y_ws), bf16_to_host(y_na), need


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: DeepSeek-V3 q_a at M = 512 (split five ways, 15.7 MB of
    # scratch); second, smaller: 130 x 576 x 4096
    for M, N, K, seed in ((512, 1536, 7168, 1), (130, 576, 4096, 2)):
        xq, xs, wq, ws = _operands(M, N, K, seed)
        y_ws, y_na, need = _both(xq, xs, wq, ws)
        say("noalloc", M, N, K, "split workspace", need)
        assert need > 0 and need <= fb.SCRATCH_BYTES
        bad = np.argwhere(y_ws != y_na)
        assert bad.size == 0, f"{M}x{N}x{K}: {len(bad)} outputs differ, first {bad[:3].tolist()}"
        rep = og.tolerance_report(y_na, og.block_gemm(xq, xs, wq, ws), og.term_magnitude(xq, xs, wq, ws))
        assert rep["ok"], rep


def test_noalloc_decode_split_and_unsplit():
    # decode split (M = 12, long K), one padded row tile split over K
    # (M = 48, long K), then a grid that needs no split
    for M, N, K, seed in ((12, 4096, 14336, 3), (48, 4096, 14336, 6), (300, 2048, 1024, 4)):
        xq, xs, wq, ws = _operands(M, N, K, seed)
        y_ws, y_na, need = _both(xq, xs, wq, ws)
        say("noalloc", M, N, K, "split workspace", need)
        assert np.array_equal(y_ws, y_na), f"{M}x{N}x{K}"
        if need == 0:
            y_plain = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
            fb.fp8_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), y_plain)
            torch.cuda.synchronize()
            assert np.array_equal(bf16_to_host(y_plain), y_na)


@pytest.mark.parametrize("M,N,K", [(8192, 7168, 16384), (512, 7168, 16384)])
def test_noalloc_stream_k_shape_runs_unsplit(M, N, K):
    """Stream-K shapes (a partly empty last round of 256x256 tiles, and a
    small grid with long K) need far more than the scratch:
    fp8_block_gemm_noalloc runs them as fp8_block_gemm, bit for bit."""
    assert fb.fp8_block_gemm_workspace_bytes(M, N, K) > fb.SCRATCH_BYTES
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(5)
    xq = torch.randint(0, 0x7e, (M, K), generator=g, device=d, dtype=torch.uint8)
    wq = torch.randint(0, 0x7e, (N, K), generator=g, device=d, dtype=torch.uint8)
    xs = torch.rand((M, K // 128), generator=g, device=d) + 0.5
    ws = torch.rand((-(-N // 128), K // 128), generator=g, device=d) + 0.5
    y_plain = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    y_na = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    fb.fp8_block_gemm(xq, xs, wq, ws, y_plain)
    fb.fp8_block_gemm_noalloc(xq, xs, wq, ws, y_na)
    torch.cuda.synchronize()
    assert torch.equal(y_plain.view(torch.int16), y_na.view(torch.int16))
