"""The entry points under HIP graph capture: they allocate nothing, never
synchronize and record only kernel launches, so a captured layer replays to
the same bits as the eager calls.  Each graph is replayed several times
with the program's own eager work in between, and every replay is checked
against the eager result (bit for bit: the same kernels run in the same
order)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from gpu_helpers import dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _replay_and_check(step, outs, ref, other):
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()                                  # warm on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for r in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outs, ref):
            assert np.array_equal(_bits(o), want), f"replay {r} differs from the eager result"
        other()                                 # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [16, 24, 48, 300])
def test_linear_layer_graph(M):
    """fp8_act_quant_group + fp8_block_gemm (prefill, and M = 48: the
    quantizer and the 8-wave decode GEMM) or the fused decode kernel
    (M = 16, 24) for two projections, captured and replayed."""
    d = dev()
    shapes = [(1024, 2048), (576, 4096)]
    xs = [to_dev_bf16(synth.dsv3_activations(7 + K, M, K, 3)) for (_, K) in shapes]
    ws = [fb.weight_block_quant(to_dev_bf16(synth.normal_bf16(N + K, (N, K), 0.02))) for (N, K) in shapes]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=d) for (N, _) in shapes]
    ws_q = [torch.empty((M, K), dtype=torch.uint8, device=d) for (_, K) in shapes]
    ws_s = [torch.empty((M, K // 128), dtype=torch.float32, device=d) for (_, K) in shapes]

    def step():
        for x, (wq, wsc), y, xq, xsc in zip(xs, ws, ys, ws_q, ws_s):
            fb.fp8_linear(x, wq, wsc, y, xq, xsc)
    step()
    torch.cuda.synchronize()
    ref = [_bits(y) for y in ys]
    junk = torch.randn((M, 2048), device=d).to(torch.bfloat16)
    _replay_and_check(step, ys, ref, lambda: fb.act_quant_group(junk))


def test_moe_pieces_graph():
    """SwiGLU + quantizer and the grouped GEMM with device offsets."""
    d = dev()
    offsets = np.array([0, 40, 40, 300, 301, 512], np.int32)
    M, I, N = 512, 256, 512                      # per-expert scale slices stay 16-byte aligned
    gu = to_dev_bf16(synth.moe_gate_up_output(9, M, I))
    wq = torch.empty((5, N, I), dtype=torch.uint8, device=d)
    wsc = torch.empty((5, N // 128, I // 128), dtype=torch.float32, device=d)
    for e in range(5):
        fb.fp8_weight_block_quant(to_dev_bf16(synth.normal_bf16(e + 1, (N, I), 0.01)), wq[e], wsc[e])
    off = torch.from_numpy(offsets).to(d)
    xq = torch.empty((M, I), dtype=torch.uint8, device=d)
    xs = torch.empty((M, I // 128), dtype=torch.float32, device=d)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)

    def step():
        fb.fp8_swiglu_act_quant(gu, xq, xs)
        fb.fp8_grouped_block_gemm(xq, xs, wq, wsc, off, y)
    step()
    torch.cuda.synchronize()
    _replay_and_check(step, [y], [_bits(y)], lambda: fb.swiglu_act_quant(gu))


@pytest.mark.parametrize("M,N,K", [(512, 1536, 7168), (16, 4096, 14336)])
def test_split_k_gemm_graph(M, N, K):
    """The K split over workgroups (two kernels through a workspace, no
    memset) captured and replayed, for the tiled split (DeepSeek-V3 q_a at
    M = 512) and the decode split (Llama down at M = 16): every replay
    equals the eager bits."""
    d = dev()
    x = to_dev_bf16(synth.dsv3_activations(21, M, K, 22))
    wq, wsc = fb.weight_block_quant(to_dev_bf16(synth.normal_bf16(23, (N, K), 0.01)))
    xq, xsc = fb.act_quant_group(x)
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    assert need > 0
    work = torch.empty(need, dtype=torch.uint8, device=d)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)

    def step():
        fb.fp8_block_gemm_ws(xq, xsc, wq, wsc, y, work)
    step()
    torch.cuda.synchronize()
    ref = [_bits(y)]
    junk = torch.randn((M, K), device=d).to(torch.bfloat16)

    def other():
        jq, js = fb.act_quant_group(junk)
        fb.fp8_block_gemm_ws(jq, js, wq, wsc, torch.empty_like(y), work)
    _replay_and_check(step, [y], ref, other)


def test_stream_k_gemm_graph():
    """The stream-K tail of a partly empty last round (8192 x 7168 x 16384:
    3.5 rounds of 256x256 tiles; the GEMM kernel with its extra range
    workgroups, then the reduction) captured and replayed: every replay
    equals the eager bits."""
    d = dev()
    M, N, K = 8192, 7168, 16384
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    assert need > 0
    g = torch.Generator(device=d)
    g.manual_seed(31)
    xq = torch.randint(0, 0x7e, (M, K), generator=g, device=d, dtype=torch.uint8)
    wq = torch.randint(0, 0x7e, (N, K), generator=g, device=d, dtype=torch.uint8)
    xs = torch.rand((M, K // 128), generator=g, device=d) + 0.5
    ws = torch.rand((N // 128, K // 128), generator=g, device=d) + 0.5
    work = torch.empty(need, dtype=torch.uint8, device=d)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)

    def step():
        fb.fp8_block_gemm_ws(xq, xs, wq, ws, y, work)
    step()
    torch.cuda.synchronize()
    ref = [_bits(y)]
    xq2 = torch.randint(0, 0x7e, (M, K), generator=g, device=d, dtype=torch.uint8)

    def other():
        fb.fp8_block_gemm_ws(xq2, xs, wq, ws, torch.empty_like(y), work)
    _replay_and_check(step, [y], ref, other)
