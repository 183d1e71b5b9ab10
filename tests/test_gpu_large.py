"""GPU parity at the large end of the size range, through the C ABI: K = 2^20
(the tiles' byte offsets into A and B reach 2^28, the workspace split runs
2^13 K blocks), the decode kernel's largest K and the first K past it,
2^20 + 77 rows (a 4097-tile grid with a ragged last tile), an activation
quantizer row of 2^20 values, a weight quantizer with 2^18-long rows and a
partial block row, and a grouped GEMM over 300 experts.  GEMM operands are
E4M3 codes distributed like quantized data, made on the device (bf16 inputs
for the quantizers); the oracle checks sampled rows and column blocks
(every output where it is cheap) to the same tolerance as the other GEMM
tests, and the quantizers bit for bit."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import gemm as og
from oracle import quant as oq
from gpu_helpers import assert_codes_equal, bf16_to_host, dev, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _codes(g, shape):
    """E4M3 codes distributed like quantized data: N(0, 64^2) values,
    clamped to +-448 and cast to E4M3 on the device (test input only; any
    finite code is a valid operand and the oracle decodes the codes
    itself)."""
    d = dev()
    v = torch.randn(shape, generator=g, device=d).mul_(64.0).clamp_(-448.0, 448.0)
    return v.to(torch.float8_e4m3fn).view(torch.uint8)


def _operands(seed, M, N, K):
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(seed)
    xq = _codes(g, (M, K))
    wq = _codes(g, (N, K))
    xs = torch.rand((M, K // 128), generator=g, device=d) + 0.5
    ws = torch.rand((-(-N // 128), K // 128), generator=g, device=d) + 0.5
    return xq, xs, wq, ws


def _check_sample(y, xq, xs, wq, ws, rows, c0, c1, what):
    """Oracle on rows `rows` x columns [c0, c1) (inside one 128-column block)."""
    assert c0 // 128 == (c1 - 1) // 128
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=y.device)
    xq_h, xs_h = host(xq.index_select(0, idx)), host(xs.index_select(0, idx))
    wq_h, ws_h = host(wq[c0:c1]), host(ws[c0 // 128:c0 // 128 + 1])
    y_hat = og.block_gemm(xq_h, xs_h, wq_h, ws_h)
    S = og.term_magnitude(xq_h, xs_h, wq_h, ws_h)
    got = bf16_to_host(y.index_select(0, idx)[:, c0:c1].contiguous())
    rep = og.tolerance_report(got, y_hat, S)
    say(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], (what, rep)


def test_gemm_k_two_to_the_20():
    """M = 520, N = 512, K = 2^20: the tiled kernel (two K groups per
    workgroup) through fp8_block_gemm, and the K split over workgroups
    through fp8_block_gemm_ws; rows across the three row tiles, the last
    column block."""
    M, N, K = 520, 512, 1 << 20
    xq, xs, wq, ws = _operands(101, M, N, K)
    d = dev()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    fb.fp8_block_gemm(xq, xs, wq, ws, y)
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
    say("K = 2^20 workspace bytes", need)
    assert need > 0
    work = torch.empty(need, dtype=torch.uint8, device=d)
    y2 = torch.empty_like(y)
    fb.fp8_block_gemm_ws(xq, xs, wq, ws, y2, work)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 256, 511, 519])
    _check_sample(y, xq, xs, wq, ws, rows, 448, 512, "K=2^20 plain")
    _check_sample(y2, xq, xs, wq, ws, rows, 448, 512, "K=2^20 split")


@pytest.mark.parametrize("K", [65536, 65536 + 128])
def test_gemm_decode_largest_k(K):
    """M = 16: K = 65536 is the decode kernel's largest (its activation
    scales, 16 rows x 512 blocks x 4 bytes, fill 32 KB of LDS); one block
    more goes to the tiled kernel.  Every output checked."""
    M, N = 16, 384
    xq, xs, wq, ws = _operands(K + 7, M, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm(xq, xs, wq, ws, y)
    torch.cuda.synchronize()
    for nb in range(N // 128):
        _check_sample(y, xq, xs, wq, ws, np.arange(M), 128 * nb, 128 * nb + 128,
                      f"decode K={K} block {nb}")


def test_gemm_two_to_the_20_rows():
    """M = 2^20 + 77, N = 256, K = 256: 4097 tiles of 256x256, the last
    with 77 rows; sampled rows, both column blocks."""
    M, N, K = (1 << 20) + 77, 256, 256
    xq, xs, wq, ws = _operands(303, M, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm(xq, xs, wq, ws, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 78, M - 77, M - 1],
                                     rng.integers(0, M, 40)]))
    _check_sample(y, xq, xs, wq, ws, rows, 0, 128, "M=2^20+77 block 0")
    _check_sample(y, xq, xs, wq, ws, rows, 128, 256, "M=2^20+77 block 1")


def test_act_quant_row_of_two_to_the_20():
    """Four rows of 2^20 values (8192 groups each), bit-exact codes and
    scales against the oracle."""
    x = synth.dsv3_activations(404, 4, 1 << 20, 405)
    xq, xs = fb.act_quant_group(to_dev_bf16(x))
    torch.cuda.synchronize()
    wq_, ws_ = oq.act_quant_group(x)
    assert_codes_equal(host(xq), host(xs), wq_, ws_, "act quant K=2^20")


def test_weight_quant_long_rows_partial_block_row():
    """N = 130 (a full and a 2-row block row), K = 2^18: codes and block
    scales bit-exact."""
    w = synth.normal_bf16(505, (130, 1 << 18), 0.01)
    wq, ws = fb.weight_block_quant(to_dev_bf16(w))
    torch.cuda.synchronize()
    oq_, os_ = oq.weight_block_quant(w)
    assert_codes_equal(host(wq), host(ws), oq_, os_, "weight quant K=2^18")


def test_grouped_gemm_300_experts():
    """300 experts with loads 0..40 rows (many empty, ragged tiles
    everywhere), N = 256, K = 256: every row against the oracle."""
    E, N, K = 300, 256, 256
    rng = np.random.default_rng(606)
    loads = rng.integers(0, 41, E)
    loads[rng.choice(E, 60, replace=False)] = 0
    off = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    total = int(off[-1])
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(607)
    xq = _codes(g, (total, K))
    wq = _codes(g, (E, N, K))
    xs = torch.rand((total, K // 128), generator=g, device=d) + 0.5
    ws = torch.rand((E, N // 128, K // 128), generator=g, device=d) + 0.5
    y = torch.full((total, N), float("nan"), dtype=torch.bfloat16, device=d)
    fb.fp8_grouped_block_gemm(xq, xs, wq, ws, to_dev(off), y)
    torch.cuda.synchronize()
    xq_h, xs_h, wq_h, ws_h = host(xq), host(xs), host(wq), host(ws)
    y_hat = og.grouped_block_gemm(xq_h, xs_h, wq_h, ws_h, off)
    S = og.grouped_term_magnitude(xq_h, xs_h, wq_h, ws_h, off)
    rep = og.tolerance_report(bf16_to_host(y), y_hat, S)
    say("300 experts", total, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], rep
