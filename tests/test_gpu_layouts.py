"""GPU parity of the batched expert layout and of row-wise ("fp8r") scales
against the CPU oracle.

Batched GEMM: to the block-scaled GEMM's tolerance, rows past each expert's
count untouched, and bit-identical to the grouped GEMM on the same rows
(same tiles).  Row-wise quantizer: codes and scales bit-exact (including
zero, subnormal and extreme rows).  Row-wise GEMM: bit-exact on an
exact-arithmetic pin, otherwise the same tolerance, in every configuration
(decode, 128x128, 256x256)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import layouts as olay
from oracle import quant as oq
from gpu_helpers import bf16_to_host, dev, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def check_tol(y_bits, y_hat, S, what):
    rep = og.tolerance_report(y_bits, y_hat, S)
    say(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], (what, rep)


# ----------------------------------------------------------------------------
# batched experts

def _batched_case(E, C, N, K, counts, seed):
    x = synth.dsv3_activations(seed, E * C, K, seed + 1)
    xq, xs = oq.act_quant_group(x)
    NB = -(-N // 128)
    wq = np.empty((E, N, K), np.uint8); ws = np.empty((E, NB, K // 128), np.float32)
    for e in range(E):
        wq[e], ws[e] = oq.weight_block_quant(synth.normal_bf16(seed + 2 + e, (N, K), 0.01))
    return xq.reshape(E, C, K), xs.reshape(E, C, K // 128), wq, ws, np.asarray(counts, np.int32)


@pytest.mark.parametrize("E,C,N,K,counts", [
    (4, 64, 256, 512, [0, 1, 64, 33]),
    (3, 300, 576, 384, [300, 17, 299]),
    (5, 256, 128, 1024, [256, 0, 255, 1, 400]),      # 400 clamps to 256
    (2, 40, 4096, 256, [-5, 40]),                    # negative count = empty
    (8, 512, 2048, 7168, [512, 100, 0, 511, 257, 256, 1, 300]),
])
def test_batched_matches_oracle(E, C, N, K, counts):
    xq, xs, wq, ws, cnt = _batched_case(E, C, N, K, counts, E + C + N)
    y = torch.full((E, C, N), 7.0, dtype=torch.bfloat16, device=dev())
    fb.fp8_batched_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(cnt), y)
    torch.cuda.synchronize()
    yb = bf16_to_host(y.reshape(E * C, N)).reshape(E, C, N)
    want = olay.batched_block_gemm(xq, xs, wq, ws, cnt)
    S = olay.batched_term_magnitude(xq, xs, wq, ws, cnt)
    used = np.clip(cnt, 0, C)
    rows = [(e, r) for e in range(E) for r in range(used[e])]
    if rows:
        ee, rr = zip(*rows)
        check_tol(yb[ee, rr], want[ee, rr], S[ee, rr], f"batched E={E} C={C}")
    for e in range(E):
        untouched = y[e, used[e]:].float().cpu().numpy()
        assert np.all(untouched == 7.0), f"expert {e}: rows past the count were written"
    # the grouped GEMM on the same rows runs the same tiles: identical bits
    off = np.concatenate([[0], np.cumsum(used)]).astype(np.int32)
    if off[-1]:
        pq = np.concatenate([xq[e, :used[e]] for e in range(E)])
        ps = np.concatenate([xs[e, :used[e]] for e in range(E)])
        yg = bf16_to_host(fb.grouped_block_gemm(to_dev(pq), to_dev(ps), to_dev(wq), to_dev(ws), to_dev(off)))
        torch.cuda.synchronize()
        for e in range(E):
            assert np.array_equal(yb[e, :used[e]], yg[off[e]:off[e + 1]]), f"expert {e} differs from grouped"


# ----------------------------------------------------------------------------
# row-wise quantizer

def gpu_rowwise_quant(bits):
    q, s = fb.rowwise_quant(to_dev_bf16(bits))
    torch.cuda.synchronize()
    return host(q), host(s)


def assert_rowwise_equal(got, want, what):
    gq, gs = got
    wq, ws = want
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32)), f"{what}: scales differ"
    bad = np.argwhere(gq != wq)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("R,K", [(1, 128), (3, 384), (17, 4096), (64, 14336), (300, 7168),
                                 (4096, 4096), (5, 18432), (1000, 256), (2, 32768),
                                 (3, 33024), (2, 40960)])
def test_rowwise_quant(R, K):
    x = synth.dsv3_activations(R * 3 + K, R, K, R + 5)
    say("rowwise quant", R, K)
    assert_rowwise_equal(gpu_rowwise_quant(x), olay.rowwise_quant(x), f"{R}x{K}")


def test_rowwise_quant_edge_rows():
    rng = np.random.default_rng(4)
    K = 512
    rows = []
    for amax in [0x0000, 0x0001, 0x0080, 0x1F80, 0x2000, 0x3F80, 0x43E0, 0x7F7F, 0x7F00]:
        r = (rng.integers(0, max(amax, 1), K) | (rng.integers(0, 2, K) << 15)).astype(np.uint16)
        r[rng.integers(0, K)] = amax | 0x8000
        rows.append(r)
    x = np.stack(rows)
    assert_rowwise_equal(gpu_rowwise_quant(x), olay.rowwise_quant(x), "edge rows")


# ----------------------------------------------------------------------------
# row-wise GEMM

def gpu_rowwise_gemm(xq, xs, wq, ws):
    y = fb.rowwise_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    return bf16_to_host(y)


@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (1, 300, 512), (64, 192, 1024),
                                   (130, 576, 4096), (2048, 4096, 512), (257, 1000, 640),
                                   (300, 2000, 2048), (1, 14380, 256), (7, 7176, 384),
                                   (16, 14380, 512), (32, 14380, 256), (24, 7176, 384),
                                   (64, 7176, 384), (48, 4100, 768)])
def test_rowwise_gemm_exact_integer_operands(M, N, K):
    """Integer codes with power-of-two row scales: exact, bit for bit.
    M = 24-64 with N = 14380, 7176 and 4100 packs four or two 16-column
    slabs per decode workgroup (ragged last slabs and groups)."""
    rng = np.random.default_rng(M + N + K)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    xs = np.exp2(rng.integers(-2, 3, M)).astype(np.float32)
    ws = np.exp2(rng.integers(-2, 3, N)).astype(np.float32)
    y = gpu_rowwise_gemm(xq, xs, wq, ws)
    want = og.bf16_rne_bits(olay.rowwise_gemm(xq, xs, wq, ws))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (15, 100, 256), (17, 576, 384),
                                   (130, 300, 1024), (257, 1000, 512), (16, 4096, 4096),
                                   (64, 1024, 2048), (520, 3000, 1280), (3, 576, 18432)])
def test_rowwise_gemm_ragged(M, N, K):
    x = synth.dsv3_activations(M + 11 * K, M, K, N)
    w = synth.normal_bf16(N + 13 * K, (N, K), 0.02)
    xq, xs = olay.rowwise_quant(x)
    wq, ws = olay.rowwise_quant(w)
    check_tol(gpu_rowwise_gemm(xq, xs, wq, ws), olay.rowwise_gemm(xq, xs, wq, ws),
              olay.rowwise_term_magnitude(xq, xs, wq, ws), f"rowwise {M}x{N}x{K}")


@pytest.mark.parametrize("shape_index", range(4))
@pytest.mark.parametrize("M", [1, 16, 32, 64, 4096])
def test_linear_rowwise_llama(shape_index, M):
    x, w = synth.llama_inputs(shape_index, M, config=3 if M > 16 else 2)
    wq_d, ws_d = fb.rowwise_quant(to_dev_bf16(w))
    y = bf16_to_host(fb.linear_rowwise(to_dev_bf16(x), wq_d, ws_d))
    torch.cuda.synchronize()
    wq, ws = olay.rowwise_quant(w)
    assert np.array_equal(host(wq_d), wq) and np.array_equal(host(ws_d).view(np.uint32), ws.view(np.uint32))
    rows = np.arange(M) if M <= 64 else np.sort(np.concatenate(
        [[0, M - 1], np.random.default_rng(shape_index).choice(np.arange(1, M - 1), 62, replace=False)]))
    xq, xs = olay.rowwise_quant(x[rows])
    check_tol(y[rows], olay.rowwise_gemm(xq, xs, wq, ws), olay.rowwise_term_magnitude(xq, xs, wq, ws),
              f"rowwise linear {synth.LLAMA_SHAPES[shape_index][0]} M={M}")
