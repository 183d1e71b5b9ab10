"""GPU parity of the power-of-two-scale (E8M0 byte) path -- both quantizers,
the GEMM and its grouped variant -- against the CPU oracle.

Quantizers: codes and scale bytes bit-exact, on ragged shapes, the
workloads' shapes, the format's edge cases and the whole (x, amax) bf16
domain (chunk digests written by tests/golden/make_exhaustive_digests.py
from the oracle).  GEMMs: the same tolerance as with fp32 scales (relative
Frobenius error <= 2e-3, per element <= 1e-2 * max(|y_hat|, 2^-6 * S)), and
bit-exact on exact-arithmetic pins."""
import hashlib
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import ue8m0 as ou
from gpu_helpers import (assert_codes_equal, bf16_to_host, dev, gpu_act_quant_ue8m0,
                         gpu_weight_quant_ue8m0, host, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _digests():
    out = {}
    for line in open(os.path.join(GOLDEN, "exhaustive_digests.txt")):
        if line.startswith("#") or not line.strip():
            continue
        kind, c, lo, hi, h = line.split()
        out[(kind, int(c))] = (int(lo, 16), int(hi, 16), h)
    return out


DIGESTS = _digests()
NCHUNKS = 1 + max([c for k, c in DIGESTS if k == "act_ue8m0"], default=-1)


def _digest(q, s):
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(q).tobytes())
    h.update(np.ascontiguousarray(s).tobytes())
    return h.hexdigest()


# ----------------------------------------------------------------------------
# quantizers

@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (17, 512), (5, 1536), (33, 2048),
                                 (4, 14336), (16, 4096), (127, 7168), (131, 128)])
def test_act_quant_ue8m0_ragged(M, K):
    x = synth.dsv3_activations(M * 7 + K, M, K, M + 3)
    say("act_quant_ue8m0", M, K)
    assert_codes_equal(*gpu_act_quant_ue8m0(x), *ou.act_quant_group_ue8m0(x), f"{M}x{K}")


@pytest.mark.parametrize("shape_index", range(4))
@pytest.mark.parametrize("M", [1, 16, 4096])
def test_act_quant_ue8m0_llama(shape_index, M):
    x = synth.llama_x(shape_index, M, config=3)
    say("act_quant_ue8m0 llama", shape_index, M)
    assert_codes_equal(*gpu_act_quant_ue8m0(x), *ou.act_quant_group_ue8m0(x), f"llama {M}")


def _edge_groups():
    """Groups whose amax sits on the format's edges: 448 * 2^j and its bf16
    neighbours, bf16's smallest subnormal and largest finite value, zero."""
    amaxes = [0x0000, 0x0001, 0x0380, 0x007F, 0x0080, 0x7F7F, 0x7F00, 0x3FE0, 0x3FE1, 0x3FDF]
    for j in (-120, -20, 0, 7, 100, 119):
        edge = np.array([448.0 * 2.0 ** j], np.float32).view(np.uint32)[0] >> 16
        amaxes += [int(edge) - 1, int(edge), int(edge) + 1]
    rng = np.random.default_rng(3)
    rows = []
    for a in amaxes:
        g = (rng.integers(0, max(a, 1), 128) | (rng.integers(0, 2, 128) << 15)).astype(np.uint16)
        g[rng.integers(0, 128)] = a | (0x8000 if rng.integers(0, 2) else 0)
        rows.append(g)
    return np.stack(rows)


def test_act_quant_ue8m0_edges():
    x = _edge_groups()
    q, s = gpu_act_quant_ue8m0(x)
    assert_codes_equal(q, s, *ou.act_quant_group_ue8m0(x), "edges")
    assert s.max() <= 254


def test_weight_quant_ue8m0_edges():
    g = _edge_groups()                       # each group becomes one 128x128 block
    w = np.concatenate([np.tile(r, (128, 1)) for r in g])
    assert_codes_equal(*gpu_weight_quant_ue8m0(w), *ou.weight_block_quant_ue8m0(w), "W edges")


@pytest.mark.parametrize("N,K", [(1, 128), (64, 256), (100, 384), (129, 128), (576, 7168),
                                 (300, 1024), (1000, 640)])
def test_weight_quant_ue8m0_ragged(N, K):
    w = synth.normal_bf16(N * 31 + K, (N, K), 0.01)
    say("weight_quant_ue8m0", N, K)
    assert_codes_equal(*gpu_weight_quant_ue8m0(w), *ou.weight_block_quant_ue8m0(w), f"W {N}x{K}")


@pytest.mark.parametrize("which", ["llama_qo", "llama_down", "dsv3_q_b"])
def test_weight_quant_ue8m0_workloads(which):
    if which == "llama_qo":
        w = synth.llama_weight(0)
    elif which == "llama_down":
        w = synth.llama_weight(3)
    else:
        _, w = synth.dsv3_inputs(1, 1)
    say("weight_quant_ue8m0", which, w.shape)
    assert_codes_equal(*gpu_weight_quant_ue8m0(w), *ou.weight_block_quant_ue8m0(w), which)


@pytest.mark.parametrize("chunk", range(NCHUNKS))
def test_act_quant_ue8m0_exhaustive(chunk):
    lo, hi, want = DIGESTS[("act_ue8m0", chunk)]
    x = synth.exhaustive_act_chunk(lo, hi)
    say(f"act_ue8m0 exhaustive chunk {chunk} amax [{lo:#x},{hi:#x}) groups {x.shape[0]}")
    q, s = gpu_act_quant_ue8m0(x)
    if _digest(q, s) != want:
        assert_codes_equal(q, s, *ou.act_quant_group_ue8m0(x), f"exhaustive act_ue8m0 chunk {chunk}")
        pytest.fail("digest differs although codes match: regenerate the digests")


@pytest.mark.parametrize("chunk", range(NCHUNKS))
def test_weight_quant_ue8m0_exhaustive(chunk):
    lo, hi, want = DIGESTS[("weight_ue8m0", chunk)]
    w = synth.exhaustive_weight_chunk(lo, hi)
    say(f"weight_ue8m0 exhaustive chunk {chunk} amax [{lo:#x},{hi:#x}) rows {w.shape[0]}")
    q, s = gpu_weight_quant_ue8m0(w)
    if _digest(q, s) != want:
        assert_codes_equal(q, s, *ou.weight_block_quant_ue8m0(w), f"exhaustive weight_ue8m0 chunk {chunk}")
        pytest.fail("digest differs although codes match: regenerate the digests")


# ----------------------------------------------------------------------------
# GEMM

def gpu_gemm_ue8m0(xq, xe, wq, we):
    y = fb.block_gemm(to_dev(xq), to_dev(xe), to_dev(wq), to_dev(we))
    torch.cuda.synchronize()
    return bf16_to_host(y)


def check_tol(y_bits, y_hat, S, what):
    rep = og.tolerance_report(y_bits, y_hat, S)
    say(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["ok"], (what, rep)
    return rep


def operands(x_bits, w_bits):
    xq, xe = ou.act_quant_group_ue8m0(x_bits)
    wq, we = ou.weight_block_quant_ue8m0(w_bits)
    return xq, xe, wq, we


@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (64, 192, 1024), (130, 576, 4096),
                                   (1, 300, 512), (300, 520, 768), (1024, 1024, 1280),
                                   (257, 1000, 640), (200, 300, 384), (1024, 1024, 1152),
                                   (1, 14380, 256), (16, 7176, 512), (16, 14336, 1024),
                                   (40, 12300, 256), (64, 14336, 384), (48, 8192, 256),
                                   (24, 14336, 256), (32, 7176, 384), (20, 4100, 512),
                                   (40, 4100, 384), (64, 8200, 256)])
def test_gemm_ue8m0_exact_integer_operands(M, N, K):
    """|codes| <= 8 integers, scale bytes 126..128 (x) and 127..128 (W):
    every product and partial sum is exact in fp32, so y must equal
    bf16_RNE(exact).  Grids of at most 256 128x128 tiles split K over two
    wave groups when the K-block count is even (130x576x4096, 300x520x768,
    1024x1024x1280) and run unsplit when it is odd (the next three); the
    next three are decode shapes wide enough for two 16-column slabs per
    workgroup (a partly empty last workgroup, a ragged last slab); at
    M = 33-64, N >= 12288 takes the 128x128 tiles (40x12300x256: two wave
    groups, 64x14336x384: an odd K-block count, unsplit) and 48x8192 the
    decode kernel.  The last five run the decode kernel past 16 rows (8
    waves): four slabs per workgroup at 24 rows, two at 32, 20 and 40 rows
    (ragged last slabs, partly empty last workgroups), one at 64 rows."""
    rng = np.random.default_rng(M + N + K)
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xe = rng.integers(126, 129, (M, KB)).astype(np.uint8)
    we = rng.integers(127, 129, (NB, KB)).astype(np.uint8)
    y = gpu_gemm_ue8m0(xq, xe, wq, we)
    want = og.bf16_rne_bits(ou.block_gemm_ue8m0(xq, xe, wq, we))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(8, 256, 1536), (33, 200, 1280), (300, 384, 1024)])
def test_gemm_ue8m0_scale_indexing(M, N, K):
    """All codes 1.0; x byte[m,kb] = 127 + (kb+m) % KB, W byte[nb,kb] =
    107 + KB*((kb+nb)%2): each output is 128 * a sum of distinct powers of
    two, exact in fp32, so a wrong or transposed scale index changes its
    bits (also the per-row scale operand of each MFMA fragment)."""
    KB, NB = K // 128, -(-N // 128)
    xq = np.full((M, K), 0x38, np.uint8); wq = np.full((N, K), 0x38, np.uint8)
    xe = np.array([[127 + (kb + m) % KB for kb in range(KB)] for m in range(M)], np.uint8)
    we = np.array([[107 + KB * ((kb + nb) % 2) for kb in range(KB)] for nb in range(NB)], np.uint8)
    y = gpu_gemm_ue8m0(xq, xe, wq, we)
    want = og.bf16_rne_bits(ou.block_gemm_ue8m0(xq, xe, wq, we))
    assert np.array_equal(y, want)


def test_gemm_ue8m0_extreme_scales():
    """Scale bytes at both ends of E8M0 (0 = 2^-127 and 254 = 2^127) on
    one operand, balanced by the other so that each product stays in
    range: K block 0 pairs x 2^-127 with W 2^127, block 1 the reverse, block
    2 gives row m the factor 2^(m % 20 - 10).  Integer codes: exact."""
    M, N, K = 20, 130, 384
    rng = np.random.default_rng(9)
    xq = oe.encode(rng.integers(-4, 5, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-4, 5, (N, K)).astype(np.float32))
    xe = np.zeros((M, 3), np.uint8)
    xe[:, 0] = 0; xe[:, 1] = 254; xe[:, 2] = 117 + np.arange(M) % 20
    we = np.zeros((2, 3), np.uint8)
    we[:, 0] = 254; we[:, 1] = 0; we[:, 2] = 127
    y = gpu_gemm_ue8m0(xq, xe, wq, we)
    want = og.bf16_rne_bits(ou.block_gemm_ue8m0(xq, xe, wq, we))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (15, 100, 256), (17, 576, 384),
                                   (130, 300, 1024), (257, 1000, 512), (16, 4096, 4096),
                                   (200, 129, 7168), (129, 257, 128), (33, 4096, 4096),
                                   (40, 300, 512), (64, 1024, 2048), (65, 256, 256),
                                   (2, 24576, 1536), (3, 576, 18432), (520, 3000, 1280),
                                   (32, 14336, 4096), (48, 7168, 16384)])
def test_gemm_ue8m0_ragged(M, N, K):
    x = synth.dsv3_activations(M + 11 * K, M, K, N)
    w = synth.normal_bf16(N + 13 * K, (N, K), 0.02)
    xq, xe, wq, we = operands(x, w)
    check_tol(gpu_gemm_ue8m0(xq, xe, wq, we), ou.block_gemm_ue8m0(xq, xe, wq, we),
              ou.term_magnitude_ue8m0(xq, xe, wq, we), f"ue8m0 ragged {M}x{N}x{K}")


def _sampled_rows_check(x, w, rows, what):
    """The GPU quantizes all of x; the oracle quantizes the sampled rows
    itself (row-local), the GPU's codes and scale bytes there must equal
    it, and the GEMM rows are checked against the oracle's GEMM of the
    oracle's operands."""
    xq, xe = fb.act_quant_group(to_dev_bf16(x), "ue8m0")
    wq, we = ou.weight_block_quant_ue8m0(w)
    y = bf16_to_host(fb.block_gemm(xq, xe, to_dev(wq), to_dev(we)))
    torch.cuda.synchronize()
    oxq, oxe = ou.act_quant_group_ue8m0(x[rows])
    assert_codes_equal(host(xq)[rows], host(xe)[rows], oxq, oxe, what)
    want = ou.block_gemm_ue8m0(oxq, oxe, wq, we)
    return check_tol(y[rows], want, ou.term_magnitude_ue8m0(oxq, oxe, wq, we), what)


@pytest.mark.parametrize("shape_index", range(4))
@pytest.mark.parametrize("M", [1, 16, 4096])
def test_gemm_ue8m0_llama(shape_index, M):
    x, w = synth.llama_inputs(shape_index, M, config=3 if M > 16 else 2)
    rows = np.arange(M) if M <= 16 else np.sort(np.concatenate(
        [[0, M - 1], np.random.default_rng(shape_index).choice(np.arange(1, M - 1), 62, replace=False)]))
    _sampled_rows_check(x, w, rows, f"ue8m0 llama {synth.LLAMA_SHAPES[shape_index][0]} M={M}")


@pytest.mark.parametrize("shape_index", range(6))
def test_gemm_ue8m0_dsv3_sampled(shape_index):
    M = 2048
    x, w = synth.dsv3_inputs(shape_index, M)
    rows = np.sort(np.concatenate([[0, M - 1], np.random.default_rng(shape_index).choice(
        np.arange(1, M - 1), 30, replace=False)]))
    _sampled_rows_check(x, w, rows, f"ue8m0 dsv3 {synth.DSV3_SHAPES[shape_index][0]}")


def test_linear_ue8m0():
    x, w = synth.llama_inputs(1, 64, config=3)
    wq, we = ou.weight_block_quant_ue8m0(w)
    y = fb.linear(to_dev_bf16(x), to_dev(wq), to_dev(we))
    torch.cuda.synchronize()
    xq, xe = ou.act_quant_group_ue8m0(x)
    check_tol(bf16_to_host(y), ou.block_gemm_ue8m0(xq, xe, wq, we),
              ou.term_magnitude_ue8m0(xq, xe, wq, we), "linear ue8m0")


@pytest.mark.parametrize("M,N,K", [(65, 1536, 7168), (130, 100, 3072), (1000, 700, 5632),
                                   (257, 129, 4096), (512, 576, 7168)])
def test_gemm_ue8m0_split_over_workgroups_exact(M, N, K):
    """fp8_block_gemm_ue8m0_ws with its K ranges (even block counts; the
    last shorter for 1000x700x5632 and 512x576x7168) on integer operands and
    scale bytes 126..128: exact, so bit-equal to bf16_RNE(exact); the
    workspace is pre-filled with NaN bytes."""
    need = fb.fp8_block_gemm_workspace_bytes(M, N, K, "ue8m0")
    assert need > 0
    rng = np.random.default_rng(M * 3 + N + K)
    xq = oe.encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    wq = oe.encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    KB, NB = K // 128, -(-N // 128)
    xe = rng.integers(126, 129, (M, KB)).astype(np.uint8)
    we = rng.integers(127, 129, (NB, KB)).astype(np.uint8)
    work = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev())
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm_ue8m0_ws(to_dev(xq), to_dev(xe), to_dev(wq), to_dev(we), y, work)
    torch.cuda.synchronize()
    want = og.bf16_rne_bits(ou.block_gemm_ue8m0(xq, xe, wq, we))
    bad = np.argwhere(bf16_to_host(y) != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


def test_gemm_ue8m0_split_dsv3_q_a_and_plain_fallback():
    """DeepSeek-V3 q_a at M = 512 with E8M0 scales: split (tolerance) and,
    with no workspace, bit for bit fp8_block_gemm_ue8m0; K/128 odd is
    never split."""
    x, w = synth.dsv3_inputs(0, 512)
    xq, xe, wq, we = operands(x, w)
    M, K = xq.shape
    N = wq.shape[0]
    assert fb.fp8_block_gemm_workspace_bytes(M, N, K, "ue8m0") > 0
    assert fb.fp8_block_gemm_workspace_bytes(512, 1536, 7040, "ue8m0") == 0      # 55 K blocks
    y = gpu_gemm_ue8m0(xq, xe, wq, we)                   # block_gemm takes the split
    check_tol(y, ou.block_gemm_ue8m0(xq, xe, wq, we), ou.term_magnitude_ue8m0(xq, xe, wq, we),
              "ue8m0 split q_a M=512")
    y0 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm_ue8m0(to_dev(xq), to_dev(xe), to_dev(wq), to_dev(we), y0)
    fb.fp8_block_gemm_ue8m0_ws(to_dev(xq), to_dev(xe), to_dev(wq), to_dev(we), y1, None)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_host(y0), bf16_to_host(y1))


def test_gemm_ue8m0_accepts_float8_e8m0fnu_and_rejects_fp32():
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("torch lacks float8_e8m0fnu")
    x, w = synth.tiny_inputs()
    xq, xe, wq, we = operands(x, w)
    y1 = gpu_gemm_ue8m0(xq, xe, wq, we)
    y2 = torch.empty((xq.shape[0], wq.shape[0]), dtype=torch.bfloat16, device=dev())
    fb.fp8_block_gemm_ue8m0(to_dev(xq), to_dev(xe).view(torch.float8_e8m0fnu), to_dev(wq),
                            to_dev(we).view(torch.float8_e8m0fnu), y2)
    torch.cuda.synchronize()
    assert np.array_equal(y1, bf16_to_host(y2))
    with pytest.raises(TypeError):
        fb.fp8_block_gemm_ue8m0(to_dev(xq), to_dev(xe).float(), to_dev(wq), to_dev(we).float(), y2)


def test_gemm_ue8m0_empty():
    d = dev()
    xq = torch.zeros((0, 256), dtype=torch.uint8, device=d)
    xe = torch.zeros((0, 2), dtype=torch.uint8, device=d)
    wq = torch.zeros((64, 256), dtype=torch.uint8, device=d)
    we = torch.zeros((1, 2), dtype=torch.uint8, device=d)
    assert fb.block_gemm(xq, xe, wq, we).shape == (0, 64)


# ----------------------------------------------------------------------------
# grouped GEMM

def _grouped_case(sizes, N, K, seed):
    E = len(sizes)
    off = synth.random_offsets(0, E, sizes=sizes)
    total = int(off[-1])
    x = synth.dsv3_activations(seed, total, K, seed + 1)
    w = synth.normal_bf16(seed + 2, (E, N, K), 0.01)
    xq, xe = ou.act_quant_group_ue8m0(x)
    NB = -(-N // 128)
    wq = np.empty((E, N, K), np.uint8); we = np.empty((E, NB, K // 128), np.uint8)
    for e in range(E):
        wq[e], we[e] = ou.weight_block_quant_ue8m0(w[e])
    return xq, xe, wq, we, off


@pytest.mark.parametrize("sizes,N,K", [
    ([0, 1, 15, 16, 17, 0, 130, 3], 256, 512),
    ([5], 576, 384),
    ([129, 255, 1, 0, 64], 300, 1024),
])
def test_grouped_ue8m0(sizes, N, K):
    xq, xe, wq, we, off = _grouped_case(sizes, N, K, sum(sizes) + N)
    y = fb.grouped_block_gemm(to_dev(xq), to_dev(xe), to_dev(wq), to_dev(we), to_dev(off))
    torch.cuda.synchronize()
    check_tol(bf16_to_host(y), ou.grouped_block_gemm_ue8m0(xq, xe, wq, we, off),
              ou.grouped_term_magnitude_ue8m0(xq, xe, wq, we, off), f"grouped ue8m0 {sizes}")


def test_grouped_ue8m0_rows_outside_experts_untouched():
    xq, xe, wq, we, off = _grouped_case([3, 4], 128, 256, 77)
    total = int(off[-1]) + 5
    xq = np.concatenate([xq, np.zeros((5, 256), np.uint8)])
    xe = np.concatenate([xe, np.full((5, 2), 127, np.uint8)])
    y = torch.full((total, 128), 7.0, dtype=torch.bfloat16, device=dev())
    fb.fp8_grouped_block_gemm_ue8m0(to_dev(xq), to_dev(xe), to_dev(wq), to_dev(we), to_dev(off), y)
    torch.cuda.synchronize()
    assert np.all(y.float().cpu().numpy()[-5:] == 7.0)


def test_grouped_ue8m0_moe_sampled():
    x, w, off = synth.moe_inputs(0)
    E, N, K = w.shape
    say("moe ue8m0", x.shape, w.shape)
    xq, xe = fb.act_quant_group(to_dev_bf16(x), "ue8m0")
    wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev())
    we = torch.empty((E, -(-N // 128), K // 128), dtype=torch.uint8, device=dev())
    for e in range(E):
        fb.fp8_weight_block_quant_ue8m0(to_dev_bf16(w[e]), wq[e], we[e])
    y = bf16_to_host(fb.grouped_block_gemm(xq, xe, wq, we, to_dev(off)))
    torch.cuda.synchronize()
    xq_h, xe_h, wq_h, we_h = host(xq), host(xe), host(wq), host(we)
    rng = np.random.default_rng(0)
    got, want, mag = [], [], []
    for e in range(E):
        # the oracle quantizes 3 rows of x and one 128-row weight block row
        # of every expert itself; the GPU's codes there must equal it
        r0, r1 = int(off[e]), int(off[e + 1])
        pick = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, 1)]))
        oxq, oxe = ou.act_quant_group_ue8m0(x[pick])
        assert_codes_equal(xq_h[pick], xe_h[pick], oxq, oxe, f"moe ue8m0 expert {e} rows")
        nb = int(rng.integers(0, -(-N // 128)))
        c0, c1 = 128 * nb, min(N, 128 * nb + 128)
        owq, owe = ou.weight_block_quant_ue8m0(w[e][c0:c1])
        assert_codes_equal(wq_h[e][c0:c1], we_h[e][nb:nb + 1], owq, owe,
                           f"moe ue8m0 expert {e} weight block row {nb}")
        got.append(y[pick][:, c0:c1])
        want.append(ou.block_gemm_ue8m0(oxq, oxe, owq, owe))
        mag.append(ou.term_magnitude_ue8m0(oxq, oxe, owq, owe))
    check_tol(np.concatenate(got), np.concatenate(want), np.concatenate(mag), "moe ue8m0")
