"""GPU parity of the two quantizers against the CPU oracle: codes and
scales must match bit for bit (uint8 codes, fp32 scale bit patterns), on
the configured workloads, on edge cases and on the whole (x, amax) bf16
domain (chunk digests written by tests/golden/make_exhaustive_digests.py)."""
import hashlib
import os

import numpy as np
import pytest

import synth
from oracle import quant as oq
from gpu_helpers import assert_codes_equal, gpu_act_quant, gpu_weight_quant, say

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
NCHUNKS = max(c for _, c in DIGESTS) + 1


# ----------------------------------------------------------------------------
# activation quantizer

def test_act_quant_tiny():
    x, _ = synth.tiny_inputs()
    say("act_quant tiny", x.shape)
    assert_codes_equal(*gpu_act_quant(x), *oq.act_quant_group(x), "tiny")


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (17, 512), (5, 1536), (33, 2048),
                                 (1, 4096), (4, 14336), (16, 4096), (127, 7168), (131, 128)])
def test_act_quant_ragged(M, K):
    x = synth.dsv3_activations(M * 7 + K, M, K, M + 3)
    say("act_quant", M, K)
    assert_codes_equal(*gpu_act_quant(x), *oq.act_quant_group(x), f"{M}x{K}")


@pytest.mark.parametrize("shape_index", range(4))
@pytest.mark.parametrize("M", [1, 4, 16, 4096])
def test_act_quant_llama(shape_index, M):
    x = synth.llama_x(shape_index, M, config=2 if M <= 16 else 3)
    say("act_quant llama", shape_index, x.shape)
    assert_codes_equal(*gpu_act_quant(x), *oq.act_quant_group(x), f"llama {shape_index} M={M}")


@pytest.mark.parametrize("shape_index", range(6))
def test_act_quant_dsv3_sampled_rows(shape_index):
    """M = 8192 on the GPU; the oracle checks 256 sampled rows (each token's
    codes depend on that token only)."""
    name, N, K = synth.DSV3_SHAPES[shape_index]
    x = synth.dsv3_activations(synth.seed_of(4, shape_index, 1), 8192, K,
                               synth.seed_of(4, shape_index, 3))
    say("act_quant dsv3", name, x.shape)
    q, s = gpu_act_quant(x)
    rows = np.sort(np.random.default_rng(shape_index).choice(8192, 256, replace=False))
    rows = np.concatenate([[0, 8191], rows])
    wq, ws = oq.act_quant_group(x[rows])
    assert_codes_equal(q[rows], s[rows], wq, ws, name)


def test_act_quant_edge_values():
    rng = np.random.default_rng(5)
    M, K = 12, 512
    x = np.zeros((M, K), np.uint16)
    x[1, :] = 0x8000                                   # all -0
    x[2, :128] = rng.integers(0, 0x80, 128)            # bf16 subnormals, +
    x[2, 128:256] = rng.integers(0x8000, 0x8080, 128)  # bf16 subnormals, -
    x[3, :] = rng.integers(0x7F00, 0x7F80, K)          # near the bf16 maximum
    x[4, :] = 0x0001                                   # smallest subnormal only
    x[5, ::2] = 0x7F7F; x[5, 1::2] = 0x0001            # widest spread in a group
    x[6, :] = synth.f32_to_bf16_bits(rng.standard_normal(K).astype(np.float32) * 1e-30)
    x[7, :] = synth.f32_to_bf16_bits(rng.standard_normal(K).astype(np.float32) * 1e30)
    x[8, :] = synth.f32_to_bf16_bits(np.full(K, 448.0, np.float32))
    x[9, :] = synth.f32_to_bf16_bits(np.linspace(-3, 3, K).astype(np.float32))
    x[10, 5] = 0x3F80                                  # one nonzero in a zero group
    x[11, :] = rng.integers(0, 0x7F80, K) | (rng.integers(0, 2, K) << 15).astype(np.uint16)
    q, s = gpu_act_quant(x)
    wq, ws = oq.act_quant_group(x)
    assert_codes_equal(q, s, wq, ws, "edge values")
    assert s[0, 0] == 0 and np.all(q[1] == 0x80)


def test_act_quant_empty():
    import torch
    import block_scaled_fp8_act_amd as fb
    from gpu_helpers import dev
    q, s = fb.act_quant_group(torch.empty((0, 256), dtype=torch.bfloat16, device=dev()))
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_act_quant_rejects_bad_k():
    import torch
    import block_scaled_fp8_act_amd as fb
    from gpu_helpers import dev
    with pytest.raises(ValueError):
        fb.act_quant_group(torch.zeros((4, 200), dtype=torch.bfloat16, device=dev()))


def _digest(q, s):
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(q).tobytes())
    h.update(np.ascontiguousarray(s, dtype=np.float32).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("chunk", range(NCHUNKS))
def test_act_quant_exhaustive(chunk):
    lo, hi, want = DIGESTS[("act", chunk)]
    x = synth.exhaustive_act_chunk(lo, hi)
    say(f"act exhaustive chunk {chunk} amax [{lo:#x},{hi:#x}) groups {x.shape[0]}")
    q, s = gpu_act_quant(x)
    if _digest(q, s) != want:
        wq, ws = oq.act_quant_group(x)
        assert_codes_equal(q, s, wq, ws, f"exhaustive act chunk {chunk}")
        pytest.fail("digest differs although codes match: regenerate the digests")


# ----------------------------------------------------------------------------
# weight quantizer

def test_weight_quant_tiny():
    _, w = synth.tiny_inputs()
    assert_codes_equal(*gpu_weight_quant(w), *oq.weight_block_quant(w), "tiny W")


@pytest.mark.parametrize("N,K", [(1, 128), (64, 256), (100, 384), (129, 128), (576, 7168),
                                 (300, 1024), (1000, 640)])
def test_weight_quant_ragged(N, K):
    w = synth.normal_bf16(N * 31 + K, (N, K), 0.01)
    say("weight_quant", N, K)
    assert_codes_equal(*gpu_weight_quant(w), *oq.weight_block_quant(w), f"W {N}x{K}")


@pytest.mark.parametrize("which", ["llama_qo", "llama_down", "dsv3_q_b", "dsv3_kv_a", "moe_down_e0"])
def test_weight_quant_workloads(which):
    if which == "llama_qo":
        w = synth.llama_weight(0)
    elif which == "llama_down":
        w = synth.llama_weight(3)
    elif which == "dsv3_q_b":
        w = synth.dsv3_inputs(1, 1)[1]
    elif which == "dsv3_kv_a":
        w = synth.dsv3_inputs(2, 1)[1]
    else:
        w = synth.normal_bf16(synth.seed_of(5, 1, 2), (7168, 2048), 0.01)
    say("weight_quant", which, w.shape)
    assert_codes_equal(*gpu_weight_quant(w), *oq.weight_block_quant(w), which)


def test_weight_quant_edge_blocks():
    rng = np.random.default_rng(9)
    N, K = 200, 512
    w = np.zeros((N, K), np.uint16)
    w[:128, 128:256] = 0x8000
    w[:128, 256:384] = rng.integers(0, 0x80, (128, 128))
    w[128:, :128] = 0x7F7F
    w[128:, 384:] = rng.integers(0, 0x7F80, (72, 128)) | 0x8000
    w[150, 300] = 0x0001
    assert_codes_equal(*gpu_weight_quant(w), *oq.weight_block_quant(w), "edge blocks")


@pytest.mark.parametrize("chunk", range(NCHUNKS))
def test_weight_quant_exhaustive(chunk):
    lo, hi, want = DIGESTS[("weight", chunk)]
    w = synth.exhaustive_weight_chunk(lo, hi)
    say(f"weight exhaustive chunk {chunk} amax [{lo:#x},{hi:#x}) rows {w.shape[0]}")
    q, s = gpu_weight_quant(w)
    if _digest(q, s) != want:
        wq, ws = oq.weight_block_quant(w)
        assert_codes_equal(q, s, wq, ws, f"exhaustive weight chunk {chunk}")
        pytest.fail("digest differs although codes match: regenerate the digests")
