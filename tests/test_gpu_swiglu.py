"""GPU parity of the fused SwiGLU + activation quantizer against the CPU
oracle: codes and fp32 scales bit-exact.

Coverage: every finite bf16 gate value (both signs) with several up values,
the hand-worked cases (including a binary64 rounding tie and gates whose
e^-g overflows), inputs built to land near bf16 rounding midpoints (where
the kernel's fp32 evaluation defers to binary64), ragged shapes, and the
mixture-of-experts down-projection input at full size (32768 tokens x
I = 2048, sampled rows compared)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as fb
import synth
from oracle import swiglu as osw
from gpu_helpers import assert_codes_equal, dev, host, say, to_dev_bf16

pytestmark = pytest.mark.gpu


def gpu_swiglu_quant(gu_bits):
    q, s = fb.swiglu_act_quant(to_dev_bf16(gu_bits))
    torch.cuda.synchronize()
    return host(q), host(s)


def check(gu_bits, what):
    say("swiglu quant", what, gu_bits.shape)
    q, s = gpu_swiglu_quant(gu_bits)
    wq, ws = osw.swiglu_act_quant(gu_bits)
    assert_codes_equal(q, s, wq, ws, what)


def bits_of(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def all_finite_gates():
    b = np.arange(0, 0x7F80, dtype=np.uint16)
    return np.concatenate([b, b | 0x8000]).astype(np.uint16)


def gate_up_from_pairs(g, u, I):
    """Pack 1-D gate and up bit arrays (same length, padded with zeros) into
    rows of a [M, 2I] gate/up block."""
    n = len(g)
    M = -(-n // I)
    gg = np.zeros(M * I, np.uint16); uu = np.zeros(M * I, np.uint16)
    gg[:n] = g; uu[:n] = u
    return np.concatenate([gg.reshape(M, I), uu.reshape(M, I)], axis=1)


@pytest.mark.parametrize("which", ["one", "neg_three", "small", "wide"])
def test_every_bf16_gate(which):
    g = all_finite_gates()
    gv = (g.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(len(which))
    if which == "one":
        u = np.full(len(g), 0x3F80, np.uint16)                       # h = SiLU(g)
    elif which == "neg_three":
        u = np.full(len(g), 0xC040, np.uint16)
        g = np.where(np.abs(gv) < 1e38, g, 0).astype(np.uint16)      # keep 3 * SiLU(g) finite
    elif which == "small":
        u = bits_of(rng.uniform(-4, 4, len(g)))
        g = np.where(np.abs(gv) < 1e37, g, 0).astype(np.uint16)
    else:
        u = bits_of(np.sign(rng.standard_normal(len(g))) * np.exp2(rng.uniform(-60, 60, len(g))))
        g = np.where(np.abs(gv) < 2.0 ** 60, g, 0).astype(np.uint16)
    check(gate_up_from_pairs(g, u, 1024), f"all gates, up={which}")


def test_hand_cases():
    from oracle_pins import read_golden
    rows = read_golden("swiglu_hand_cases.txt")
    g = np.array([int(r.split("|")[0], 16) for r in rows], np.uint16)
    u = np.array([int(r.split("|")[1], 16) for r in rows], np.uint16)
    want = [int(r.split("|")[2], 16) for r in rows]
    # each case in a group of its own (the group's amax is the case itself)
    gu = np.zeros((len(rows), 256), np.uint16)
    gu[:, 0] = g; gu[:, 128] = u
    q, s = gpu_swiglu_quant(gu)
    wq, ws = osw.swiglu_act_quant(gu)
    assert osw.swiglu_bf16(gu)[:, 0].tolist() == want
    assert_codes_equal(q, s, wq, ws, "hand cases")


def test_near_midpoints():
    """Gates >= 37 make 1 + e^-g round to 1 in binary64, so h is the exact
    product g * u rounded once; choosing u so that g * u falls on, or within
    a few fp32 ulps of, a bf16 rounding midpoint exercises the kernel's
    binary64 fallback and its ties-to-even."""
    rng = np.random.default_rng(7)
    n = 4096
    g = (np.float32(64.0) * (1 + rng.integers(0, 128, n) / 128)).astype(np.float32)   # exact bf16
    u = (1 + rng.integers(0, 128, n) / 128).astype(np.float32)
    # g * u: 16 significant bits at most; keep the pairs whose product sits
    # exactly on a midpoint (bit 8 below the leading one set, the rest clear)
    gu = np.concatenate([bits_of(g), bits_of(u)])
    prod = (g.astype(np.float64) * u.astype(np.float64)).astype(np.float32).view(np.uint32)
    on_mid = (prod & 0xFFFF) == 0x8000
    say("pairs on a midpoint:", int(on_mid.sum()))
    assert on_mid.sum() > 50
    # plus small gates whose fp32 result lands close to a midpoint
    g2 = bits_of(rng.uniform(-6, 6, 20000))
    u2 = bits_of(rng.uniform(-2, 2, 20000))
    gg = np.concatenate([gu[:n], g2]); uu = np.concatenate([gu[n:], u2])
    check(gate_up_from_pairs(gg, uu, 512), "near midpoints")


def test_zero_heavy():
    """Half the gates and a third of the up values exact (signed) zeros:
    the products are exact signed zeros on both sides."""
    rng = np.random.default_rng(19)
    gu = synth.moe_gate_up_output(23, 96, 512)
    I = 512
    zg = rng.random((96, I)) < 0.5
    zu = rng.random((96, I)) < 0.33
    gu[:, :I] = np.where(zg, (rng.integers(0, 2, (96, I)) << 15).astype(np.uint16), gu[:, :I])
    gu[:, I:] = np.where(zu, (rng.integers(0, 2, (96, I)) << 15).astype(np.uint16), gu[:, I:])
    gu[0, :I] = 0x8000                                   # a row of -0 gates: all-zero groups
    check(gu, "zero-heavy")


@pytest.mark.parametrize("M,I", [(1, 128), (3, 384), (17, 2048), (130, 256), (5, 7168), (64, 128)])
def test_ragged(M, I):
    gu = synth.moe_gate_up_output(M * 31 + I, M, I)
    check(gu, f"{M}x{I}")


def test_tail_of_the_grid():
    """More groups than one pass of the grid covers (the grid-stride loop)
    with a group count that is not a multiple of the 16-group tile."""
    M, I = 8195, 384
    gu = synth.moe_gate_up_output(11, M, I)
    check(gu, f"{M}x{I}")


def test_moe_down_input_full_size():
    """The down-projection input of the MoE share: 32768 token rows, gate/up
    [32768, 4096] -> codes [32768, 2048]; 96 sampled rows (first and last
    included) against the oracle."""
    M, I = synth.MOE_TOKENS * synth.MOE_TOPK, synth.MOE_INTERMEDIATE
    gu = synth.moe_gate_up_output(synth.seed_of(5, 1, 4), M, I)
    q, s = gpu_swiglu_quant(gu)
    rows = np.sort(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(np.arange(1, M - 1), 94, replace=False)]))
    wq, ws = osw.swiglu_act_quant(gu[rows])
    assert_codes_equal(q[rows], s[rows], wq, ws, "moe down input (sampled rows)")


def test_empty_and_errors():
    d = dev()
    gu = torch.empty((0, 512), dtype=torch.bfloat16, device=d)
    q, s = fb.swiglu_act_quant(gu)
    assert q.shape == (0, 256) and s.shape == (0, 2)
    with pytest.raises(ValueError):
        fb.swiglu_act_quant(torch.zeros((4, 400), dtype=torch.bfloat16, device=d))   # I = 200


def test_fused_equals_quantizer_of_oracle_h():
    """The fused kernel's codes equal the plain activation quantizer's codes
    of the oracle's h, run on the GPU: h never needs to exist in memory."""
    gu = synth.moe_gate_up_output(21, 64, 2048)
    h = osw.swiglu_bf16(gu)
    q1, s1 = gpu_swiglu_quant(gu)
    q2, s2 = fb.act_quant_group(to_dev_bf16(h))
    torch.cuda.synchronize()
    assert_codes_equal(q1, s1, host(q2), host(s2), "fused vs quantizer of h")


# ----------------------------------------------------------------------------
# power-of-two (E8M0) scales on the same h

def gpu_swiglu_quant_ue8m0(gu_bits):
    q, s = fb.swiglu_act_quant(to_dev_bf16(gu_bits), "ue8m0")
    torch.cuda.synchronize()
    return host(q), host(s)


def check_ue8m0(gu_bits, what):
    say("swiglu quant ue8m0", what, gu_bits.shape)
    q, s = gpu_swiglu_quant_ue8m0(gu_bits)
    wq, ws = osw.swiglu_act_quant_ue8m0(gu_bits)
    assert_codes_equal(q, s, wq, ws, what)


@pytest.mark.parametrize("which", ["one", "wide"])
def test_ue8m0_every_bf16_gate(which):
    g = all_finite_gates()
    gv = (g.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(3 + len(which))
    if which == "one":
        u = np.full(len(g), 0x3F80, np.uint16)
    else:
        u = bits_of(np.sign(rng.standard_normal(len(g))) * np.exp2(rng.uniform(-60, 60, len(g))))
        g = np.where(np.abs(gv) < 2.0 ** 60, g, 0).astype(np.uint16)
    check_ue8m0(gate_up_from_pairs(g, u, 1024), f"ue8m0 all gates, up={which}")


@pytest.mark.parametrize("M,I", [(1, 128), (17, 2048), (130, 384), (8195, 256)])
def test_ue8m0_ragged(M, I):
    check_ue8m0(synth.moe_gate_up_output(M * 13 + I, M, I), f"ue8m0 {M}x{I}")


def test_ue8m0_hand_cases_and_zeros():
    from oracle_pins import read_golden
    rows = read_golden("swiglu_hand_cases.txt")
    gu = np.zeros((len(rows) + 1, 256), np.uint16)
    for i, r in enumerate(rows):
        gu[i, 0], gu[i, 128] = int(r.split("|")[0], 16), int(r.split("|")[1], 16)
    gu[-1, :128] = 0x8000                                 # an all-zero group: byte 0
    check_ue8m0(gu, "ue8m0 hand cases")


def test_ue8m0_moe_down_input_full_size():
    M, I = synth.MOE_TOKENS * synth.MOE_TOPK, synth.MOE_INTERMEDIATE
    gu = synth.moe_gate_up_output(synth.seed_of(5, 1, 5), M, I)
    q, s = gpu_swiglu_quant_ue8m0(gu)
    rows = np.sort(np.concatenate([[0, M - 1], np.random.default_rng(4).choice(np.arange(1, M - 1), 62, replace=False)]))
    wq, ws = osw.swiglu_act_quant_ue8m0(gu[rows])
    assert_codes_equal(q[rows], s[rows], wq, ws, "ue8m0 moe down input (sampled rows)")


def test_ue8m0_accepts_float8_e8m0fnu():
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("torch has no float8_e8m0fnu")
    gu = synth.moe_gate_up_output(31, 8, 256)
    gd = to_dev_bf16(gu)
    q = torch.empty((8, 256), dtype=torch.uint8, device=dev())
    s = torch.empty((8, 2), dtype=torch.float8_e8m0fnu, device=dev())
    fb.fp8_swiglu_act_quant_ue8m0(gd, q, s)
    torch.cuda.synchronize()
    wq, ws = osw.swiglu_act_quant_ue8m0(gu)
    assert_codes_equal(host(q), s.view(torch.uint8).cpu().numpy(), wq, ws, "e8m0fnu scales")
