"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching)
and check that at least one pin fails for each: the pins are strong enough
to catch a wrong scale constant, a wrong rounding rule, a dropped sign, a
transposed operand, a wrong scale index and a dropped K block."""
import numpy as np
import pytest

import oracle_pins as P
from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import quant as oq
from oracle import ue8m0 as ou
from oracle import static as ost
from oracle import layouts as olay
from oracle import swiglu as osw


def _fails(pins):
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return [pin.__name__]
        except Exception as e:  # a crash also counts as caught
            return [pin.__name__ + ":" + type(e).__name__]
    return failed


def _encode_ties_away(t):
    t = np.asarray(t, np.float32).astype(np.float64)
    a = np.minimum(np.abs(t), 448.0)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    q = np.exp2(np.maximum(e, -6) - 3)
    v = np.floor(a / q + 0.5) * q
    return _orig_encode(np.copysign(v, t).astype(np.float32))


_orig_encode = oe.encode


def _quant_map_reciprocal(x_f32, amax_f32):
    x = np.asarray(x_f32, np.float32); amax = np.asarray(amax_f32, np.float32)
    s = (amax / np.float32(448)).astype(np.float32)
    r = np.where(s == 0, np.float32(1), np.float32(1) / np.where(s == 0, 1, s)).astype(np.float32)
    return oe.encode((x * r).astype(np.float32)), s


MUTANTS = {
    "scale_uses_240": lambda mp: mp.setattr(oq, "_F32_448", np.float32(240.0)),
    "encode_ties_away": lambda mp: mp.setattr(oq, "encode", _encode_ties_away),
    "divide_by_reciprocal": lambda mp: mp.setattr(oq, "quant_element_map", _quant_map_reciprocal),
    "decode_bias_8": lambda mp: mp.setattr(oe, "decode", lambda c: _orig_decode(c) / 2.0),
    "gemm_transposed_weight_scale": lambda mp: mp.setattr(
        og, "dequant_weight", lambda q, s: _orig_dw(q, s.T.copy() if s.shape[0] == s.shape[1] else s[::-1].copy())),
    "gemm_drops_last_kblock": lambda mp: mp.setattr(
        og, "dequant_act", lambda q, s: _orig_da(q, np.concatenate([s[:, :-1], 0 * s[:, -1:]], 1))),
    "bf16_truncates": lambda mp: mp.setattr(
        og, "bf16_rne_bits", lambda y: (np.asarray(y, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)),
    "grouped_off_by_one": lambda mp: mp.setattr(
        og, "grouped_block_gemm", _grouped_shift),
    "weight_amax_full_block_rows": lambda mp: mp.setattr(oq, "GROUP", 64),
    "ue8m0_floor_exponent": lambda mp: mp.setattr(ou, "e8m0_exponent", _e8m0_floor),
    "ue8m0_strict_bound": lambda mp: mp.setattr(ou, "e8m0_exponent", _e8m0_strict),
    "ue8m0_no_lower_clamp": lambda mp: mp.setattr(ou, "E_MIN", -133),
    "e8m0_bias_128": lambda mp: mp.setattr(ou, "E8M0_BIAS", 128),
    "batched_ignores_count": lambda mp: mp.setattr(
        olay, "batched_block_gemm", lambda xq, xs, wq, ws, c: _orig_batched(xq, xs, wq, ws, np.full_like(c, xq.shape[1]))),
    "rowwise_scale_per_group": lambda mp: mp.setattr(olay, "rowwise_quant", _rowwise_group),
    "rowwise_gemm_swapped_scales": lambda mp: mp.setattr(
        olay, "rowwise_gemm", lambda xq, xs, wq, ws: _orig_rowwise_gemm(xq, np.resize(ws, xs.shape), wq, np.resize(xs, ws.shape))),
    "static_no_saturation": lambda mp: mp.setattr(ost, "act_quant_static", _static_nosat),
    "static_reciprocal_multiply": lambda mp: mp.setattr(ost, "act_quant_static", _static_recip),
    "static_scale_multiplies": lambda mp: mp.setattr(ost, "act_quant_static", _static_mul),
    "swiglu_halves_swapped": lambda mp: mp.setattr(osw, "swiglu_bf16", _swiglu_swapped),
    "swiglu_sigmoid_sign": lambda mp: mp.setattr(osw, "swiglu_bf16", lambda b: _swiglu_variant(b, sign=+1)),
    "swiglu_rounds_silu_first": lambda mp: mp.setattr(osw, "swiglu_bf16", lambda b: _swiglu_variant(b, two_roundings=True)),
    "swiglu_quantizes_unrounded_h": lambda mp: mp.setattr(osw, "swiglu_act_quant", _swiglu_quant_f32),
    "ue8m0_gemm_weight_bytes_reversed": lambda mp: mp.setattr(
        ou, "block_gemm_ue8m0", lambda xq, xe, wq, we: _orig_bg_ue(xq, xe, wq, we[::-1].copy())),
}

_orig_decode = oe.decode
_orig_e8m0_exponent = ou.e8m0_exponent
_orig_bg_ue = ou.block_gemm_ue8m0


_orig_swiglu = osw.swiglu_bf16


def _swiglu_swapped(bits):
    b = np.asarray(bits, np.uint16)
    I = b.shape[1] // 2
    return _orig_swiglu(np.concatenate([b[:, I:], b[:, :I]], axis=1))


def _swiglu_variant(bits, sign=-1, two_roundings=False):
    b = np.asarray(bits, np.uint16)
    I = b.shape[1] // 2
    v = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, u = v[:, :I], v[:, I:]
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(sign * g))
    if two_roundings:
        silu = og.bf16_bits_to_f64(og.bf16_rne_bits(silu))
    return og.bf16_rne_bits(silu * u)


def _swiglu_quant_f32(bits):
    b = np.asarray(bits, np.uint16)
    I = b.shape[1] // 2
    v = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    h = (v[:, :I] / (1.0 + np.exp(-v[:, :I])) * v[:, I:]).astype(np.float32)
    M = h.shape[0]
    hg = h.reshape(M, I // 128, 128)
    q, s = oq.quant_element_map(hg, np.max(np.abs(hg), axis=2, keepdims=True))
    return q.reshape(M, I), s.reshape(M, I // 128)


_orig_batched = olay.batched_block_gemm
_orig_rowwise_gemm = olay.rowwise_gemm


def _rowwise_group(bits):
    q, s = oq.act_quant_group(np.asarray(bits, np.uint16))
    return q, s[:, 0].copy()


def _static_nosat(x_bits, scale):
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    t = (x / np.float32(scale)).astype(np.float32)
    a = np.abs(t).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    q = np.exp2(np.maximum(e, -6) - 3)
    v = np.rint(a / q) * q                  # no clamp: values above 448 stay large
    v = np.where(v > 448, np.nan, v)        # which has no finite code
    c = oe.encode(np.nan_to_num(np.copysign(v, t), nan=0.0).astype(np.float32))
    return np.where(np.isnan(v), 0x7F, c).astype(np.uint8)


def _static_recip(x_bits, scale):
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    r = np.float32(1.0) / np.float32(scale)
    return oe.encode(np.clip((x * r).astype(np.float32), -448, 448))


def _static_mul(x_bits, scale):
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return oe.encode(np.clip((x * np.float32(scale)).astype(np.float32), -448, 448))


def _e8m0_floor(amax):
    a = np.asarray(amax, np.float32).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0) / 448.0))
    return np.maximum(np.where(a > 0, e, -127), -127).astype(np.int64)


def _e8m0_strict(amax):
    a = np.asarray(amax, np.float32).astype(np.float64)
    e = _orig_e8m0_exponent(amax)
    return np.where(a == 448.0 * np.exp2(e.astype(np.float64)), e + 1, e)
_orig_dw = og.dequant_weight
_orig_da = og.dequant_act
_orig_grouped = og.grouped_block_gemm


def _grouped_shift(x_q, x_s, w_q, w_s, offsets):
    off = np.asarray(offsets).copy()
    off[1:-1] = np.maximum(off[1:-1] - 1, 0)
    return _orig_grouped(x_q, x_s, w_q, w_s, off)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    failed = _fails(P.ALL_PINS)
    assert failed, f"planted mistake {name} passed every pin"
