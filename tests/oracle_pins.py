"""Pins for the CPU oracle: checks against facts fixed by the E4M3 format,
by exact arithmetic, by brute force and by the hand-worked golden files.

Each ``pin_*`` function raises AssertionError when the oracle disagrees.
They are collected by ``test_oracle_pins.py`` and re-run against planted
mistakes by ``test_oracle_mutations.py`` (every plausible mistake must trip
at least one pin).  Nothing here calls the GPU path.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

import oracle
from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import quant as oq
from oracle import ue8m0 as ou
from oracle import static as ost
from oracle import layouts as olay
from oracle import swiglu as osw

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent exact helpers (pure Python integers / fractions)

def f32_value(bits: int) -> Fraction:
    """Exact value of an fp32 bit pattern (finite)."""
    s = -1 if bits >> 31 else 1
    e = (bits >> 23) & 0xFF
    f = bits & 0x7FFFFF
    if e == 0:
        return s * Fraction(f, 1 << 149)
    return s * Fraction(f | 0x800000) * Fraction(2) ** (e - 150)


def fl32_of(q: Fraction) -> float:
    """Round an exact rational to binary32, nearest with ties to even
    (subnormals kept; no overflow handling needed for the callers)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    quantum_exp = max(e, -126) - 23
    scaled = a / Fraction(2) ** quantum_exp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) * Fraction(2) ** quantum_exp)


def bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def e4m3_finite_table():
    """All 254 finite E4M3 values listed from the OCP definition by
    enumeration (value of each code), for brute-force nearest searches."""
    codes, vals = [], []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        codes.append(c)
        vals.append(-v if s else v)
    return codes, vals


def brute_force_encode(t: float) -> int:
    """Nearest finite E4M3 value to clamp(t, +-448) by exhaustive search;
    ties go to the code with an even mantissa; the sign of t is kept."""
    codes, vals = e4m3_finite_table()
    tt = Fraction(min(max(t, -448.0), 448.0))
    best = None
    for c, v in zip(codes, vals):
        if (c >> 7) != (1 if math.copysign(1.0, t) < 0 else 0):
            continue
        d = abs(v - tt)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1]


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


# ----------------------------------------------------------------------------
# codec pins

def pin_format_points():
    for row in read_golden("e4m3_format_points.txt"):
        code_s, val_s = row.split()
        code, want = int(code_s, 16), float(val_s)
        got = float(oe.decode(np.array([code], np.uint8))[0])
        if math.isnan(want):
            assert math.isnan(got), (hex(code), got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(code), got, want)


def pin_hand_encodings():
    for row in read_golden("e4m3_hand_cases.txt"):
        v_s, c_s = row.split()[:2]
        got = int(oe.encode(np.array([float(v_s)], np.float32))[0])
        assert got == int(c_s, 16), (v_s, hex(got), c_s)


def pin_decode_matches_enumeration():
    codes, vals = e4m3_finite_table()
    got = oe.decode(np.array(codes, np.uint8))
    for c, v, g in zip(codes, vals, got):
        assert g == float(v), (hex(c), g, float(v))
    assert np.isnan(oe.decode(np.array([0x7F, 0xFF], np.uint8))).all()


def pin_encode_roundtrip_and_monotone():
    codes, vals = e4m3_finite_table()
    back = oe.encode(np.array([math.copysign(float(v), -1.0 if c >> 7 else 1.0)
                               for c, v in zip(codes, vals)], np.float32))
    for c, v, b in zip(codes, vals, back):
        assert b == c, (hex(c), hex(b))
    t = np.sort(np.random.default_rng(7).uniform(-500, 500, 20000).astype(np.float32))
    dv = oe.decode(oe.encode(t))
    assert np.all(np.diff(dv) >= 0)


def pin_encode_brute_force(n=3000, seed=11):
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-14, 9.2, n))
    t = (mags * rng.choice([-1, 1], n)).astype(np.float32)
    # add exact midpoints between neighbouring codes and their fp32 neighbours
    codes, vals = e4m3_finite_table()
    pos = sorted(float(v) for v in vals if v > 0)
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])][::5]
    mids = np.array(mids, np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                            -mids, np.array([464.0, 463.9, 447.9, 0.0], np.float32)])
    t = np.concatenate([t, extra]).astype(np.float32)
    got = oe.encode(t)
    for ti, gi in zip(t, got):
        want = brute_force_encode(float(ti))
        assert gi == want, (float(ti), hex(gi), hex(want))


def pin_fl32_div(n=4000, seed=3):
    rng = np.random.default_rng(seed)
    a_bits = rng.integers(0, 0x7F80, n).astype(np.uint32) << 16   # bf16-valued
    b = (rng.integers(0x00000001, 0x7F7FFFFF, n)).astype(np.uint32)
    a = a_bits.view(np.float32)
    bf = b.view(np.float32)
    q = oe.fl32_div(a, bf)
    for ai, bi, qi, ab, bb in zip(a, bf, q, a_bits, b):
        exact = f32_value(int(ab)) / f32_value(int(bb))
        if abs(exact) > Fraction(2) ** 127:
            continue
        assert float(qi) == fl32_of(exact), (float(ai), float(bi), float(qi))


# ----------------------------------------------------------------------------
# quantizer pins

def pin_hand_groups():
    for row in read_golden("quant_hand_groups.txt"):
        amax_s, xs_s, s_s, q_s = [p.strip() for p in row.split("|")]
        xb = np.array([int(v, 16) for v in xs_s.split()], np.uint16)
        want_q = [int(v, 16) for v in q_s.split()]
        # put the group in a 128-wide row, padded with zeros
        row128 = np.zeros((1, 128), np.uint16)
        row128[0, : len(xb)] = xb
        q, s = oq.act_quant_group(row128)
        assert int(s.view(np.uint32)[0, 0]) == int(s_s, 16), (hex(int(s.view(np.uint32)[0, 0])), s_s)
        assert list(q[0, : len(xb)]) == want_q, ([hex(c) for c in q[0, : len(xb)]], q_s)
        # the same element map through the weight quantizer (one 128x128 block)
        blk = np.zeros((128, 128), np.uint16)
        blk[5, : len(xb)] = xb
        wq, ws = oq.weight_block_quant(blk)
        assert int(ws.view(np.uint32)[0, 0]) == int(s_s, 16)
        assert list(wq[5, : len(xb)]) == want_q


def pin_scale_is_fl32_amax_over_448(n=300, seed=5):
    rng = np.random.default_rng(seed)
    amax_bits = rng.integers(1, 0x7F80, n)
    x = np.zeros((n, 128), np.uint16)
    x[:, 17] = amax_bits
    x[:, 3] = amax_bits // 3
    _, s = oq.act_quant_group(x)
    for ab, si in zip(amax_bits, s[:, 0]):
        want = fl32_of(Fraction(bf16_value(int(ab))) / 448)
        assert float(si) == want, (int(ab), float(si), want)


def pin_exact_on_representable(seed=13):
    """x = c * 2^j with the group's amax 448 * 2^j: s = 2^j, codes = c."""
    rng = np.random.default_rng(seed)
    codes, vals = e4m3_finite_table()
    for j in (-20, -3, 0, 5, 40):
        pick = rng.choice(len(codes), 127)
        cs = [codes[i] for i in pick]
        x = np.array([448.0 * 2.0 ** j] + [math.copysign(float(vals[i]) * 2.0 ** j, -1.0 if codes[i] >> 7 else 1.0)
                                           for i in pick], np.float32)
        xb = (x.view(np.uint32) >> 16).astype(np.uint16)
        assert np.all((xb.astype(np.uint32) << 16).view(np.float32) == x)
        q, s = oq.act_quant_group(xb[None, :])
        assert float(s[0, 0]) == 2.0 ** j
        assert q[0, 0] == 0x7E
        assert list(q[0, 1:]) == cs
        # amax = 7 * 2^j gives s = 2^(j-6) exactly
        x7 = np.zeros(128, np.float32); x7[0] = 7 * 2.0 ** j; x7[1] = 2.0 ** j
        _, s7 = oq.act_quant_group((x7.view(np.uint32) >> 16).astype(np.uint16)[None, :])
        assert float(s7[0, 0]) == 2.0 ** (j - 6)


def pin_quant_ties():
    """Quotients that land exactly halfway between two E4M3 values (s = 2^j
    exact) round to the even mantissa through the whole quantizer."""
    base = [448.0, 1.0625, 1.1875, 232.0, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, -232.0]
    want = [0x7E, 0x38, 0x3A, 0x76, 0x02, 0x00, 0xB8, 0xF6]
    for j in (-7, 0, 9):
        x = np.zeros(128, np.float32)
        x[: len(base)] = np.array(base) * 2.0 ** j
        xb = (x.view(np.uint32) >> 16).astype(np.uint16)
        q, s = oq.act_quant_group(xb[None, :])
        assert float(s[0, 0]) == 2.0 ** j
        assert list(q[0, : len(base)]) == want, [hex(c) for c in q[0, : len(base)]]
        wq, ws = oq.weight_block_quant(np.tile(xb, (3, 1)))
        assert list(wq[2, : len(base)]) == want


def pin_group_invariants(seed=17):
    rng = np.random.default_rng(seed)
    M, K = 24, 512
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 30, (M, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = oq.act_quant_group(xb)
    assert q.shape == (M, K) and s.shape == (M, K // 128)
    assert not np.any((q & 0x7F) == 0x7F), "NaN code produced"
    qq = q.reshape(M, K // 128, 128)
    assert np.all(np.any((qq & 0x7F) == 0x7E, axis=2)), "a group lacks its +-448 code"
    # token independence: quantizing a subset of rows gives the same rows
    q2, s2 = oq.act_quant_group(xb[5:9])
    assert np.array_equal(q2, q[5:9]) and np.array_equal(s2.view(np.uint32), s[5:9].view(np.uint32))
    # group independence: perturb group 2 of row 0 only
    xb3 = xb.copy(); xb3[0, 256:384] = xb3[0, 256:384][::-1]
    q3, s3 = oq.act_quant_group(xb3)
    assert np.array_equal(q3[1:], q[1:]) and np.array_equal(q3[0, :256], q[0, :256])
    assert np.array_equal(q3[0, 384:], q[0, 384:])
    # permutation within a group permutes the codes and keeps the scale
    assert np.array_equal(q3[0, 256:384], q[0, 256:384][::-1]) and s3[0, 2] == s[0, 2]
    # power-of-two equivariance (well inside the fp32 range)
    for j in (-5, 7):
        xj = (x * np.float32(2.0 ** j)).astype(np.float32)
        qj, sj = oq.act_quant_group((xj.view(np.uint32) >> 16).astype(np.uint16))
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))


def pin_roundtrip_bound(seed=19):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, s = oq.act_quant_group(xb)
    deq = og.dequant_act(q, s)
    sb = np.repeat(s.astype(np.float64), 128, axis=1)
    t = xv / sb
    at = np.maximum(np.abs(t), 1e-300)
    ulp = np.exp2(np.maximum(np.floor(np.log2(at)), -6) - 3)
    bound = sb * (0.5 * ulp + 2.0 ** -24 * np.abs(t)) * (1 + 1e-12)
    assert np.all(np.abs(xv - deq) <= bound)


def pin_weight_blocks(seed=23):
    rng = np.random.default_rng(seed)
    N, K = 576, 384                                      # last block row has 64 rows
    w = (rng.standard_normal((N, K)) * 0.01).astype(np.float32)
    w[520, 300] = 3.0                                    # lives in block (4, 2)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    q, s = oq.weight_block_quant(wb)
    assert q.shape == (N, K) and s.shape == (5, 3)
    assert s[4, 2] == np.float32(3.0) / np.float32(448.0)
    # each block's scale is fl32(max over that block only)
    wv = (wb.astype(np.uint32) << 16).view(np.float32)
    for nb in range(5):
        for kb in range(3):
            blk = wv[nb * 128: min(N, nb * 128 + 128), kb * 128: kb * 128 + 128]
            am = float(np.abs(blk).max())
            assert float(s[nb, kb]) == fl32_of(Fraction(am) / 448)
    # block independence: change one block, only it changes
    wb2 = wb.copy(); wb2[130:140, 0:128] = 0
    q2, s2 = oq.weight_block_quant(wb2)
    mask = np.zeros_like(q, bool); mask[128:256, 0:128] = True
    assert np.array_equal(q2[~mask], q[~mask])
    assert np.array_equal(np.delete(s2.ravel(), 3), np.delete(s.ravel(), 3))
    # a block treated alone gives the same result
    qa, sa = oq.weight_block_quant(wb[512:576, 128:256])
    assert np.array_equal(qa, q[512:576, 128:256]) and sa[0, 0] == s[4, 1]


def pin_zero_groups():
    x = np.zeros((2, 256), np.uint16)
    x[0, 5] = 0x8000
    x[1, 130] = 0x3F80
    q, s = oq.act_quant_group(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert q[0, 5] == 0x80 and q[0, 4] == 0x00
    assert q[1, 130] == 0x7E


# ----------------------------------------------------------------------------
# GEMM pins

def _triple_loop(A, B):
    M, K = A.shape
    N = B.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += A[m, k] * B[n, k]
            y[m, n] = acc
    return y


def _e4m3_int_codes(rng, shape):
    """Codes of small integers |c| <= 16 (all exactly representable)."""
    ints = rng.integers(-16, 17, size=shape)
    codes = oe.encode(ints.astype(np.float32))
    return ints, codes


def pin_gemm_exact_integers(seed=29):
    """Integer-valued operands with power-of-two scales: the exact result is
    an integer sum, computed here with Python integers."""
    rng = np.random.default_rng(seed)
    M, N, K = 9, 131, 384
    xi, xq = _e4m3_int_codes(rng, (M, K))
    wi, wq = _e4m3_int_codes(rng, (N, K))
    xs = np.exp2(rng.integers(-4, 5, (M, K // 128))).astype(np.float32)
    ws = np.exp2(rng.integers(-4, 5, (2, K // 128))).astype(np.float32)
    y = og.block_gemm(xq, xs, wq, ws)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(K // 128):
                part = int(np.dot(xi[m, kb * 128:(kb + 1) * 128].astype(object),
                                  wi[n, kb * 128:(kb + 1) * 128].astype(object)))
                tot += part * Fraction(float(xs[m, kb])) * Fraction(float(ws[n // 128, kb]))
            assert y[m, n] == float(tot), (m, n, y[m, n], float(tot))


def pin_gemm_scale_indexing(seed=31):
    """All codes 1.0 and distinct powers of two as scales: y = 128*sum_kb
    x_s[m,kb]*W_s[nb,kb], so a wrong or transposed scale index shows."""
    rng = np.random.default_rng(seed)
    M, N, K = 5, 300, 640
    KB, NB = K // 128, 3
    xq = np.full((M, K), 0x38, np.uint8)
    wq = np.full((N, K), 0x38, np.uint8)
    xs = np.exp2(rng.permutation(np.arange(M * KB)).reshape(M, KB) - 12).astype(np.float32)
    ws = np.exp2(rng.permutation(np.arange(NB * KB)).reshape(NB, KB) - 3).astype(np.float32)
    y = og.block_gemm(xq, xs, wq, ws)
    for m in range(M):
        for n in range(N):
            want = 128 * sum(float(xs[m, kb]) * float(ws[n // 128, kb]) for kb in range(KB))
            assert y[m, n] == want


def pin_gemm_brute_force(seed=37):
    import synth
    x, w = synth.tiny_inputs()
    rng = np.random.default_rng(seed)
    cases = [(x[:, :], w[:, :]), (x[:3, :128], w[:128, :128])]
    # N = 576-style partial block: take 64 extra rows
    w576 = synth.normal_bf16(seed, (192, 256), 0.01)
    cases.append((x[:4, :256], w576))
    for xb, wb in cases:
        xq, xs = oq.act_quant_group(xb)
        wq, wsc = oq.weight_block_quant(wb)
        y = og.block_gemm(xq, xs, wq, wsc)
        A = og.dequant_act(xq, xs)
        B = og.dequant_weight(wq, wsc)
        # dequantization entries are exact products of code value and scale
        assert np.all(A == oe.decode(xq) * np.repeat(xs.astype(np.float64), 128, axis=1))
        sub = (slice(0, 3), slice(0, 40)) if xb.shape[1] == 512 else (slice(None), slice(None))
        yt = _triple_loop(A[sub[0]], B[sub[1]])
        np.testing.assert_allclose(y[sub], yt, rtol=1e-12, atol=1e-12 * np.abs(yt).max())
        # the in-loop promotion form gives the same numbers
        KB = xb.shape[1] // 128
        y2 = np.zeros_like(y)
        dx, dw = oe.decode(xq), oe.decode(wq)
        for kb in range(KB):
            ks = slice(kb * 128, kb * 128 + 128)
            part = dx[:, ks] @ dw[:, ks].T
            scale = xs[:, kb][:, None].astype(np.float64) * np.repeat(wsc[:, kb].astype(np.float64), 128)[None, :wb.shape[0]]
            y2 += part * scale
        np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def pin_bf16_rounding(seed=41):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000))
    # add exact ties: bf16 value + half its ulp
    base = np.array([1.0, 3.0, 1.5 + 2 ** -7, -2.0 - 2 ** -6], np.float64)
    ties = base + np.sign(base) * np.exp2(np.floor(np.log2(np.abs(base))) - 8)
    v = np.concatenate([v, ties, base, [0.0, -0.0]])
    bits = og.bf16_rne_bits(v)
    for vi, b in zip(v, bits):
        # neighbours of vi among bf16 values: brute force via the fp32 grid
        f = Fraction(float(vi))
        got = Fraction(bf16_value(int(b)))
        lo_bits = int(b) & 0x7FFF
        for nb in (lo_bits - 1, lo_bits + 1):
            if 0 <= nb < 0x7F80:
                other = Fraction(bf16_value(nb)) * (-1 if (int(b) >> 15) else 1)
                assert abs(got - f) <= abs(other - f), (vi, hex(b))
                if abs(got - f) == abs(other - f):
                    assert (int(b) & 1) == 0, (vi, hex(b))
        if vi == 0:
            assert (int(b) >> 15) == (1 if math.copysign(1, vi) < 0 else 0)
    exp = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82, -3.0: 0xC040}
    for k, want in exp.items():
        assert int(og.bf16_rne_bits(np.array([k]))[0]) == want, k


def pin_grouped(seed=43):
    import synth
    rng = np.random.default_rng(seed)
    E, N, K = 5, 160, 256
    off = synth.random_offsets(0, E, sizes=[0, 3, 17, 1, 0])
    total = int(off[-1])
    xb = synth.normal_bf16(seed, (total, K))
    wb = synth.normal_bf16(seed + 1, (E, N, K), 0.02)
    xq, xs = oq.act_quant_group(xb)
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, 2, 2), np.float32)
    for e in range(E):
        wq[e], ws[e] = oq.weight_block_quant(wb[e])
    y = og.grouped_block_gemm(xq, xs, wq, ws, off)
    # independent route: each row finds its expert by search over offsets
    A = og.dequant_act(xq, xs)
    for r in range(total):
        e = int(np.searchsorted(off, r, side="right") - 1)
        want = A[r] @ og.dequant_weight(wq[e], ws[e]).T
        np.testing.assert_allclose(y[r], want, rtol=1e-13, atol=1e-13)
    # one expert owning every row is the plain GEMM
    y1 = og.grouped_block_gemm(xq, xs, wq[2:3], ws[2:3], np.array([0, total], np.int32))
    np.testing.assert_array_equal(y1, og.block_gemm(xq, xs, wq[2], ws[2]))


def pin_tolerance_report(seed=47):
    import synth
    x, w = synth.tiny_inputs()
    xq, xs = oq.act_quant_group(x)
    wq, ws = oq.weight_block_quant(w)
    y = og.block_gemm(xq, xs, wq, ws)
    S = og.term_magnitude(xq, xs, wq, ws)
    # S bounds |y| and equals it when every term has the same sign
    assert np.all(S >= np.abs(y) * (1 - 1e-12))
    one = np.full((1, 128), 0x38, np.uint8)
    assert og.term_magnitude(one, np.ones((1, 1), np.float32), one, np.ones((1, 1), np.float32))[0, 0] == 128
    rep = og.tolerance_report(og.bf16_rne_bits(y), y, S)
    assert rep["ok"] and rep["bitwise_equal_frac"] == 1.0 and rep["rel_frob"] < 2e-3
    # dropping one K block must fail
    xs_drop = xs.copy(); xs_drop[:, 1] = 0
    assert not og.tolerance_report(og.bf16_rne_bits(og.block_gemm(xq, xs_drop, wq, ws)), y, S)["ok"]
    # a sign flip of the largest output must fail
    yb = og.bf16_rne_bits(y)
    i, j = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    yb[i, j] ^= 0x8000
    assert not og.tolerance_report(yb, y, S)["ok"]
    # an error of 3% on the output with the largest |y|/S must fail
    yb = og.bf16_rne_bits(y)
    i, j = np.unravel_index(np.argmax(np.abs(y) / S), y.shape)
    yb[i, j] = og.bf16_rne_bits(np.array([y[i, j] * 1.03]))[0]
    assert not og.tolerance_report(yb, y, S)["ok"]
    # on the output that cancels most, an error of 2^-12 S must fail and
    # one of 2^-14 S must pass (the allowance is 2^-13 S)
    i, j = np.unravel_index(np.argmin(np.abs(y) / S), y.shape)
    for err, ok in ((2.0 ** -12, False), (2.0 ** -14, True)):
        yt = y.copy()
        yt[i, j] += err * S[i, j]
        yb = og.bf16_rne_bits(yt)
        assert og.tolerance_report(yb, y, S)["ok"] == ok, (err, ok)
    # with the sum exact, the report's S-relative error beyond bf16 is zero
    assert og.tolerance_report(og.bf16_rne_bits(y), y, S)["acc_err_over_S"] == 0.0


# ----------------------------------------------------------------------------
# UE8M0 (power-of-two scale) pins

def pin_e8m0_codec():
    """Byte b is 2^(b-127) for b in [0, 254], NaN for 0xff (no zero)."""
    got = ou.e8m0_decode(np.arange(256, dtype=np.uint8))
    for b in range(255):
        assert Fraction(float(got[b])) == Fraction(2) ** (b - 127), (b, got[b])
    assert math.isnan(got[255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def _e_brute(amax: Fraction) -> int:
    e = -127
    while amax > 448 * Fraction(2) ** e:
        e += 1
    return e


def pin_e8m0_exponent_exhaustive():
    """Every non-negative finite bf16 amax: e is the smallest integer >= -127
    with amax <= 448 * 2^e (walked up from -127 in exact rationals)."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    got = ou.e8m0_exponent(amax)
    # the brute force walk is quadratic; check the binade edges exhaustively
    # and every value through a monotone sweep
    e = -127
    for i, a in enumerate(amax):
        fa = f32_value(int(bits[i]) << 16)
        while fa > 448 * Fraction(2) ** e:
            e += 1
        assert got[i] == e, (hex(int(bits[i])), int(got[i]), e)
        if i % 4096 == 0:
            assert _e_brute(fa) == e
    # fp32 amax values at and just around the edges 448 * 2^j: the edge
    # itself and the value just below it take e = j, the value just above j+1
    for j in (-126, -100, -3, 0, 1, 60, 119):
        edge = np.float32(448.0 * 2.0 ** j)
        above = np.nextafter(edge, np.float32(np.inf))
        below = np.nextafter(edge, np.float32(0))
        assert int(ou.e8m0_exponent(edge)) == j
        assert int(ou.e8m0_exponent(below)) == j
        assert int(ou.e8m0_exponent(above)) == j + 1
    assert int(ou.e8m0_exponent(np.float32(448.0 * 2.0 ** -127))) == -127
    assert int(ou.e8m0_exponent(np.float32(2.0 ** -149))) == -127


def pin_ue8m0_hand_groups():
    for row in read_golden("ue8m0_hand_groups.txt"):
        amax_s, xs_s, b_s, q_s = [p.strip() for p in row.split("|")]
        xb = np.array([int(v, 16) for v in xs_s.split()], np.uint16)
        want_q = [int(v, 16) for v in q_s.split()]
        row128 = np.zeros((1, 128), np.uint16)
        row128[0, : len(xb)] = xb
        q, b = ou.act_quant_group_ue8m0(row128)
        assert int(b[0, 0]) == int(b_s, 16), (amax_s, hex(int(b[0, 0])), b_s)
        assert list(q[0, : len(xb)]) == want_q, (amax_s, [hex(c) for c in q[0, : len(xb)]], q_s)
        blk = np.zeros((130, 128), np.uint16)          # ragged: a 2-row second block row
        blk[129, : len(xb)] = xb
        wq, wb = ou.weight_block_quant_ue8m0(blk)
        assert wb.shape == (2, 1) and int(wb[1, 0]) == int(b_s, 16) and int(wb[0, 0]) == 0
        assert list(wq[129, : len(xb)]) == want_q


def pin_ue8m0_invariants(seed=53):
    rng = np.random.default_rng(seed)
    M, K = 32, 512
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-60, 60, (M, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, b = ou.act_quant_group_ue8m0(xb)
    assert q.shape == (M, K) and b.shape == (M, K // 128) and b.dtype == np.uint8
    assert not np.any((q & 0x7F) == 0x7F), "NaN code produced"
    s = np.exp2(b.astype(np.float64) - 127)
    amax = np.abs(xv.reshape(M, K // 128, 128)).max(axis=2)
    ratio = amax / s
    assert np.all(ratio <= 448) and np.all((ratio > 224) | (b == 0))
    # the quotient is exact, so dequantization errs by at most half a quantum
    t = xv / np.repeat(s, 128, axis=1)
    at = np.maximum(np.abs(t), 1e-300)
    ulp = np.exp2(np.maximum(np.floor(np.log2(at)), -6) - 3)
    deq = oe.decode(q) * np.repeat(s, 128, axis=1)
    assert np.all(np.abs(xv - deq) <= 0.5 * ulp * np.repeat(s, 128, axis=1))
    # same codes as the fp32-scale map on the exact quotient
    assert np.array_equal(q, oe.encode(t.astype(np.float32)))
    # power-of-two equivariance: the codes stay, the bytes shift by j
    for j in (-9, 4):
        xj = (xv * 2.0 ** j).astype(np.float32)
        qj, bj = ou.act_quant_group_ue8m0((xj.view(np.uint32) >> 16).astype(np.uint16))
        assert np.array_equal(qj, q) and np.array_equal(bj.astype(int), b.astype(int) + j)
    # token independence
    q2, b2 = ou.act_quant_group_ue8m0(xb[7:11])
    assert np.array_equal(q2, q[7:11]) and np.array_equal(b2, b[7:11])
    # exact on representable values: x = c * 2^j with amax = 448 * 2^j
    codes, vals = e4m3_finite_table()
    pick = rng.choice(len(codes), 127)
    xr = np.array([448.0] + [math.copysign(float(vals[i]), -1.0 if codes[i] >> 7 else 1.0) for i in pick])
    for j in (-30, 0, 17):
        xe = (xr * 2.0 ** j).astype(np.float32)
        qe, be = ou.act_quant_group_ue8m0((xe.view(np.uint32) >> 16).astype(np.uint16)[None, :])
        assert int(be[0, 0]) == 127 + j and list(qe[0, 1:]) == [codes[i] for i in pick]


def pin_ue8m0_weight_blocks(seed=59):
    rng = np.random.default_rng(seed)
    N, K = 300, 384                                      # last block row has 44 rows
    w = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-8, 8, (N, 1)))).astype(np.float32)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    q, b = ou.weight_block_quant_ue8m0(wb)
    assert q.shape == (N, K) and b.shape == (3, 3)
    wv = (wb.astype(np.uint32) << 16).view(np.float32)
    for nb in range(3):
        for kb in range(3):
            blk = wv[nb * 128: min(N, nb * 128 + 128), kb * 128: kb * 128 + 128]
            e = _e_brute(Fraction(float(np.abs(blk).max())))
            assert int(b[nb, kb]) == e + 127, (nb, kb)
            want = oe.encode((blk.astype(np.float64) * 2.0 ** -e).astype(np.float32))
            assert np.array_equal(q[nb * 128: min(N, nb * 128 + 128), kb * 128: kb * 128 + 128], want)


def pin_ue8m0_gemm(seed=61):
    """With power-of-two scales every dequantized entry is a dyadic rational:
    the exact dot products (rational arithmetic) match the fp64 result."""
    import synth
    x = synth.normal_bf16(seed, (3, 256))
    w = synth.normal_bf16(seed + 1, (130, 256), 0.02)
    w[128:] = synth.normal_bf16(seed + 2, (2, 256), 0.5)   # block row 1: other exponents
    xq, xe = ou.act_quant_group_ue8m0(x)
    wq, we = ou.weight_block_quant_ue8m0(w)
    y = ou.block_gemm_ue8m0(xq, xe, wq, we)
    dx = [[Fraction(float(v)) for v in r] for r in oe.decode(xq)]
    dw = [[Fraction(float(v)) for v in r] for r in oe.decode(wq)]
    for m in range(3):
        for n in (0, 1, 77, 127, 128, 129):
            acc = Fraction(0)
            for k in range(256):
                sx = Fraction(2) ** (int(xe[m, k // 128]) - 127)
                sw = Fraction(2) ** (int(we[n // 128, k // 128]) - 127)
                acc += dx[m][k] * sx * dw[n][k] * sw
            assert abs(Fraction(float(y[m, n])) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000), (m, n)
    S = ou.term_magnitude_ue8m0(xq, xe, wq, we)
    assert np.all(S >= np.abs(y) * (1 - 1e-12))
    # grouped: two experts split the rows
    wq2 = np.stack([wq, wq[::-1].copy()]); we2 = np.stack([we, we[::-1].copy()])
    off = np.array([0, 1, 3], np.int32)
    assert np.all(we[0] != we[1])
    yg = ou.grouped_block_gemm_ue8m0(xq, xe, wq2, we2, off)
    np.testing.assert_array_equal(yg[0], y[0])
    np.testing.assert_array_equal(yg[1:], ou.block_gemm_ue8m0(xq[1:], xe[1:], wq2[1], we2[1]))


# ----------------------------------------------------------------------------
# static activation quantization pins

def pin_static_hand_cases():
    for row in read_golden("static_hand_cases.txt"):
        s_s, xs_s, q_s = [p.strip() for p in row.split("|")]
        scale = np.array([int(s_s, 16)], np.uint32).view(np.float32)[0]
        xb = np.array([[int(v, 16) for v in xs_s.split()]], np.uint16)
        # pad K to 128 (the quantizer is element-wise; K is free here)
        x = np.zeros((1, 128), np.uint16); x[0, : xb.shape[1]] = xb
        q = ost.act_quant_static(x, scale)
        want = [int(v, 16) for v in q_s.split()]
        assert list(q[0, : xb.shape[1]]) == want, (s_s, [hex(c) for c in q[0, : xb.shape[1]]], q_s)
        assert np.all(q[0, xb.shape[1]:] == 0)


def pin_static_brute_force(n=1500, seed=67):
    """Random bf16 x and fp32 scales over a wide range: the code is the
    nearest E4M3 value (ties to even) to the exactly rounded, saturated
    quotient, found by exhaustive search over the 254 finite values."""
    rng = np.random.default_rng(seed)
    xb = rng.integers(0, 0x7F80, n).astype(np.uint32) | (rng.integers(0, 2, n).astype(np.uint32) << 15)
    sb = (rng.integers(0x00800000, 0x7F000000, n)).astype(np.uint32)      # positive normal fp32
    sb[:20] = np.array([0x3F800000 + (i << 23) for i in range(-10, 10)], np.uint32)  # powers of two
    x = np.zeros((1, 128), np.uint16)
    for i in range(n):
        x[0, 0] = xb[i]
        scale = np.array([sb[i]], np.uint32).view(np.float32)[0]
        got = int(ost.act_quant_static(x, scale)[0, 0])
        t = fl32_of(f32_value(int(xb[i]) << 16) / f32_value(int(sb[i])))
        t = max(-448.0, min(448.0, t)) if math.isfinite(t) else math.copysign(448.0, t)
        if t == 0.0:
            want = 0x80 if (xb[i] >> 15) else 0x00
        else:
            want = brute_force_encode(t)
        assert got == want, (hex(int(xb[i])), hex(int(sb[i])), hex(got), hex(want))


def pin_static_invariants(seed=71):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((16, 256)) * 40).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = (xb.astype(np.uint32) << 16).view(np.float32)
    for j in (-3, 0, 2):
        q = ost.act_quant_static(xb, np.float32(2.0 ** j))
        # a power-of-two scale divides exactly: the fp32 map on x * 2^-j
        assert np.array_equal(q, oe.encode(np.clip(xv * np.float32(2.0 ** -j), -448, 448)))
    q = ost.act_quant_static(xb, np.float32(0.37))
    qn = ost.act_quant_static(((xb.astype(np.uint32) ^ 0x8000)).astype(np.uint16), np.float32(0.37))
    assert np.array_equal(qn, q ^ 0x80), "sign symmetry"
    d = oe.decode(q)
    order = np.argsort(xv.ravel(), kind="stable")
    assert np.all(np.diff(d.ravel()[order]) >= 0), "monotone in x"
    assert not np.any((q & 0x7F) == 0x7F)


def pin_static_gemm(seed=73):
    """Integer codes, a power-of-two activation scale and power-of-two weight
    scales: the fp64 result equals the exact integer sum."""
    rng = np.random.default_rng(seed)
    M, N, K = 5, 130, 256
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    ws = np.exp2(rng.integers(-2, 3, (2, 2))).astype(np.float32)
    y = ost.block_gemm_static(xq, np.float32(0.25), wq, ws)
    for m in range(M):
        for n in (0, 64, 127, 128, 129):
            want = sum(Fraction(int(xi[m, k]) * int(wi[n, k])) * Fraction(float(ws[n // 128, k // 128]))
                       for k in range(K)) * Fraction(1, 4)
            assert Fraction(float(y[m, n])) == want, (m, n)
    assert np.all(ost.term_magnitude_static(xq, 0.25, wq, ws) >= np.abs(y))


# ----------------------------------------------------------------------------
# batched expert layout and row-wise ("fp8r") scale pins

def pin_batched(seed=79):
    """The batched layout is the grouped GEMM on each expert's first
    count[e] rows; counts clamp to [0, C]; rows past the count are NaN."""
    import synth
    E, C, N, K = 4, 20, 160, 256
    counts = np.array([0, 7, 20, 33], np.int32)          # 33 clamps to 20
    x = synth.normal_bf16(seed, (E * C, K))
    xq, xs = oq.act_quant_group(x)
    xq, xs = xq.reshape(E, C, K), xs.reshape(E, C, K // 128)
    wq = np.empty((E, N, K), np.uint8); ws = np.empty((E, 2, 2), np.float32)
    for e in range(E):
        wq[e], ws[e] = oq.weight_block_quant(synth.normal_bf16(seed + 1 + e, (N, K), 0.02))
    y = olay.batched_block_gemm(xq, xs, wq, ws, counts)
    used = [min(max(int(c), 0), C) for c in counts]
    off = np.concatenate([[0], np.cumsum(used)]).astype(np.int32)
    packed_q = np.concatenate([xq[e, :used[e]] for e in range(E)])
    packed_s = np.concatenate([xs[e, :used[e]] for e in range(E)])
    yg = og.grouped_block_gemm(packed_q, packed_s, wq, ws, off)
    for e in range(E):
        np.testing.assert_array_equal(y[e, :used[e]], yg[off[e]:off[e + 1]])
        assert np.all(np.isnan(y[e, used[e]:]))
    # a negative count is an empty expert
    y2 = olay.batched_block_gemm(xq, xs, wq, ws, np.array([-3, 1, 1, 1], np.int32))
    assert np.all(np.isnan(y2[0]))
    np.testing.assert_allclose(y2[1, :1], y[1, :1], rtol=1e-13, atol=0)   # BLAS blocking may differ


def pin_rowwise_quant(seed=83):
    rng = np.random.default_rng(seed)
    R, K = 40, 384
    v = (rng.standard_normal((R, K)) * np.exp2(rng.integers(-20, 20, (R, 1)))).astype(np.float32)
    v[3] = 0.0
    v[4, 300] = 1e3                                      # amax in the last 128-group
    vb = (v.view(np.uint32) >> 16).astype(np.uint16)
    q, s = olay.rowwise_quant(vb)
    assert q.shape == (R, K) and s.shape == (R,)
    vv = (vb.astype(np.uint32) << 16).view(np.float32)
    for r in range(R):
        am = float(np.abs(vv[r]).max())
        assert float(s[r]) == fl32_of(Fraction(am) / 448), r
    assert s[3] == 0 and np.all((q[3] & 0x7F) == 0)
    assert np.all(np.any((q.reshape(R, K) & 0x7F) == 0x7E, axis=1) | (s == 0))
    # every row is quantized on its own
    q2, s2 = olay.rowwise_quant(vb[10:13])
    assert np.array_equal(q2, q[10:13]) and np.array_equal(s2, s[10:13])
    # with K = 128 a row is one group: the group quantizer gives the same codes
    qg, sg = oq.act_quant_group(vb[:, :128])
    qr, sr = olay.rowwise_quant(vb[:, :128])
    assert np.array_equal(qg, qr) and np.array_equal(sg[:, 0].view(np.uint32), sr.view(np.uint32))


def pin_rowwise_gemm(seed=89):
    rng = np.random.default_rng(seed)
    M, N, K = 3, 5, 256
    xi = rng.integers(-8, 9, (M, K)); wi = rng.integers(-8, 9, (N, K))
    xq = oe.encode(xi.astype(np.float32)); wq = oe.encode(wi.astype(np.float32))
    xs = np.exp2(rng.integers(-3, 4, M)).astype(np.float32)
    ws = np.exp2(rng.integers(-3, 4, N)).astype(np.float32)
    y = olay.rowwise_gemm(xq, xs, wq, ws)
    for m in range(M):
        for n in range(N):
            want = sum(int(xi[m, k]) * int(wi[n, k]) for k in range(K)) * Fraction(float(xs[m])) * Fraction(float(ws[n]))
            assert Fraction(float(y[m, n])) == want, (m, n)
    assert np.all(olay.rowwise_term_magnitude(xq, xs, wq, ws) >= np.abs(y))


# ----------------------------------------------------------------------------
# SwiGLU + activation quantizer pins

def bf16_rne_exact(q: Fraction, zero_sign: int):
    """Round an exact rational to bf16 bits (nearest, ties to even,
    subnormals kept; finite results only).  Returns (bits, distance of the
    scaled value from the nearest rounding midpoint, in quanta)."""
    if q == 0:
        return (0x8000 if zero_sign < 0 else 0), Fraction(1, 2)
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    qexp = max(e, -126) - 7                      # bf16 quantum of a's binade
    scaled = a / Fraction(2) ** qexp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    dist = abs(rem - Fraction(1, 2))
    if n == 0:
        return sign, dist
    # n * 2^qexp with n < 2^9: exponent and mantissa fields
    if n >= 256:                                 # carried into the next binade
        n //= 2
        qexp += 1
    if n < 128:                                  # subnormal (qexp == -133)
        return sign | n, dist
    field = qexp + 7 + 127
    assert field < 255, "overflow is outside the contract"
    return sign | (field << 7) | (n - 128), dist


def swiglu_exact(g: float, u: float) -> Fraction:
    """SiLU(g) * u to 80 significant digits (decimal arithmetic, no binary
    floating point), as an exact rational of that decimal."""
    with localcontext() as ctx:
        ctx.prec = 80
        dg, du = Decimal(g), Decimal(u)          # exact conversions
        h = dg / (1 + (-dg).exp()) * du
    return Fraction(h)


def pin_swiglu_hand_cases():
    rows = read_golden("swiglu_hand_cases.txt")
    I = 128
    gu = np.zeros((len(rows), 2 * I), np.uint16)
    want = []
    for i, row in enumerate(rows):
        g_s, u_s, h_s = [p.strip() for p in row.split("|")]
        gu[i, 0], gu[i, I] = int(g_s, 16), int(u_s, 16)
        want.append(int(h_s, 16))
    h = osw.swiglu_bf16(gu)
    for i, w in enumerate(want):
        assert int(h[i, 0]) == w, (rows[i], hex(int(h[i, 0])))
    assert np.all(h[:, 1:] == 0)                 # g = u = +0 elsewhere: h = +0


def _random_gate_up(rng, M, I):
    """bf16 gate values over a wide range (typical N(0, 3) mixed with
    +-2^[-30, 12) and a few specials) and up values +-2^[-60, 60)."""
    g = rng.standard_normal((M, I)) * 3
    wide = rng.random((M, I)) < 0.5
    g = np.where(wide, np.sign(g) * np.exp2(rng.uniform(-30, 12, (M, I))), g)
    u = np.sign(rng.standard_normal((M, I))) * np.exp2(rng.uniform(-60, 60, (M, I)))
    flat = g.reshape(-1)
    specials = [0.0, -0.0, -800.0, -500.0, 1e-40, -1e-40, 37.0, 48.0, -37.0]
    flat[: len(specials)] = specials
    gb = (g.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ub = (u.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.concatenate([gb, ub], axis=1)


def pin_swiglu_brute_force(seed=97):
    """Every h of a [3, 2*256] gate/up block against the exact SiLU(g) * u
    (80-digit decimal) rounded to bf16 by an integer rule; g is read from
    column j and u from column I + j.  Values within 2^-40 of a rounding
    midpoint (in quanta) are where binary64 evaluation may round differently
    from the exact value (hand case (6)); they are counted, not compared."""
    rng = np.random.default_rng(seed)
    M, I = 3, 256
    gu = _random_gate_up(rng, M, I)
    h = osw.swiglu_bf16(gu)
    assert h.shape == (M, I)
    near = 0
    for m in range(M):
        for j in range(I):
            g = bf16_value(int(gu[m, j])); u = bf16_value(int(gu[m, I + j]))
            zs = int(math.copysign(1, g) * math.copysign(1, u))
            want, dist = bf16_rne_exact(swiglu_exact(g, u), zs)
            if dist < Fraction(1, 2 ** 40):
                near += 1
                continue
            assert int(h[m, j]) == want, (m, j, g, u, hex(int(h[m, j])), hex(want))
    assert near < 8, near


def pin_swiglu_quant(seed=101):
    """The quantizer runs on the bf16-rounded h: every scale is
    fl32(amax(h) / 448) and every code the nearest E4M3 value (exhaustive
    search) to fl32(h / s), with h taken from the exact SiLU(g) * u."""
    rng = np.random.default_rng(seed)
    M, I = 2, 256
    gu = _random_gate_up(rng, M, I)
    gu[:, :I] = (((rng.standard_normal((M, I)) * 3).astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)
    gu[:, I:] = (((rng.standard_normal((M, I))).astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)
    q, s = osw.swiglu_act_quant(gu)
    assert q.shape == (M, I) and s.shape == (M, I // 128)
    for m in range(M):
        hb = []
        for j in range(I):
            g = bf16_value(int(gu[m, j])); u = bf16_value(int(gu[m, I + j]))
            zs = int(math.copysign(1, g) * math.copysign(1, u))
            hb.append(bf16_rne_exact(swiglu_exact(g, u), zs)[0])
        for grp in range(I // 128):
            vals = [Fraction(bf16_value(b)) for b in hb[128 * grp: 128 * grp + 128]]
            amax = max(abs(v) for v in vals)
            sc = fl32_of(amax / 448)
            assert float(s[m, grp]) == sc, (m, grp)
            for k in range(0, 128, 7):
                t = fl32_of(vals[k] / Fraction(sc))
                want = brute_force_encode(t) if t != 0 else (0x80 if hb[128 * grp + k] >> 15 else 0)
                assert int(q[m, 128 * grp + k]) == want, (m, grp, k)



def pin_swiglu_quant_ue8m0(seed=103):
    """Power-of-two scales on the same h: every byte is 127 + e with e the
    smallest integer >= -127 such that amax(h) <= 448 * 2^e (exact
    rationals), and every code the nearest E4M3 value (exhaustive search) to
    the exact quotient h / 2^e."""
    rng = np.random.default_rng(seed)
    M, I = 2, 256
    gu = np.concatenate([
        (((rng.standard_normal((M, I)) * 3).astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16),
        (((rng.standard_normal((M, I))).astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)], axis=1)
    q, b = osw.swiglu_act_quant_ue8m0(gu)
    assert q.shape == (M, I) and b.shape == (M, I // 128) and b.dtype == np.uint8
    for m in range(M):
        hb = []
        for j in range(I):
            g = bf16_value(int(gu[m, j])); u = bf16_value(int(gu[m, I + j]))
            zs = int(math.copysign(1, g) * math.copysign(1, u))
            hb.append(bf16_rne_exact(swiglu_exact(g, u), zs)[0])
        for grp in range(I // 128):
            vals = [Fraction(bf16_value(x)) for x in hb[128 * grp: 128 * grp + 128]]
            amax = max(abs(v) for v in vals)
            e = -127
            while amax > 448 * Fraction(2) ** e:
                e += 1
            assert int(b[m, grp]) == e + 127, (m, grp)
            for k in range(0, 128, 7):
                t = vals[k] / Fraction(2) ** e
                want = brute_force_encode(float(t)) if t != 0 else (0x80 if hb[128 * grp + k] >> 15 else 0)
                assert int(q[m, 128 * grp + k]) == want, (m, grp, k)


ALL_PINS = [
    pin_format_points, pin_hand_encodings, pin_decode_matches_enumeration,
    pin_encode_roundtrip_and_monotone, pin_encode_brute_force, pin_fl32_div,
    pin_hand_groups, pin_quant_ties, pin_scale_is_fl32_amax_over_448, pin_exact_on_representable,
    pin_group_invariants, pin_roundtrip_bound, pin_weight_blocks, pin_zero_groups,
    pin_gemm_exact_integers, pin_gemm_scale_indexing, pin_gemm_brute_force,
    pin_bf16_rounding, pin_grouped, pin_tolerance_report,
    pin_e8m0_codec, pin_e8m0_exponent_exhaustive, pin_ue8m0_hand_groups,
    pin_ue8m0_invariants, pin_ue8m0_weight_blocks, pin_ue8m0_gemm,
    pin_static_hand_cases, pin_static_brute_force, pin_static_invariants, pin_static_gemm,
    pin_batched, pin_rowwise_quant, pin_rowwise_gemm,
    pin_swiglu_hand_cases, pin_swiglu_brute_force, pin_swiglu_quant, pin_swiglu_quant_ue8m0,
]
