"""Seeded synthetic inputs for the fine-grained FP8 linear layer.

This module only draws random numbers and lays them out; it holds none of
the quantization or matrix arithmetic.  Both the CPU oracle (via the tests
and the bench) and the GPU path consume exactly the bytes produced here.

Every tensor is returned as numpy: bf16 values as uint16 bit patterns
(fp32 draws rounded to nearest-even bf16), expert offsets as int32.

Workloads (shapes are the published projection shapes of the named
models; no weights or datasets are involved):

* ``tiny``       x[16,512], W[512,512], i.i.d. N(0,1).
* ``llama``      Llama-3-8B projections (q/o 4096x4096, kv 1024x4096,
                 gate/up 14336x4096, down 4096x14336); x ~ N(0,1) with 1 %
                 of the input channels scaled by 20; W ~ N(0, 0.02).
* ``dsv3``       DeepSeek-V3 dense projections; x ~ N(0,1) with 0.5 % of
                 entries replaced by 10 * Student-t(3); W ~ N(0, 0.01).
* ``moe``        DeepSeek-V3 MoE share of one device: 32 experts, gate/up
                 4096x7168, down 7168x2048; 4096 tokens routed to 8
                 distinct experts each with Zipf(1.1) popularity.
                 The SwiGLU step between the two projections takes the
                 gate/up output [sum M_e, 2*2048], drawn directly as
                 N(0, 1.34^2): the spread of a 7168-term sum of inputs with
                 mean square ~2.5 (N(0,1) plus the 0.5 % t(3) tail) times
                 N(0, 0.01) weights.

Seeds follow ``1000*config + 10*shape_index + {1: x, 2: W, 3: outliers}``.
"""
from __future__ import annotations

import numpy as np

LLAMA_SHAPES = (  # (name, N, K)
    ("qo", 4096, 4096),
    ("kv", 1024, 4096),
    ("gate_up", 14336, 4096),
    ("down", 4096, 14336),
)

DSV3_SHAPES = (
    ("q_a", 1536, 7168),
    ("q_b", 24576, 1536),
    ("kv_a", 576, 7168),
    ("o_proj", 7168, 16384),
    ("mlp_up", 18432, 7168),
    ("mlp_down", 7168, 18432),
)

MOE_EXPERTS = 32
MOE_TOPK = 8
MOE_TOKENS = 4096
MOE_SHAPES = (("gate_up", 4096, 7168), ("down", 7168, 2048))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 draws to the nearest bf16 (ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def seed_of(config: int, shape_index: int, what: int) -> int:
    return 1000 * config + 10 * shape_index + what


def normal_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def llama_activations(seed: int, M: int, K: int, outlier_seed: int) -> np.ndarray:
    """x ~ N(0,1) with round(0.01*K) channels (same for every token) times 20."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=(M, K), dtype=np.float32)
    n_out = int(round(0.01 * K))
    cols = np.random.default_rng(outlier_seed).choice(K, size=n_out, replace=False)
    a[:, cols] *= np.float32(20.0)
    return f32_to_bf16_bits(a)


def dsv3_activations(seed: int, M: int, K: int, outlier_seed: int) -> np.ndarray:
    """x ~ N(0,1); 0.5 % of entries (i.i.d. positions) become 10 * t(3)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=(M, K), dtype=np.float32)
    orng = np.random.default_rng(outlier_seed)
    mask = orng.random(size=(M, K)) < 0.005
    n = int(mask.sum())
    a[mask] = (10.0 * orng.standard_t(3.0, size=n)).astype(np.float32)
    return f32_to_bf16_bits(a)


def tiny_inputs():
    """x[16,512], W[512,512], both N(0,1)."""
    x = normal_bf16(seed_of(1, 0, 1), (16, 512))
    w = normal_bf16(seed_of(1, 0, 2), (512, 512))
    return x, w


def llama_inputs(shape_index: int, M: int, config: int = 3):
    name, N, K = LLAMA_SHAPES[shape_index]
    x = llama_activations(seed_of(config, shape_index, 1), M, K,
                          seed_of(config, shape_index, 3))
    w = normal_bf16(seed_of(config, shape_index, 2), (N, K), std=0.02)
    return x, w


def llama_weight(shape_index: int, config: int = 3):
    name, N, K = LLAMA_SHAPES[shape_index]
    return normal_bf16(seed_of(config, shape_index, 2), (N, K), std=0.02)


def llama_x(shape_index: int, M: int, config: int = 3, variant: int = 0):
    """Activations for one Llama projection; ``variant`` gives further
    independent batches of the same distribution (buffer rotation)."""
    name, N, K = LLAMA_SHAPES[shape_index]
    return llama_activations(seed_of(config, shape_index, 1) + 100000 * variant, M, K,
                             seed_of(config, shape_index, 3))


def dsv3_inputs(shape_index: int, M: int, config: int = 4):
    name, N, K = DSV3_SHAPES[shape_index]
    x = dsv3_activations(seed_of(config, shape_index, 1), M, K,
                         seed_of(config, shape_index, 3))
    w = normal_bf16(seed_of(config, shape_index, 2), (N, K), std=0.01)
    return x, w


def moe_routing(seed: int = 5000, tokens: int = MOE_TOKENS, experts: int = MOE_EXPERTS,
                topk: int = MOE_TOPK):
    """Each token picks ``topk`` distinct experts, sampled without replacement
    with probability proportional to rank**-1.1 (expert e has rank e+1), via
    Gumbel-top-k.  Returns (token_of_row, expert_offsets) for the rows sorted
    by expert: row r of the grouped matrix is token ``token_of_row[r]``."""
    rng = np.random.default_rng(seed)
    logits = -1.1 * np.log(np.arange(1, experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(tokens, experts)) + logits[None, :]
    choice = np.argsort(-g, axis=1, kind="stable")[:, :topk]  # [tokens, topk]
    tok = np.repeat(np.arange(tokens), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))  # by expert, then token
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return tok[order].astype(np.int64), offsets


def moe_inputs(which: int, config: int = 5, experts: int = MOE_EXPERTS,
               rows: int | None = None, offsets: np.ndarray | None = None):
    """Grouped inputs for projection ``which`` (0 gate/up, 1 down).

    gate/up: the 4096 token rows (drawn like the DeepSeek-V3 dense inputs)
    gathered into expert-sorted order; down: an independent [sum M_e, 2048]
    draw of the same distribution.  Returns (x [sumM,K], w [E,N,K], offsets).
    """
    name, N, K = MOE_SHAPES[which]
    if offsets is None:
        tok, offsets = moe_routing(experts=experts)
    else:
        tok = None
    total = int(offsets[-1]) if rows is None else rows
    if which == 0 and tok is not None:
        base = dsv3_activations(seed_of(config, which, 1), MOE_TOKENS, K,
                                seed_of(config, which, 3))
        x = base[tok]
    else:
        x = dsv3_activations(seed_of(config, which, 1), total, K, seed_of(config, which, 3))
    w = normal_bf16(seed_of(config, which, 2), (experts, N, K), std=0.01)
    return x, w, offsets


MOE_INTERMEDIATE = 2048
MOE_GATE_UP_STD = 1.34


def moe_gate_up_output(seed: int, M: int, I: int = MOE_INTERMEDIATE) -> np.ndarray:
    """Gate/up projection output [M, 2I] (gate columns first) as bf16 bits."""
    return normal_bf16(seed, (M, 2 * I), std=MOE_GATE_UP_STD)


def random_offsets(seed: int, experts: int, sizes=None, max_rows: int = 64):
    """Expert offsets for small grouped tests; ``sizes`` overrides the draw."""
    if sizes is None:
        sizes = np.random.default_rng(seed).integers(0, max_rows + 1, size=experts)
    sizes = np.asarray(sizes, dtype=np.int64)
    off = np.zeros(len(sizes) + 1, dtype=np.int32)
    off[1:] = np.cumsum(sizes)
    return off


# ----------------------------------------------------------------------------
# The exhaustive (x, amax) domain of the element map on bf16 inputs.
#
# For every positive finite bf16 amax a (bit patterns 0x0001..0x7F7F) the
# values are all bf16 x with |x| <= a: bit patterns 0..a and 0x8000..0x8000+a,
# 2(a+1) values, 1,065,402,238 pairs in all.  Each set (an activation group
# of 128, or a weight block of 128x128) holds a itself first, then up to
# 127 (or 16383) of the values, padded with +0, so its amax is exactly a.
# The amax range is cut into chunks of roughly equal element counts.

EXH_AMAX_LO, EXH_AMAX_HI = 0x0001, 0x7F7F


def exhaustive_chunk_bounds(nchunks: int):
    a = np.arange(EXH_AMAX_LO, EXH_AMAX_HI + 1, dtype=np.int64)
    cum = np.cumsum(2 * (a + 1))
    targets = cum[-1] * np.arange(1, nchunks) / nchunks
    cuts = np.searchsorted(cum, targets) + EXH_AMAX_LO
    bounds = [EXH_AMAX_LO, *[int(c) for c in cuts], EXH_AMAX_HI + 1]
    return [(bounds[i], bounds[i + 1]) for i in range(nchunks)]


def _exhaustive_sets(a_lo: int, a_hi: int, set_size: int) -> np.ndarray:
    per = set_size - 1
    out = []
    for a in range(a_lo, a_hi):
        vals = np.concatenate([np.arange(0, a + 1, dtype=np.uint16),
                               np.arange(0x8000, 0x8000 + a + 1, dtype=np.uint16)])
        n = -(-vals.size // per)
        s = np.zeros((n, set_size), dtype=np.uint16)
        s[:, 0] = a
        flat = s[:, 1:].reshape(-1)
        flat[: vals.size] = vals
        s[:, 1:] = flat.reshape(n, per)
        out.append(s)
    return np.concatenate(out) if out else np.zeros((0, set_size), np.uint16)


def exhaustive_act_chunk(a_lo: int, a_hi: int) -> np.ndarray:
    """[G, 128] bf16 bits: one activation group per row (K = 128)."""
    return _exhaustive_sets(a_lo, a_hi, 128)


def exhaustive_weight_chunk(a_lo: int, a_hi: int) -> np.ndarray:
    """[128*B, 128] bf16 bits: B weight blocks of 128x128 stacked by rows."""
    s = _exhaustive_sets(a_lo, a_hi, 128 * 128)
    return s.reshape(-1, 128)
