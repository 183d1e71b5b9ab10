"""The CPU oracle against its pins (format points, hand-worked cases, exact
arithmetic, brute force, invariants) -- no GPU involved."""
import numpy as np
import pytest

import oracle_pins as P
from oracle import e4m3 as oe


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_codec_agrees_with_torch_float8_e4m3fn():
    """torch's float8_e4m3fn (CPU) implements the same OCP format: decode of
    all 256 codes, and RNE encode on values inside +-448."""
    torch = pytest.importorskip("torch")
    c = np.arange(256, dtype=np.uint8)
    d = oe.decode(c)
    t = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.all((d == t) | (np.isnan(d) & np.isnan(t)))
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(400000) * np.exp2(rng.integers(-14, 9, 400000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oe.encode(x), want)


def test_e8m0_decode_agrees_with_torch_float8_e8m0fnu():
    """torch's float8_e8m0fnu (CPU) decodes the same OCP MX scale type."""
    torch = pytest.importorskip("torch")
    from oracle import ue8m0 as ou
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("torch lacks float8_e8m0fnu")
    b = np.arange(256, dtype=np.uint8)
    d = ou.e8m0_decode(b)
    t = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).double().numpy()
    assert np.all((d == t) | (np.isnan(d) & np.isnan(t)))
