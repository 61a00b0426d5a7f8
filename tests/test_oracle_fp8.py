"""Pins of the oracle's FP8 payload: the E4M3 code table from the format's
closed forms, the encoder against torch's float8_e4m3fn cast (a library
routine, round-to-nearest-even), and the group quantizer's properties."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def test_e4m3_closed_forms():
    v = O.e4m3_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9                 # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9             # largest subnormal
    assert v(0x08) == 2.0 ** -6                 # smallest normal
    assert v(0x38) == 1.0
    assert v(0x39) == 1.125
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    t = v(np.arange(0x7F))
    assert np.all(np.diff(t) > 0)                 # codes 0..0x7E increase


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(1)
    table = O.e4m3_value(np.arange(0x7F))
    mids = (table[1:] + table[:-1]) / 2          # exact ties, all fp32-representable
    vals = np.concatenate([
        (rng.standard_normal(100000) * 40).clip(-448, 448),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),          # subnormal range
        mids, -mids, table, -table, [0.0, -0.0, 448.0, -448.0, 1e-30, -1e-30],
    ]).astype(np.float32)
    got = O.e4m3_encode(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([449.0]))


def test_quantize_group_properties():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((37, 512)) * rng.uniform(0.01, 100, (37, 1))).astype(np.float32)
    x[3, 128:256] = 0.0                           # an all-zero group
    x[5, :128] = -x[5, :128]
    x[7, 256:384] *= np.float32(1e-32)           # amax below 2^-100: zero codes
    codes, scales = O.quantize_fp8(x)
    assert codes.dtype == np.uint8 and codes.shape == x.shape
    assert scales.dtype == np.float32 and scales.shape == (37, 4)
    g = x.reshape(37, 4, 128)
    amax = np.abs(g).max(2)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    c = codes.reshape(37, 4, 128)
    assert scales[3, 1] == 0 and (c[3, 1] & 0x7F == 0).all()
    assert scales[7, 2] > 0 and (c[7, 2] & 0x7F == 0).all()
    for r in range(37):
        for j in range(4):
            if amax[r, j] >= 2.0 ** -100:         # the group's largest value maps to +-448
                assert (c[r, j] & 0x7F).max() == 0x7E
    # round trip: within half a code step of the scaled value
    back = O.dequantize_fp8(codes, scales).astype(np.float64)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6) + s * 1e-6
    big = np.repeat(amax >= 2.0 ** -100, 128, axis=1)
    assert (np.abs(back - x) <= bound)[big].all()
    assert (back[~big] == 0).all()
    assert np.array_equal(np.sign(back[back != 0]), np.sign(x[back != 0]))


def test_quantize_is_exact_on_representable_groups():
    # values that are e4m3 values times a power of two, with the group's
    # largest magnitude at 448 * 2^k: the scale is exactly 2^k and every
    # value comes back unchanged
    rng = np.random.default_rng(3)
    table = O.e4m3_value(np.arange(0x7F))
    R = 16
    x = rng.choice(table, size=(R, 256)) * rng.choice([-1, 1], size=(R, 256))
    x[:, 0] = 448.0
    x[:, 128] = -448.0
    k = rng.integers(-8, 8, size=(R, 1)).astype(np.float64)
    x = (x * 2.0 ** k).astype(np.float32)
    codes, scales = O.quantize_fp8(x)
    assert np.array_equal(scales, np.repeat((2.0 ** k).astype(np.float32), 2, axis=1))
    assert np.array_equal(O.dequantize_fp8(codes, scales), x)
