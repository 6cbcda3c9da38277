"""Pins of the oracle's storage codecs against library casts (torch), the
OCP code tables written out from the format definitions, exhaustive round
trips and hand-worked rounding cases.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import codecs as K


# ----------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = K.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0),
])
def test_e4m3_table(code, value):
    assert K.e4m3_decode(np.array([code], np.uint8))[0] == value


def test_e4m3_encode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = K.e4m3_decode(codes)
    back = K.e4m3_encode(vals)
    # -0.0 encodes to 0x80, +0.0 to 0x00
    assert np.array_equal(back, codes)


def test_e4m3_encode_matches_torch_rne_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 150)])
    x = x[np.abs(x) <= 448]
    # add exact midpoints between neighbouring codes
    pos = K.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32).astype(np.float64)
    ours = K.e4m3_decode(K.e4m3_encode(x))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    x = np.array([448.0, 463.9, 464.0, 500.0, 1e9, -1e9, -470.0])
    assert list(K.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_midpoint_goes_to_even():
    # 1.0625 is halfway between 1.0 (0x38, mantissa 0) and 1.125 (0x39, mantissa 1)
    assert K.e4m3_encode(np.array([1.0625]))[0] == 0x38
    # 1.1875 is halfway between 1.125 (m=1) and 1.25 (m=2): goes to 1.25
    assert K.e4m3_encode(np.array([1.1875]))[0] == 0x3A


# ----------------------------------------------------------------- bf16

def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact midpoints between bf16 neighbours
    hi = rng.integers(0, 0x7F7F, 5000).astype(np.uint32)
    mids = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, mids, -mids, np.array([0.0, -0.0, 1e-40], np.float32)])
    ours = K.bf16_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode():
    assert K.bf16_decode(np.array([0x3F80], np.uint16))[0] == 1.0
    assert K.bf16_decode(np.array([0xC040], np.uint16))[0] == -3.0
    assert K.bf16_decode(np.array([0x0001], np.uint16))[0] == 2.0 ** -133


# ----------------------------------------------------------------- E2M1 / E8M0 / MXFP4

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table():
    v = K.e2m1_decode(np.arange(16))
    assert list(v[:8]) == E2M1_TABLE
    assert list(-v[8:]) == E2M1_TABLE
    assert np.signbit(v[8])


@pytest.mark.parametrize("x,val", [
    (0.25, 0.0), (0.26, 0.5), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
    (3.5, 4.0), (5.0, 4.0), (5.1, 6.0), (7.0, 6.0), (100.0, 6.0), (-2.5, -2.0), (-0.1, 0.0),
])
def test_e2m1_rounding(x, val):
    assert K.e2m1_decode(K.e2m1_encode(np.array([x])))[0] == val


def test_e2m1_encode_is_nearest():
    rng = np.random.default_rng(3)
    x = rng.uniform(-6, 6, 10000)
    got = K.e2m1_decode(K.e2m1_encode(x))
    grid = np.array(E2M1_TABLE)
    best = np.min(np.abs(np.abs(x)[:, None] - grid[None, :]), axis=1)
    assert np.allclose(np.abs(np.abs(got) - np.abs(x)), best)
    assert np.all((got == 0) | (np.sign(got) == np.sign(x)))


def test_e8m0_decode():
    v = K.e8m0_decode(np.array([0, 126, 127, 128, 254, 255]))
    assert v[0] == 2.0 ** -127 and v[1] == 0.5 and v[2] == 1.0 and v[3] == 2.0
    assert v[4] == 2.0 ** 127 and np.isnan(v[5])


def test_mxfp4_scale_rule_and_nibble_order():
    x = np.zeros(32)
    x[0], x[1] = 6.0, 0.5            # amax 6 -> floor(log2 6) = 2 -> X = 2**0
    codes, scales = K.mxfp4_encode(x)
    assert scales[0] == 127
    assert codes[0] == (0x7 | (0x1 << 4))
    x[0] = 3.0                        # amax 3 -> X = 2**-1 -> element 6.0
    codes, scales = K.mxfp4_encode(x)
    assert scales[0] == 126 and codes[0] & 0xF == 0x7
    x[0] = 1.5                        # amax 1.5 -> X = 2**-2 -> element 6.0
    codes, scales = K.mxfp4_encode(x)
    assert scales[0] == 125 and codes[0] & 0xF == 0x7 and (codes[0] >> 4) == 0x4   # 0.5/0.25 = 2 -> code 4
    codes, scales = K.mxfp4_encode(np.zeros(64))
    assert list(scales) == [0, 0] and not codes.any()


def test_mxfp4_error_bound_and_round_trip():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((500, 64))
    codes, scales = K.mxfp4_encode(x)
    y = K.mxfp4_decode(codes, scales)
    X = np.repeat(K.e8m0_decode(scales), 32, axis=-1)
    # every element is within half a local E2M1 step (<= 1.0*X) or saturated at 6X
    a = np.abs(x) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    ok = (np.abs(x - y) <= step * X / 2 + 1e-12) | (np.abs(y) == 6 * X)
    assert ok.all()
    c2, s2 = K.mxfp4_encode(y)        # decoded values are fixed points
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_row_layout_fp8_rope_bf16():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 512))
    enc, _ = K.encode_rows(x, K.ROW_FP8_ROPE_BF16)
    assert enc.shape == (4, 576) and enc.dtype == np.uint8
    y = K.decode_rows(enc, K.ROW_FP8_ROPE_BF16, 512)
    assert np.array_equal(y[:, :448], K.e4m3_round(x[:, :448]))
    assert np.array_equal(y[:, 448:], K.bf16_round(x[:, 448:]))


def test_mxfp8_scale_rule_and_codes():
    """OCP MX with E4M3 elements: the shared scale is 2^(floor(log2 amax) - 8),
    so a block maximum of 1.0 is stored as 256 (code 0x78) at scale 2^-8 (code
    119) and 1.75 as 448 (0x7E); values between 1.75 and 2 times a power of two
    saturate to the 448 code; an all-zero block has scale code 0."""
    x = np.zeros(32)
    x[:4] = [1.0, 0.5, -0.25, 1.0 / 3.0]
    codes, scales = K.mxfp8_encode(x)
    assert scales[0] == 119 and codes[0] == 0x78 and codes[1] == 0x70 and codes[2] == 0xE8 and codes[3] == 0x6B
    y = K.mxfp8_decode(codes, scales)
    assert y[0] == 1.0 and y[1] == 0.5 and y[2] == -0.25
    assert y[3] == 0.34375              # 85.33 rounds to 88 on the E4M3 grid (steps of 8 in [64, 128))
    x[0] = 1.75
    codes, scales = K.mxfp8_encode(x)
    assert codes[0] == 0x7E and K.mxfp8_decode(codes, scales)[0] == 1.75
    x[0] = 1.9
    codes, scales = K.mxfp8_encode(x)
    assert codes[0] == 0x7E and K.mxfp8_decode(codes, scales)[0] == 1.75
    codes, scales = K.mxfp8_encode(np.zeros(64))
    assert (scales == 0).all() and (codes == 0).all()


def test_mxfp8_elements_match_torch_and_round_trip():
    """Element codes equal torch's float8_e4m3fn cast of x / scale (the scale is
    a power of two, so the division is exact); the error is at most half an
    E4M3 step outside the saturation band; decoded values are fixed points."""
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 128)) * np.exp(rng.uniform(-6, 6, (6, 1)))
    codes, scales = K.mxfp8_encode(x)
    X = np.repeat(K.e8m0_decode(scales), 32, axis=-1)
    ref = torch.from_numpy((x / X).astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())
    y = K.mxfp8_decode(codes, scales)
    blocks = np.abs(x).reshape(6, 4, 32)
    band = np.repeat((blocks.max(-1) >= 1.75 * 2.0 ** np.floor(np.log2(blocks.max(-1)))), 32, axis=-1).reshape(6, 128)
    small = np.abs(x) < 2.0**-6 * X
    ok = band | small | (np.abs(y - x) <= 2.0**-4 * np.abs(x) * (1 + 1e-12))
    assert ok.all()
    c2, s2 = K.mxfp8_encode(y)
    assert np.array_equal(K.mxfp8_decode(c2, s2), y)
