"""Oracle-side storage codecs, written in plain numpy float64.

TEST INFRASTRUCTURE ONLY.  This package is the slow reference that the HIP
library is checked against; the library never imports, links or calls it.

The pages fix the storage precisions but not the bit formats:
  * DeepSeek-V4 digest (ai-papers-daily page "DeepSeek-V4: Towards Highly
    Efficient Million-Token Context Intelligence"), 模块 F: the RoPE dims of a
    KV entry are kept in BF16, the other dims in FP8, and the lightning
    indexer runs in FP4.
The formats chosen (and pinned in tests/test_oracle_codecs.py against the
library casts of torch and against exhaustive code tables) are:
  * bf16: IEEE-754 binary32 with the low 16 bits dropped, round-to-nearest-even.
  * fp8:  OCP E4M3 ("e4m3fn"): bias 7, no infinities, 0x7F/0xFF are NaN,
          largest finite 448; encoding rounds to nearest even and saturates.
  * fp4:  OCP E2M1: bias 1, values {0, .5, 1, 1.5, 2, 3, 4, 6}; saturating.
  * e8m0: OCP MX scale, value 2**(E-127), E=255 is NaN.
  * MXFP4 block of 32: shared scale X = 2**(floor(log2(amax)) - 2) (2 is the
    largest exponent of E2M1), elements = E2M1(x / X); amax == 0 gives scale
    code 0 and all-zero elements.
"""
import numpy as np

# --------------------------------------------------------------------------
# generic "round to a binary floating-point format" in float64
# --------------------------------------------------------------------------


def _round_to_format(x, mant_bits, emin, max_finite, saturate):
    """Round float64 values to the nearest value of a binary format with
    `mant_bits` explicit mantissa bits and smallest normal exponent `emin`
    (round half to even, gradual underflow).  Values whose rounded magnitude
    exceeds `max_finite` saturate to it or become inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])           # x = f * 2**e, 0.5 <= |f| < 1
    expo = np.maximum(e - 1, emin)   # exponent of the leading bit, floored at emin
    quantum = np.ldexp(1.0, expo - mant_bits)
    r = np.round(x[nz] / quantum) * quantum   # np.round is half-to-even; exact division
    big = np.abs(r) > max_finite
    if saturate:
        r[big] = np.sign(r[big]) * max_finite
    else:
        r[big] = np.sign(r[big]) * np.inf
    out[nz] = r
    out[~nz] = x[~nz]          # zeros keep their sign; inf and nan pass through
    return out


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_decode(u16):
    u = np.asarray(u16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(x):
    """Value of x rounded to bf16 (RNE, overflow to inf)."""
    return _round_to_format(x, 7, -126, float(np.ldexp(255.0 / 128.0, 127)), False)


def bf16_encode(x):
    """float64 -> bf16 bit patterns (uint16), round to nearest even."""
    r = bf16_round(x).astype(np.float32)   # exact: a bf16 value is a float32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# OCP E4M3
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes):
    b = np.asarray(codes).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    v = s * np.where(e == 0, sub, nor)
    v = np.where((b & 0x7F) == 0x7F, np.nan, v)
    return v


def e4m3_round(x):
    return _round_to_format(x, 3, -6, E4M3_MAX, True)


def e4m3_encode(x):
    """float64 -> E4M3 codes (uint8), RNE, saturating at +-448."""
    r = e4m3_round(x)
    sign = (np.signbit(r)).astype(np.int64) << 7
    a = np.abs(r)
    codes = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    _, e = np.frexp(a[nz])
    expo = e - 1                       # a = 1.f * 2**expo
    normal = expo >= -6
    ef = np.where(normal, expo + 7, 0)
    mant = np.where(normal, a[nz] / np.ldexp(1.0, expo) - 1.0, a[nz] / 2.0 ** -6) * 8.0
    codes[nz] = (ef << 3) | np.rint(mant).astype(np.int64)
    return (codes | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# OCP E2M1, E8M0 and MXFP4 blocks
# --------------------------------------------------------------------------

E2M1_MAX = 6.0


def e2m1_decode(nibbles):
    b = np.asarray(nibbles).astype(np.int64) & 0xF
    s = np.where(b & 0x8, -1.0, 1.0)
    e = (b >> 1) & 0x3
    m = (b & 0x1).astype(np.float64)
    v = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return s * v


def e2m1_round(x):
    return _round_to_format(x, 1, 0, E2M1_MAX, True)


def e2m1_encode(x):
    r = e2m1_round(x)
    sign = np.signbit(r).astype(np.int64) << 3
    a = np.abs(r)
    codes = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    _, e = np.frexp(a[nz])
    expo = e - 1
    normal = expo >= 0
    ef = np.where(normal, expo + 1, 0)
    # normal: a = (1 + m/2) * 2**expo; subnormal: a = m * 0.5
    mant = np.where(normal, (a[nz] / np.ldexp(1.0, expo) - 1.0) * 2.0, a[nz] / 0.5)
    codes[nz] = (ef << 1) | np.rint(mant).astype(np.int64)
    return (codes | sign).astype(np.uint8)


def e8m0_decode(codes):
    E = np.asarray(codes).astype(np.int64)
    return np.where(E == 255, np.nan, np.ldexp(1.0, E - 127))


def mxfp4_encode_block(x):
    """One block of float64 values (last axis = 32) -> (element codes, scale code)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    scale_codes = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, e = np.frexp(amax[nz])
    shared = (e - 1) - 2                     # floor(log2 amax) - emax(E2M1)
    shared = np.clip(shared, -127, 127)
    scale_codes[nz] = shared + 127
    X = np.where(nz, np.ldexp(1.0, scale_codes - 127), 1.0)
    elems = e2m1_encode(x / X[..., None])
    elems[~nz] = 0
    return elems, scale_codes.astype(np.uint8)


def mxfp4_encode(x):
    """[..., c] float64 -> (codes [..., c/2] uint8, scales [..., c/32] uint8).
    Element 2j sits in the low nibble of byte j, element 2j+1 in the high nibble."""
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    assert c % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (c // 32, 32))
    elems, scales = mxfp4_encode_block(blocks)
    elems = elems.reshape(x.shape[:-1] + (c,)).astype(np.uint8)
    codes = (elems[..., 0::2] & 0xF) | ((elems[..., 1::2] & 0xF) << 4)
    return codes.astype(np.uint8), scales


def mxfp4_decode(codes, scales):
    codes = np.asarray(codes).astype(np.int64)
    lo = e2m1_decode(codes & 0xF)
    hi = e2m1_decode(codes >> 4)
    c = codes.shape[-1] * 2
    v = np.empty(codes.shape[:-1] + (c,), dtype=np.float64)
    v[..., 0::2] = lo
    v[..., 1::2] = hi
    X = e8m0_decode(scales)                   # [..., c/32]
    return v * np.repeat(X, 32, axis=-1)


def mxfp8_encode(x):
    """[..., c] float64 -> (E4M3 codes [..., c] uint8, E8M0 scales [..., c/32] uint8):
    OCP MX blocks of 32 consecutive values sharing the scale
    2^(floor(log2 amax) - 8) (8 = emax of E4M3), elements rounded to nearest
    even and saturated at +-448; an all-zero block has scale code 0."""
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    assert c % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (c // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    scale_codes = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, e = np.frexp(amax[nz])
    shared = np.clip((e - 1) - 8, -127, 127)   # floor(log2 amax) - emax(E4M3)
    scale_codes[nz] = shared + 127
    X = np.where(nz, np.ldexp(1.0, scale_codes - 127), 1.0)
    elems = e4m3_encode(blocks / X[..., None])
    elems[~nz] = 0
    return elems.reshape(x.shape).astype(np.uint8), scale_codes.astype(np.uint8)


def mxfp8_decode(codes, scales):
    X = e8m0_decode(scales)
    return e4m3_decode(codes) * np.repeat(X, 32, axis=-1)


# --------------------------------------------------------------------------
# KV row layouts
# --------------------------------------------------------------------------
# ROW_F32:            c float32 values
# ROW_BF16:           c bf16 values
# ROW_FP8_ROPE_BF16:  dims [0, c-64) as E4M3 bytes, then dims [c-64, c) as bf16
#                     (the last 64 dims carry RoPE; digest 模块 D and 模块 F)
ROW_F32, ROW_BF16, ROW_FP8_ROPE_BF16, ROW_MXFP4 = 0, 1, 2, 3
ROPE_DIMS = 64


def row_bytes(layout, c):
    if layout == ROW_F32:
        return 4 * c
    if layout == ROW_BF16:
        return 2 * c
    if layout == ROW_FP8_ROPE_BF16:
        return (c - ROPE_DIMS) + 2 * ROPE_DIMS
    if layout == ROW_MXFP4:
        return c // 2
    raise ValueError(layout)


def decode_rows(buf, layout, c, scales=None):
    """Stored rows (uint8 [..., row_bytes] or a typed array) -> float64 [..., c]."""
    buf = np.ascontiguousarray(buf)
    if layout == ROW_F32:
        return buf.view(np.float32).reshape(buf.shape[:-1] + (-1,))[..., :c].astype(np.float64) \
            if buf.dtype == np.uint8 else buf.astype(np.float64)
    if layout == ROW_BF16:
        u = buf.view(np.uint16) if buf.dtype == np.uint8 else buf
        return bf16_decode(u)
    if layout == ROW_FP8_ROPE_BF16:
        assert buf.dtype == np.uint8 and buf.shape[-1] == row_bytes(layout, c)
        nf8 = c - ROPE_DIMS
        lo = e4m3_decode(buf[..., :nf8])
        hi = bf16_decode(np.ascontiguousarray(buf[..., nf8:]).view(np.uint16))
        return np.concatenate([lo, hi], axis=-1)
    if layout == ROW_MXFP4:
        return mxfp4_decode(buf, scales)
    raise ValueError(layout)


def encode_rows(x, layout):
    """float64 [..., c] -> stored rows (and scales for MXFP4)."""
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    if layout == ROW_F32:
        return x.astype(np.float32), None
    if layout == ROW_BF16:
        return bf16_encode(x), None
    if layout == ROW_FP8_ROPE_BF16:
        nf8 = c - ROPE_DIMS
        lo = e4m3_encode(x[..., :nf8])
        hi = bf16_encode(x[..., nf8:]).view(np.uint8).reshape(x.shape[:-1] + (2 * ROPE_DIMS,))
        return np.concatenate([lo, hi], axis=-1), None
    if layout == ROW_MXFP4:
        return mxfp4_encode(x)
    raise ValueError(layout)


def round_rows(x, layout):
    """The values a row layout stores for float64 input x."""
    enc, sc = encode_rows(x, layout)
    return decode_rows(enc, layout, np.asarray(x).shape[-1], sc)
