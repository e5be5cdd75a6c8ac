"""Pins for the oracle's CAST across all 49 (source, target) pairs of the
seven dtypes (limn README, "The op set", dtype paragraph: float16 and
bfloat16 are storage widths computed in float32, ints wrap modulo 2^width).

The expected values come from closed forms written here, independent of the
oracle's numpy code: an exact rational round-to-nearest-even into each float
format (with subnormals and overflow to infinity), math.trunc for float ->
int, and Python integer arithmetic for the wraparound. The convention pinned:
a value bound for a half width is a float32 first (a float64 or a large int32
source rounds twice, as torch's conversions do), float -> int truncates
toward zero and wraps (defined while the truncated value fits in int32).
CPU only."""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import interp
from reduce_view_amd import synth

DTS = synth.DTYPES
FLOATS = ("f32", "bf16", "f16", "f64")
INT_W = {"i32": 32, "i16": 16, "i8": 8}
# (significand bits with the hidden one, smallest normal exponent, largest exponent)
FMT = {"f64": (53, -1022, 1023), "f32": (24, -126, 127), "f16": (11, -14, 15), "bf16": (8, -126, 127)}


def rne(v, fmt):
    """Round the exact value of a Python int or float to the nearest value of
    ``fmt``, ties to even; NaN stays NaN, overflow gives infinity, the sign of
    a zero is kept."""
    if isinstance(v, float):
        if math.isnan(v) or math.isinf(v):
            return v
        if v == 0.0:
            return v
    if v == 0:
        return 0.0
    p, emin, emax = FMT[fmt]
    q = Fraction(v)
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax:
        return sign * math.inf
    return math.copysign(float(r), sign)


def wrap(i, w):
    return (i + 2 ** (w - 1)) % 2 ** w - 2 ** (w - 1)


def decode(arr, dt):
    """Exact Python values of a storage array (bfloat16 as bit patterns)."""
    if dt == "bf16":
        return [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in arr]
    if dt in INT_W:
        return [int(x) for x in arr]
    return [float(x) for x in arr]


def expected(v, src, dst):
    """The pinned CAST of one source value, or None where it is undefined
    (float -> int of NaN, an infinity, or a value whose truncation leaves
    int32)."""
    if dst in INT_W:
        if src in INT_W:
            return wrap(v, INT_W[dst])
        if math.isnan(v) or math.isinf(v):
            return None
        t = math.trunc(v)
        if not -2 ** 31 <= t < 2 ** 31:
            return None
        return wrap(t, INT_W[dst])
    if dst == "f64":
        return float(v)
    if dst == "f32":
        return rne(v, "f32")
    return rne(rne(v, "f32"), dst)


def same(got, want):
    if isinstance(want, int):
        return got == want
    if math.isnan(want):
        return math.isnan(got)
    return got == want and math.copysign(1.0, got) == math.copysign(1.0, want)


@pytest.fixture(scope="module")
def cast_run():
    inp = synth.inputs_cast(1024)
    outs = oracle.run(synth.cast_matrix(1024), inp)
    return inp, outs


def test_cast_matrix_matches_closed_forms(cast_run):
    inp, outs = cast_run
    it = iter(outs)
    checked = 0
    for src in DTS:
        xs = decode(inp[f"x_{src}"], src)
        for dst in DTS:
            got = decode(next(it), dst)
            for x, g in zip(xs, got):
                want = expected(x, src, dst)
                if want is None:
                    continue
                assert same(g, want), (src, dst, x, g, want)
                checked += 1
    assert checked > 45000


WITNESS = [
    # (src, dst, source value, pinned result)
    ("f64", "bf16", 1 + 2 ** -8 + 2 ** -30, 1.0),          # through float32: a tie, to even
    ("f64", "f16", 1 + 2 ** -11 + 2 ** -40, 1.0),          # the same for float16
    ("f64", "f32", 1 + 2 ** -24, 1.0),                     # a tie, to even
    ("f64", "f32", 1 + 2 ** -24 + 2 ** -50, 1 + 2 ** -23),  # above the tie
    ("f64", "f32", 3.5e38, math.inf),
    ("i32", "bf16", 2 ** 24 + 2 ** 16 + 1, float(2 ** 24)),  # 2^24 + 2^17 if rounded once
    ("i32", "f32", 2 ** 24 + 1, float(2 ** 24)),
    ("i32", "f32", 2 ** 24 + 3, float(2 ** 24 + 4)),
    ("i32", "f32", -(2 ** 24 + 1), -float(2 ** 24)),
    ("i32", "f16", 2049, 2048.0),
    ("i32", "f16", 2051, 2052.0),
    ("i32", "f16", 65519, 65504.0),
    ("i32", "f16", 65520, math.inf),
    ("f32", "f16", 1 + 2 ** -11, 1.0),
    ("f32", "f16", 1 + 3 * 2 ** -11, 1 + 2 ** -9),
    ("f32", "f16", 65504.0, 65504.0),
    ("f32", "f16", 65520.0, math.inf),
    ("f32", "f16", 2 ** -24, 2 ** -24),
    ("f32", "f16", 2 ** -25, 0.0),
    ("f32", "f16", 1.5 * 2 ** -25, 2 ** -24),
    ("f32", "bf16", 1 + 2 ** -8, 1.0),
    ("f32", "bf16", 1 + 3 * 2 ** -8, 1 + 2 ** -6),
    ("f32", "bf16", 3.4e38, math.inf),
    ("f32", "i8", 300.0, 44),
    ("f32", "i8", -129.5, 127),
    ("f32", "i8", 127.9, 127),
    ("f32", "i8", 128.0, -128),
    ("f32", "i8", -0.5, 0),
    ("f32", "i8", 1.5, 1),
    ("f32", "i8", -1.5, -1),
    ("f32", "i8", -0.0, 0),
    ("f32", "i16", 40000.0, -25536),
    ("f32", "i32", -2147483648.0, -2 ** 31),
    ("f32", "i32", 2147483520.0, 2147483520),
    ("bf16", "i32", -2.5, -2),
    ("f16", "i16", 65504.0, -32),
    ("f64", "i8", -2.9999, -2),
    ("i32", "i8", 300, 44),
    ("i32", "i8", -129, 127),
    ("i32", "i8", 255, -1),
    ("i32", "i16", 40000, -25536),
    ("i8", "i32", -128, -128),
    ("i16", "f16", -32768, -32768.0),
]


_STORE = {"f32": np.float32, "f16": np.float16, "f64": np.float64, "i32": np.int32, "i16": np.int16, "i8": np.int8}


def _encode(src, value):
    """One source value in its storage (bfloat16 by torch's RNE cast)."""
    if src == "bf16":
        return synth.to_bf16_bits(np.array([value], dtype=np.float32))
    return np.array([value], dtype=_STORE[src])


def _one(src, dst, value):
    g = synth.Spec()
    x = g.buffer("x", (1,), src)
    g.output(g.cast(x, dst))
    return decode(oracle.run(g, {"x": _encode(src, value)})[0], dst)[0]


@pytest.mark.parametrize("src,dst,value,want", WITNESS)
def test_cast_witness_table(src, dst, value, want):
    """Hand-derived results, checked against the oracle and the closed form."""
    got = _one(src, dst, value)
    assert same(got, want), (got, want)
    assert same(expected(decode(_encode(src, value), src)[0], src, dst), want)


_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64,
          "i32": torch.int32, "i16": torch.int16, "i8": torch.int8}


def _to_torch(arr, dt):
    if dt == "bf16":
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(arr.copy())


def test_cast_matrix_agrees_with_torch(cast_run):
    """torch's Tensor.to on the same values, where the cast is defined."""
    inp, outs = cast_run
    it = iter(outs)
    for src in DTS:
        xs = decode(inp[f"x_{src}"], src)
        t = _to_torch(inp[f"x_{src}"], src)
        for dst in DTS:
            ours = decode(next(it), dst)
            ref = t.to(_TORCH[dst])
            ref = ref.to(torch.float64).tolist() if dst in FLOATS else ref.tolist()
            for x, a, b in zip(xs, ours, ref):
                if expected(x, src, dst) is None:
                    continue
                if isinstance(b, float) and math.isnan(b):
                    assert math.isnan(a), (src, dst, x)
                else:
                    assert a == b, (src, dst, x, a, b)


def test_planted_rounding_float_to_int_is_caught(monkeypatch, cast_run):
    real = interp._to_dtype_from_float

    def rounding(x, dtype):
        if dtype in interp.INTS:
            return np.rint(x.astype(np.float64)).astype(np.int64).astype(interp.STORAGE[dtype])
        return real(x, dtype)
    monkeypatch.setattr(interp, "_to_dtype_from_float", rounding)
    with pytest.raises(AssertionError):
        test_cast_witness_table("f32", "i8", 1.5, 1)


def test_planted_saturating_int_cast_is_caught(monkeypatch):
    real = interp._cast

    def saturating(x, s, d):
        if s in interp.INTS and d in interp.INTS:
            info = np.iinfo(interp.STORAGE[d])
            return np.clip(x.astype(np.int64), info.min, info.max).astype(interp.STORAGE[d])
        return real(x, s, d)
    monkeypatch.setattr(interp, "_cast", saturating)
    with pytest.raises(AssertionError):
        test_cast_witness_table("i32", "i8", 300, 44)


def test_planted_single_rounding_to_bf16_is_caught(monkeypatch):
    real = interp._to_dtype_from_float

    def direct(x, dtype):
        if dtype == "bf16" and x.dtype == np.float64:
            # round the float64 value once, straight to 8 significant bits
            m, e = np.frexp(x)
            return interp.f32_to_bf16(np.ldexp(np.round(m * 256.0) / 256.0, e).astype(np.float32))
        return real(x, dtype)
    monkeypatch.setattr(interp, "_to_dtype_from_float", direct)
    with pytest.raises(AssertionError):
        test_cast_witness_table("f64", "bf16", 1 + 2 ** -8 + 2 ** -30, 1.0)
