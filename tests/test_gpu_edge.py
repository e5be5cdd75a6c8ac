"""GPU parity on the edges of the contract: empty tensors and reduces over an
empty range (the reduce identity), size-1 dims, cuts through workspace and
several outputs, dtype variants, MAX over all-negative rows and NaN, denormal
outputs, and the transcendental sweeps (EXP over every float32 in
[-2048, 88.7]; LOG, SQRT, RECIP over a strided sample of all positive
floats). The HIP path runs through the C ABI; every expected value comes from
the oracle or from a closed form checked against the oracle here."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from reduce_view_amd import synth
from tests.harness import U, gamma, report, run, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from reduce_view_amd import rv
    rv.rv_init(0)


def _prog(spec):
    from reduce_view_amd import rv
    return rv.compile_spec(spec)


def _case(name):
    print(f"CASE {name}", flush=True)


def _same(got, ref):
    """Bit-identical, NaN bit patterns aside (any NaN matches any NaN)."""
    assert got.shape == ref.shape and got.dtype == ref.dtype
    if got.dtype.kind == "f":
        gn, rn = np.isnan(got), np.isnan(ref)
        assert np.array_equal(gn, rn)
        return got[~gn].tobytes() == ref[~rn].tobytes()
    return got.tobytes() == ref.tobytes()


def _ord(a: np.ndarray) -> np.ndarray:
    """float32 -> int64 in the float order, +0 and -0 both 0: the difference
    of two is their distance in ulps."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


# ---- empty ranges, identities, size-1 dims ---------------------------------

def _sum_max(shape, axes):
    g = synth.Spec(f"summax_{'x'.join(map(str, shape))}")
    x = g.buffer("x", shape, "f32")
    g.output(g.sum(x, axes), g.max(x, axes))
    return g


def _softmax_outputs(rows, n):
    g = synth.Spec(f"softmax_stats_{rows}x{n}")
    x = g.buffer("x", (rows, n), "f32")
    m = g.max(x, (1,))
    e = g.exp(g.add(x, g.neg(g.view(m, ("expand", (rows, n))))))
    s = g.sum(e, (1,))
    y = g.mul(e, g.view(g.recip(s), ("expand", (rows, n))))
    g.output(y, m, s)
    return g


@pytest.mark.parametrize("shape,axes", [((3, 0), (1,)), ((0, 4), (1,)), ((0, 4), (0,)), ((2, 3, 0), (1, 2)),
                                        ((2, 0, 3), (1,)), ((1, 7, 1, 3), (1, 3)), ((1, 1), (0, 1))])
def test_reduce_identity_empty_and_unit_dims(shape, axes):
    """A reduce over an empty range writes its identity (0 for SUM, -inf for
    MAX); an empty output launches nothing; size-1 dims fold in order."""
    _case(f"sum/max {shape} over {axes}")
    x = np.random.default_rng(11).standard_normal(shape).astype(np.float32)
    spec = _sum_max(shape, axes)
    got = run(_prog(spec), {"x": x})
    ref = oracle.run(spec, {"x": x})
    for g, r in zip(got, ref):
        assert _same(g, r), (shape, axes, g, r)


def test_softmax_over_empty_rows_writes_row_stats():
    _case("softmax stats over (3, 0)")
    spec = _softmax_outputs(3, 0)
    x = np.zeros((3, 0), np.float32)
    got = run(_prog(spec), {"x": x})
    ref = oracle.run(spec, {"x": x})
    assert got[0].shape == (3, 0)
    assert _same(got[1], ref[1]) and np.all(got[1] == -np.inf)
    assert _same(got[2], ref[2]) and np.all(got[2] == 0)


def test_empty_elementwise_output():
    _case("exp over (0, 5)")
    g = synth.Spec()
    x = g.buffer("x", (0, 5), "f32")
    g.output(g.exp(x))
    got = run(_prog(g), {"x": np.zeros((0, 5), np.float32)})
    assert got[0].shape == (0, 5)


# ---- cuts, workspace, several outputs ----------------------------------------

def test_cuts_workspace_and_several_outputs():
    _case("permuted computed value (cut through workspace)")
    g = synth.Spec()
    a = g.buffer("a", (40, 72), "f32")
    b = g.buffer("b", (40, 72), "f32")
    s = g.add(a, b)
    g.output(g.mul(g.view(s, ("permute", (1, 0))), g.view(s, ("permute", (1, 0)))))
    rng = np.random.default_rng(12)
    inp = {"a": rng.standard_normal((40, 72)).astype(np.float32), "b": rng.standard_normal((40, 72)).astype(np.float32)}
    assert _same(run(_prog(g), inp)[0], oracle.run(g, inp)[0])

    _case("reduces over different axes")
    g = synth.Spec()
    x = g.buffer("x", (6, 7, 5), "f32")
    g.output(g.max(g.sum(x, (2,)), (0,)))
    xi = rng.standard_normal((6, 7, 5)).astype(np.float32)
    assert _same(run(_prog(g), {"x": xi})[0], oracle.run(g, {"x": xi})[0])

    _case("an input returned as an output, one value output twice")
    g = synth.Spec()
    x = g.buffer("x", (5, 3), "f32")
    m = g.max(x, (1,))
    g.output(x, m, m)
    xi = rng.standard_normal((5, 3)).astype(np.float32)
    for a_, b_ in zip(run(_prog(g), {"x": xi}), oracle.run(g, {"x": xi})):
        assert _same(a_, b_)


# ---- dtype variants ------------------------------------------------------------

@pytest.mark.parametrize("dt", ["i8", "i16", "i32", "f16", "f64", "bf16"])
def test_dtype_variants(dt):
    """ADD/MUL/NEG in the dtype (ints wrap), a SUM along rows and a MAX down
    columns. Ints and MAX are bit-exact; float SUMs within the
    reduction-order bound of their float32 (f64: float64) running total
    plus one rounding to the storage dtype."""
    _case(f"dtype {dt} (67, 300)")
    rng = np.random.default_rng(13)
    shape = (67, 300)
    mk = {
        "i8": lambda: rng.integers(-128, 128, shape).astype(np.int8),
        "i16": lambda: rng.integers(-2 ** 15, 2 ** 15, shape).astype(np.int16),
        "i32": lambda: rng.integers(-2 ** 31, 2 ** 31, shape, dtype=np.int64).astype(np.int32),
        "f16": lambda: rng.standard_normal(shape).astype(np.float16),
        "f64": lambda: rng.standard_normal(shape),
        "bf16": lambda: synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32)),
    }[dt]
    g = synth.Spec(f"dtypes_{dt}")
    a = g.buffer("a", shape, dt)
    b = g.buffer("b", shape, dt)
    s = g.add(g.mul(a, b), g.neg(b))
    g.output(s, g.sum(s, (1,)), g.max(s, (0,)))
    inp = {"a": mk(), "b": mk()}
    got = run(_prog(g), inp)
    ref = oracle.run(g, inp)
    assert _same(got[0], ref[0]) and _same(got[2], ref[2])
    if dt.startswith("i"):
        assert _same(got[1], ref[1])
        return
    to64 = (lambda v: oracle.bf16_to_f32(v).astype(np.float64)) if dt == "bf16" else (lambda v: v.astype(np.float64))
    sval = to64(ref[0])
    u = 2.0 ** -53 if dt == "f64" else U
    out_ulp = {"f16": 2.0 ** -10, "bf16": 2.0 ** -7, "f64": 0.0}[dt]
    mag = np.abs(to64(ref[1])).ravel()
    bound = 4 * gamma(shape[1] - 1, u) * np.abs(sval).sum(axis=1) + out_ulp * np.maximum(mag, 2.0 ** -14) * 2
    err = np.abs(to64(got[1]).ravel() - to64(ref[1]).ravel())
    report(f"dtype_{dt}_sum", err, bound)
    assert np.all(err <= bound)


# ---- MAX: all-negative rows, NaN, denormal outputs ------------------------------

def test_max_all_negative_rows_and_nan():
    """MAX starts from -inf, not 0 (an all-negative row keeps its negative
    maximum), and a NaN anywhere in the reduced range gives NaN: through a
    row-resident kernel (softmax's row max) and a cells kernel (column max)."""
    _case("max over all-negative rows with NaNs")
    rng = np.random.default_rng(14)
    x = -(rng.random((48, 1000)).astype(np.float32) + 0.5)
    x[5, 17] = np.nan
    x[30, 999] = np.nan
    spec = _softmax_outputs(48, 1000)
    got = run(_prog(spec), {"x": x})
    ref = oracle.run(spec, {"x": x})
    assert _same(got[1], ref[1])
    assert np.isnan(got[1][5, 0]) and np.isnan(got[1][30, 0])
    assert np.all(got[1][~np.isnan(got[1])] < 0)
    spec = _sum_max((48, 1000), (0,))
    got = run(_prog(spec), {"x": x})
    ref = oracle.run(spec, {"x": x})
    assert _same(got[1], ref[1]) and np.isnan(got[1][0, 17]) and np.isnan(got[1][0, 999])


def test_softmax_keeps_denormal_outputs():
    """x - m in [-103.3, -87.3] gives subnormal probabilities; they are kept,
    not flushed to zero (the oracle preserves denormals). At the very bottom
    of the range (2^-149) a one-ulp difference in EXP may round y to 0 or to
    the next subnormal, inside the softmax bound's absolute term 3 * 2^-149;
    from 2^-140 up a flush would show as a zero."""
    _case("softmax denormal window 64x4096")
    inp = synth.inputs_softmax(64, 4096)
    spec = synth.softmax(64, 4096)
    got = run(_prog(spec), inp)[0]
    ref = oracle.run(spec, inp)[0]
    tiny = np.finfo(np.float32).tiny
    sub = (ref > 0) & (ref < tiny)
    deep = sub & (ref >= 2.0 ** -140)
    assert sub.sum() > 1000 and deep.sum() > 500  # about 30 subnormals per row
    d = np.abs(_ord(got[sub]) - _ord(ref[sub]))
    print(f"subnormal outputs {int(sub.sum())} ({int(deep.sum())} >= 2^-140); zero on the GPU "
          f"{int((got[sub] == 0).sum())}; max ulp distance {int(d.max())}", flush=True)
    assert np.all(got[deep] > 0)
    assert np.all((got[sub] > 0) | (ref[sub] <= 3 * 2.0 ** -149))


# ---- transcendental sweeps --------------------------------------------------------

CHUNK = 1 << 26


def _oracle_unary(op: str, x: np.ndarray) -> np.ndarray:
    """The oracle's OP over x, in pieces on a thread pool (numpy drops the GIL
    inside the ufuncs)."""
    piece = 1 << 22
    parts = [x[i:i + piece] for i in range(0, x.size, piece)]
    with ThreadPoolExecutor(max_workers=16) as ex:
        outs = list(ex.map(lambda p: oracle.run(synth.unary_map(op, p.size), {"x": p})[0], parts))
    return np.concatenate(outs) if outs else np.zeros(0, np.float32)


def _gpu_unary(prog, x: np.ndarray):
    """The HIP path's OP over x (padded with +1 to the program's size),
    left on the device."""
    import torch
    n = x.size
    if n < CHUNK:
        x = np.concatenate([x, np.ones(CHUNK - n, np.float32)])
    out = prog.launch({"x": to_device(x)})[0]
    torch.cuda.synchronize()
    return out[:n]


def _max_ulps_to_const(out_dev, c: float) -> int:
    import torch
    b = out_dev.view(torch.int32).to(torch.int64)
    o = torch.where(b < 0, -(b & 0x7FFFFFFF), b)
    ref = int(_ord(np.array([c], np.float32))[0])
    return int((o - ref).abs().max().item())


def test_exp_exhaustive_sweep():
    """Every float32 in [-2048, 88.7]: GPU EXP within 2 ulp of the oracle's
    (float64 exp rounded once). Where |x| < 2^-25 the exact result rounds to
    1, and where x <= -104 it rounds to +0 (e^-104 < 2^-150); those ranges are
    checked against the constant, itself pinned to the oracle on a sample."""
    prog = _prog(synth.unary_map("EXP", CHUNK))
    regions = [
        ("tiny+", 0x00000000, 0x33000000, 1.0),
        ("tiny-", 0x80000000, 0xB3000000, 1.0),
        ("main+", 0x33000000, 0x42B16667, None),  # up to 88.7 (0x42B16666)
        ("main-", 0xB3000000, 0xC2D00000, None),  # |x| in [2^-25, 104)
        ("under", 0xC2D00000, 0xC5000001, 0.0),  # [-2048, -104]
    ]
    worst = 0
    for name, lo, hi, const in regions:
        _case(f"exp sweep {name} [{lo:#010x}, {hi:#010x})")
        if const is not None:
            pin = synth.fp32_sweep(lo, hi, 65537)
            assert np.all(_oracle_unary("EXP", pin) == np.float32(const)), name
        for c0 in range(lo, hi, CHUNK):
            x = synth.fp32_sweep(c0, min(hi, c0 + CHUNK))
            out = _gpu_unary(prog, x)
            if const is not None:
                d = _max_ulps_to_const(out, const)
            else:
                d = int(np.abs(_ord(to_host(out)) - _ord(_oracle_unary("EXP", x))).max())
            worst = max(worst, d)
            assert d <= 2, (name, hex(c0), d)
    print(f"BOUND exp sweep max ulp {worst} (bound 2)", flush=True)


SAMPLE_STEP = 97


def _positive_sample() -> np.ndarray:
    s = synth.fp32_sweep(0x00000001, 0x7F800000, SAMPLE_STEP)
    special = np.array([0.0, -0.0, -1.0, np.inf, -np.inf, np.nan, 1.0, 2.0, 0.5, np.finfo(np.float32).tiny,
                        np.finfo(np.float32).max, 1e-45, 3.0, 10.0], np.float32)
    return np.concatenate([s, special])


@pytest.mark.parametrize("op,ulps", [("LOG", 2), ("SQRT", 0), ("RECIP", 0)])
def test_log_sqrt_recip_sampled(op, ulps):
    """Every 97th positive float32 (subnormals included) plus special values:
    LOG within 2 ulp of the oracle; SQRT and RECIP correctly rounded, so
    bit-identical (NaN for NaN and for LOG/SQRT of negatives)."""
    _case(f"{op} sampled sweep")
    x = _positive_sample()
    prog = _prog(synth.unary_map(op, CHUNK))
    got = to_host(_gpu_unary(prog, x))
    ref = _oracle_unary(op, x)
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn)
    fin = ~rn & np.isfinite(ref)
    assert np.array_equal(got[~rn & ~fin], ref[~rn & ~fin])  # infinities
    d = np.abs(_ord(got[fin]) - _ord(ref[fin]))
    print(f"BOUND {op} sampled max ulp {int(d.max())} (bound {ulps})", flush=True)
    assert int(d.max()) <= ulps
