"""Pins for the CPU oracle: each check ties it to something other than
itself (a closed form, an invariant, a library routine on a special case, or
brute force on tiny inputs), so that a dropped term, a wrong sign or index or
a transposed operand in the oracle fails at least one of them. CPU only."""

from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import interp
from reduce_view_amd import synth

U = 2.0 ** -24  # float32 unit roundoff


def gamma(n, u=U):
    return n * u / (1.0 - n * u)


def f32(x):
    return np.float32(x)


# ---------------------------------------------------------------------------
# View algebra (limn README, "Architecture": a View is (shape, strides,
# offset, mask) and the five movement ops compose into one)
# ---------------------------------------------------------------------------

def _view_only(base, *movement, raw=None):
    g = synth.Spec()
    b = g.buffer("x", base.shape, "f32")
    v = g.raw_view(b, **raw) if raw is not None else g.view(b, *movement)
    g.output(g.contiguous(v))
    return oracle.run(g, {"x": base})[0]


def test_view_permute_expand_shrink_pad_by_hand():
    x = np.arange(12, dtype=np.float32).reshape(3, 4)
    t = _view_only(x, ("permute", (1, 0)))
    assert t.shape == (4, 3)
    for i in range(4):
        for j in range(3):
            assert t[i, j] == x[j, i]
    row = np.arange(4, dtype=np.float32).reshape(1, 4)
    e = _view_only(row, ("expand", (5, 4)))
    for i in range(5):
        for j in range(4):
            assert e[i, j] == j
    s = _view_only(x, ("shrink", ((1, 3), (1, 4))))
    assert s.tolist() == [[5, 6, 7], [9, 10, 11]]
    p = _view_only(x, ("pad", ((1, 0), (0, 2))))
    assert p.shape == (4, 6)
    assert (p[0] == 0).all() and (p[:, 4:] == 0).all()
    assert (p[1:, :4] == x).all()
    r = _view_only(x, ("reshape", (2, 6)))
    assert r.tolist() == [[0, 1, 2, 3, 4, 5], [6, 7, 8, 9, 10, 11]]


def test_view_shrink_pad_round_trip_and_masked_border():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, 11)).astype(np.float32)
    y = _view_only(x, ("shrink", ((2, 7), (3, 8))), ("pad", ((2, 2), (3, 3))))
    assert y.shape == x.shape
    inside = np.zeros_like(x, dtype=bool)
    inside[2:7, 3:8] = True
    assert (y[inside] == x[inside]).all()
    assert (y[~inside] == 0).all()


def test_raw_view_is_offset_plus_strides_with_mask():
    x = np.arange(30, dtype=np.float32)
    raw = dict(shape=(4, 5), strides=(6, 1), offset=2, mask_lo=(1, 0), mask_hi=(4, 4))
    y = _view_only(x, raw=raw)
    for i in range(4):
        for j in range(5):
            expect = x[2 + 6 * i + j] if (1 <= i < 4 and 0 <= j < 4) else 0.0
            assert y[i, j] == expect
    # a negative offset is legal when the mask keeps every read in bounds
    raw = dict(shape=(3, 3), strides=(3, 1), offset=-4, mask_lo=(1, 1), mask_hi=(3, 3))
    y = _view_only(np.arange(9, dtype=np.float32), raw=raw)
    assert y.tolist() == [[0, 0, 0], [0, 0, 1], [0, 3, 4]]


def test_raw_view_matches_movement_chain():
    """shrink then pad of a (6,7) buffer is offset 0, strides (7,1), mask
    [1,5) x [2,5): the same View written two ways."""
    x = np.random.default_rng(3).standard_normal((6, 7)).astype(np.float32)
    a = _view_only(x, ("shrink", ((1, 5), (2, 5))), ("pad", ((1, 1), (2, 2))))
    b = _view_only(x, raw=dict(shape=(6, 7), strides=(7, 1), offset=0, mask_lo=(1, 2), mask_hi=(5, 5)))
    assert a.tobytes() == b.tobytes()


def test_raw_view_out_of_bounds_is_refused():
    with pytest.raises(oracle.OracleError):
        _view_only(np.arange(6, dtype=np.float32), raw=dict(shape=(2, 4), strides=(3, 1), offset=0))


# ---------------------------------------------------------------------------
# transpose (CONTIGUOUS of a permuted View)
# ---------------------------------------------------------------------------

def test_transpose_involution_and_index():
    x = np.random.default_rng(5).uniform(-1, 1, (37, 53)).astype(np.float32)
    t, = oracle.run(synth.transpose(37, 53), {"X": x})
    assert t.shape == (53, 37)
    i, j = np.meshgrid(np.arange(53), np.arange(37), indexing="ij")
    assert (t[i, j] == x[j, i]).all()
    tt, = oracle.run(synth.transpose(53, 37), {"X": t})
    assert tt.tobytes() == x.tobytes()


# ---------------------------------------------------------------------------
# broadcast MUL + SUM over k (limn README "Reading the schedule"; Luminal IR
# blog, "Naive Matrix Multiplication")
# ---------------------------------------------------------------------------

def _brute_matmul_f32(a, b):
    m, k = a.shape
    n = b.shape[1]
    y = np.zeros((m, n), dtype=np.float32)
    for i in range(m):
        for j in range(n):
            acc = f32(0.0)
            for kk in range(k):
                acc = f32(acc + f32(a[i, kk] * b[kk, j]))
            y[i, j] = acc
    return y


@pytest.mark.parametrize("m,n,k", [(4, 3, 5), (7, 5, 9), (1, 6, 1)])
def test_matmul_broadcast_bit_equals_triple_loop(m, n, k):
    inp = synth.inputs_matmul(m, n, k, seed=0)
    y, = oracle.run(synth.matmul_broadcast(m, n, k), inp)
    assert y.shape == (m, n, 1)
    assert y[:, :, 0].tobytes() == _brute_matmul_f32(inp["A"], inp["B"]).tobytes()
    yr, = oracle.run(synth.matmul_broadcast_raw(m, n, k), inp)
    assert yr.tobytes() == y.tobytes()


def test_matmul_identity_and_integers():
    a = np.random.default_rng(1).standard_normal((6, 6)).astype(np.float32)
    y, = oracle.run(synth.matmul_broadcast(6, 6, 6), {"A": a, "B": np.eye(6, dtype=np.float32)})
    assert y[:, :, 0].tobytes() == a.tobytes()
    rng = np.random.default_rng(2)
    ai = rng.integers(-2, 3, (9, 13))
    bi = rng.integers(-2, 3, (13, 7))
    y, = oracle.run(synth.matmul_broadcast(9, 7, 13), {"A": ai.astype(np.float32), "B": bi.astype(np.float32)})
    assert (y[:, :, 0] == (ai @ bi).astype(np.float32)).all()


# ---------------------------------------------------------------------------
# elementwise chain with permuted, stride-0 and masked operands
# ---------------------------------------------------------------------------

def test_ew_chain_special_cases_close_form():
    r, c = 13, 19
    rng = np.random.default_rng(9)
    bb = rng.uniform(10, 20, (c, r)).astype(np.float32)
    cv = np.zeros(c, dtype=np.float32)
    # a = 1 < b everywhere, c = 0: out = 1*b = Bb transposed, exactly
    out, = oracle.run(synth.ew_chain(r, c), {"a": np.ones((r, c), np.float32), "Bb": bb, "c": cv})
    assert out.tobytes() == np.ascontiguousarray(bb.T).tobytes()
    # a = 0 >= b everywhere: out = exp(-0) + c[j] = 1 + c[j] down every row
    cv = rng.uniform(-4, 4, c).astype(np.float32)
    out, = oracle.run(synth.ew_chain(r, c), {"a": np.zeros((r, c), np.float32), "Bb": -bb, "c": cv})
    assert (out == (f32(1.0) + cv)[None, :]).all()


def test_ew_chain_masked_border_closed_form():
    r, c, er, ec = 17, 23, 3, 5
    inp = synth.inputs_ew(r, c, seed=1)
    out, = oracle.run(synth.ew_chain(r, c, masked=True, edges=(er, ec)), inp)
    b = inp["Bb"].T
    inside = np.zeros((r, c), dtype=bool)
    inside[er:r - er, ec:c - ec] = True
    # a masked cell reads 0: CMPLT(0, b) picks 0*b = +0 when b > 0, else
    # EXP(-0) = 1; then c[j] is added
    expect = np.where(b > 0, inp["c"][None, :], f32(1.0) + inp["c"][None, :])
    assert (out[~inside] == expect[~inside]).all()
    full, = oracle.run(synth.ew_chain(r, c), {"a": inp["Abig"], "Bb": inp["Bb"], "c": inp["c"]})
    assert (out[inside] == full[inside]).all()


def test_exp_is_correctly_rounded_including_subnormals():
    getcontext().prec = 60
    xs = np.concatenate([
        np.linspace(-103.9, -87.0, 400), np.linspace(-20, 20, 400), np.linspace(80, 88.7, 100),
        np.array([0.0, -0.0, 1e-8, -1e-8]),
    ]).astype(np.float32)
    g = synth.Spec()
    x = g.buffer("x", xs.shape, "f32")
    g.output(g.exp(x))
    got, = oracle.run(g, {"x": xs})
    for xv, gv in zip(xs, got):
        exact = Decimal(float(xv)).exp()
        best = _round_decimal_to_f32(exact)
        assert gv == best, (xv, gv, best)


def _round_decimal_to_f32(d):
    f = np.float32(float(d))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: abs(Decimal(float(c)) - d))


# ---------------------------------------------------------------------------
# softmax (Litmus README, ToleranceBound lemmas R1 and R2)
# ---------------------------------------------------------------------------

def test_softmax_invariants():
    rows, n = 8, 4096
    x = synth.inputs_softmax(rows, n)["x"]
    it = oracle.Interpreter(synth.softmax(rows, n), {"x": x})
    y = it.value(synth.softmax(rows, n).outputs[0])
    # rows sum to one within the in-order fold bound plus the roundings
    s = y.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= gamma(n - 1) + 4 * U)
    # R1: x - max(x) <= 0 and R2: the denominator is >= 1
    spec = it.spec
    d = [i for i, nd in enumerate(spec.nodes) if nd["op"] == "ADD"][0]
    sden = [i for i, nd in enumerate(spec.nodes) if nd["op"] == "SUM"][0]
    assert (it.value(d) <= 0).all() and (it.value(d).max(axis=1) == 0).all()
    assert (it.value(sden) >= 1).all()
    # against float64 softmax of the same data (a library routine)
    ref = scipy.special.softmax(x.astype(np.float64), axis=1)
    bound = ref * (gamma(n - 1) + 4 * U) + 3 * 2.0 ** -149
    assert np.all(np.abs(y - ref) <= bound)


def test_softmax_shift_invariance_is_bit_exact():
    rows, n = 4, 1000
    rng = np.random.default_rng(4)
    x = (rng.integers(-2 ** 14, 2 ** 14, (rows, n)) * 2.0 ** -10).astype(np.float32)
    y0, = oracle.run(synth.softmax(rows, n), {"x": x})
    y1, = oracle.run(synth.softmax(rows, n), {"x": (x + np.float32(37.0)).astype(np.float32)})
    assert y0.tobytes() == y1.tobytes()


def test_softmax_constant_row_and_noshift_overflow():
    n = 4096
    y, = oracle.run(synth.softmax(2, n), {"x": np.full((2, n), 123.25, np.float32)})
    assert (y == np.float32(2.0 ** -12)).all()
    x = synth.inputs_softmax(4, 256)["x"]
    bad, = oracle.run(synth.softmax_noshift(4, 256), {"x": x})
    assert not np.isfinite(bad).all()
    good, = oracle.run(synth.softmax(4, 256), {"x": x})
    assert np.isfinite(good).all()


# ---------------------------------------------------------------------------
# RMSNorm (Tiki README, "Compile model code")
# ---------------------------------------------------------------------------

def test_rmsnorm_constant_power_of_two_row_is_weight():
    rows, n = 3, 4096
    w = synth.inputs_rmsnorm(1, n)["w"]
    for p in (3, 5):
        y, = oracle.run(synth.rmsnorm(rows, n), {"x": np.full((rows, n), 2.0 ** p, np.float32), "w": w})
        assert (y == w[None, :]).all()


def test_rmsnorm_constant_row_bound_and_float64_reference():
    n, eps = 4096, 1e-6
    w = synth.inputs_rmsnorm(1, n)["w"]
    for c in (0.3, 0.01, 1.7):
        y, = oracle.run(synth.rmsnorm(1, n, eps), {"x": np.full((1, n), c, np.float32), "w": w})
        rel = np.abs(y.astype(np.float64) / w - 1.0)
        assert rel.max() <= eps / (2 * np.float64(np.float32(c)) ** 2) + gamma(n - 1) + 8 * U
    inp = synth.inputs_rmsnorm(6, n)
    y, = oracle.run(synth.rmsnorm(6, n, eps), inp)
    x64 = inp["x"].astype(np.float64)
    ref = x64 / np.sqrt((x64 * x64).mean(axis=1, keepdims=True) + eps) * inp["w"]
    assert np.all(np.abs(y - ref) <= np.abs(ref) * (0.5 * gamma(n - 1) + 8 * U))


# ---------------------------------------------------------------------------
# LayerNorm (limn README, "nn, optim and checkpoints": torch semantics with a
# biased variance)
# ---------------------------------------------------------------------------

def test_layernorm_constant_row_is_beta():
    n = 512
    inp = synth.inputs_layernorm(1, n)
    x = interp.f32_to_bf16(np.full((2, n), 100.0, np.float32))
    y, = oracle.run(synth.layernorm(2, n), {"x": x, "gamma": inp["gamma"], "beta": inp["beta"]})
    assert (y == inp["beta"][None, :]).all()


def test_layernorm_mean_is_exact_and_matches_torch_float64():
    rows, n = 4, 8192
    inp = synth.inputs_layernorm(rows, n)
    spec = synth.layernorm(rows, n)
    it = oracle.Interpreter(spec, inp)
    y = it.value(spec.outputs[0])
    xf = interp.bf16_to_f32(inp["x"]).astype(np.float64)
    # the float32 sum of bfloat16 values near 100 is exact, so mu is exact
    mu_node = [i for i, nd in enumerate(spec.nodes) if nd["op"] == "MUL"][0]
    assert (it.value(mu_node)[:, 0].astype(np.float64) == xf.sum(axis=1) / n).all()
    g = interp.bf16_to_f32(inp["gamma"]).astype(np.float64)
    b = interp.bf16_to_f32(inp["beta"]).astype(np.float64)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(xf), (n,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    yf = interp.bf16_to_f32(y).astype(np.float64)
    # one bfloat16 rounding of the output plus float32 error far below it
    assert np.all(np.abs(yf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(ref) + 1e-6)
    # normalised rows: mean 0 and biased variance v / (v + eps)
    z = (yf - b) / g
    v = xf.var(axis=1)
    assert np.all(np.abs(z.mean(axis=1)) < 0.02)
    assert np.all(np.abs(z.var(axis=1) - v / (v + 1e-5)) < 0.02)


# ---------------------------------------------------------------------------
# bf16 contraction with relu^2 epilogue and full SUM
# ---------------------------------------------------------------------------

def test_gemm_integer_valued_is_exact():
    m, n, k = 24, 20, 40
    inp = synth.inputs_gemm_integer(m, n, k)
    y, = oracle.run(synth.gemm_bf16(m, n, k), inp)
    ai = interp.bf16_to_f32(inp["A"]).astype(np.int64)
    bi = interp.bf16_to_f32(inp["B"]).astype(np.int64)
    yi = ai @ bi
    assert (y[:, :, 0] == yi.astype(np.float32)).all()
    s, = oracle.run(synth.gemm_relu2_sum(m, n, k), inp)
    assert s.shape == (1, 1, 1)
    assert s[0, 0, 0] == np.float32((np.maximum(yi, 0) ** 2).sum())


def test_gemm_relu2_sum_statistics():
    m = n = k = 128
    inp = synth.inputs_gemm(m, n, k)
    s, = oracle.run(synth.gemm_relu2_sum(m, n, k), inp)
    # A ~ N(0, 1/sqrt(k)), B ~ N(0, 1): y ~ N(0, 1), so E[relu(y)^2] = 1/2
    assert 0.4 < s[0, 0, 0] / (m * n) < 0.6


def test_slab_evaluation_changes_no_bit():
    m, n, k = 16, 12, 33
    inp = synth.inputs_gemm(m, n, k)
    spec = synth.gemm_relu2_sum(m, n, k, emit_y=True)
    whole = oracle.run(spec, inp)
    slabs = oracle.run(spec, inp, max_elems=1000, slab_elems=700)
    for a, b in zip(whole, slabs):
        assert a.tobytes() == b.tobytes()


# ---------------------------------------------------------------------------
# dtype rules, reduce identities, folds
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    special = np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125 + 2 ** -9, 3.0e38, 3.4e38, -3.4e38,
                        np.inf, -np.inf, np.nan, 1e-40, -1e-40, 2 ** -126, 2 ** -133], dtype=np.float32)
    ties = (np.arange(1, 300, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([special, ties, rng.standard_normal(5000).astype(np.float32) * 1e3])
    ours = interp.f32_to_bf16(x)
    ref = synth.to_bf16_bits(x)
    nan = np.isnan(x)
    assert (ours[~nan] == ref[~nan]).all()
    assert np.isnan(interp.bf16_to_f32(ours[nan])).all()
    assert (interp.bf16_to_f32(ours[~nan]).astype(np.float64) == torch.from_numpy(x[~nan]).to(
        torch.bfloat16).to(torch.float64).numpy()).all()


def test_int_wraparound():
    g = synth.Spec()
    a = g.buffer("a", (4,), "i8")
    b = g.buffer("b", (4,), "i8")
    g.output(g.add(a, b), g.mul(a, b), g.neg(a))
    av = np.array([127, -128, 100, 3], np.int8)
    bv = np.array([1, -1, 100, 5], np.int8)
    s, p, ng = oracle.run(g, {"a": av, "b": bv})
    assert s.tolist() == [-128, 127, -56, 8]
    assert p.tolist() == [127, -128, 16, 15]
    assert ng.tolist() == [-127, -128, -100, -3]
    g = synth.Spec()
    x = g.buffer("x", (2, 200), "i8")
    g.output(g.sum(x, (1,)), g.max(x, (1,)))
    xv = np.ones((2, 200), np.int8)
    xv[1] = -5
    sm, mx = oracle.run(g, {"x": xv})
    assert sm[:, 0].tolist() == [-56, (200 * -5) % 256 - 256 if (200 * -5) % 256 >= 128 else (200 * -5) % 256]
    assert mx[:, 0].tolist() == [1, -5]


def test_reduce_identities():
    g = synth.Spec()
    x = g.buffer("x", (3, 50), "f32")
    g.output(g.max(x, (1,)))
    xv = -np.random.default_rng(2).uniform(1, 5, (3, 50)).astype(np.float32)
    m, = oracle.run(g, {"x": xv})
    assert (m[:, 0] == xv.max(axis=1)).all() and (m < 0).all()
    g = synth.Spec()
    e = g.buffer("e", (3, 0), "f32")
    g.output(g.sum(e, (1,)), g.max(e, (1,)))
    s, mx = oracle.run(g, {"e": np.zeros((3, 0), np.float32)})
    assert (s == 0).all() and (mx == -np.inf).all()


def test_max_propagates_nan():
    g = synth.Spec()
    x = g.buffer("x", (2, 5), "f32")
    g.output(g.max(x, (1,)))
    xv = np.array([[1, 2, np.nan, 3, 4], [1, 2, 3, 4, 5]], np.float32)
    m, = oracle.run(g, {"x": xv})
    assert np.isnan(m[0, 0]) and m[1, 0] == 5


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_max_signed_zeros_do_not_depend_on_order(dt):
    """-0 orders below +0 (IEEE 754-2019 maximum): every arrangement of
    signed zeros (and negatives) gives +0 whenever a +0 is present, -0 when
    only -0 and negatives are."""
    import itertools
    npdt = np.float32 if dt == "f32" else np.float64
    rows = []
    for perm in itertools.permutations([-0.0, 0.0, -1.0]):
        rows.append(perm)
    rows.append((-0.0, -2.0, -0.0))
    xv = np.array(rows, npdt)
    g = synth.Spec()
    x = g.buffer("x", xv.shape, dt)
    g.output(g.max(x, (1,)))
    m, = oracle.run(g, {"x": xv})
    m = m[:, 0]
    assert all(v == 0 and not np.signbit(v) for v in m[:-1])
    assert m[-1] == 0 and np.signbit(m[-1])


def test_sum_order_is_ascending():
    """A fold in ascending order gives a specific, order-revealing result."""
    g = synth.Spec()
    x = g.buffer("x", (1, 3), "f32")
    g.output(g.sum(x, (1,)))
    s, = oracle.run(g, {"x": np.array([[2.0 ** 24, 1.0, 1.0]], np.float32)})
    assert s[0, 0] == np.float32(2.0 ** 24)          # (2^24 + 1) + 1 rounds twice
    s, = oracle.run(g, {"x": np.array([[1.0, 1.0, 2.0 ** 24]], np.float32)})
    assert s[0, 0] == np.float32(2.0 ** 24 + 2)       # 2 + 2^24 is exact


def test_long_float32_sum_widens():
    n = (1 << 24) + 4
    g = synth.Spec()
    x = g.buffer("x", (n,), "f32")
    g.output(g.sum(x, (0,)))
    s, = oracle.run(g, {"x": np.ones(n, np.float32)})
    assert s[0] == np.float32(n)


def test_threaded_fold_equals_serial(tmp_path):
    import subprocess
    import sys
    code = ("import numpy as np, sys; sys.path.insert(0, %r); from oracle import interp; "
            "x = np.random.default_rng(0).standard_normal((64, 5000)).astype(np.float32); "
            "sys.stdout.write(interp._reduce('SUM', x, 'f32', (1,)).tobytes().hex())") % (
        str(__import__('os').path.dirname(__import__('os').path.dirname(__file__))),)
    outs = []
    for t in ("1", "7"):
        env = dict(__import__('os').environ, OMP_NUM_THREADS=t)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                                   text=True, check=True).stdout)
    assert outs[0] == outs[1] and len(outs[0]) > 0


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ---------------------------------------------------------------------------

def test_planted_max_identity_zero_is_caught(monkeypatch):
    real = interp._reduce

    def bad(op, x, dt, axes):
        r = real(op, x, dt, axes)
        return np.maximum(r, 0) if op == "MAX" else r
    monkeypatch.setattr(interp, "_reduce", bad)
    with pytest.raises(AssertionError):
        test_reduce_identities()


def test_planted_transposed_operand_is_caught(monkeypatch):
    real = interp._apply_movement

    def bad(arr, mv):
        if mv[0] == "permute":
            return arr
        return real(arr, mv)
    monkeypatch.setattr(interp, "_apply_movement", bad)
    with pytest.raises(Exception):
        test_transpose_involution_and_index()
    with pytest.raises(Exception):
        test_matmul_broadcast_bit_equals_triple_loop(4, 3, 5)


def test_planted_dropped_weight_is_caught(monkeypatch):
    real = interp._binary

    def bad(op, x, y, dt):
        # drop the final "* w": the one MUL whose right operand is the
        # broadcast weight (identical rows, varying along the row)
        if op == "MUL" and x.ndim == 2 and (y == y[0:1]).all() and not (y == y.flat[0]).all():
            return x.copy()
        return real(op, x, y, dt)
    monkeypatch.setattr(interp, "_binary", bad)
    with pytest.raises(AssertionError):
        test_rmsnorm_constant_power_of_two_row_is_weight()


def test_planted_sign_error_in_softmax_is_caught(monkeypatch):
    real = interp._unary

    def bad(op, x, dt):
        if op == "NEG":
            return x.copy()
        return real(op, x, dt)
    monkeypatch.setattr(interp, "_unary", bad)
    with pytest.raises(AssertionError):
        test_softmax_invariants()


def test_planted_unbiased_variance_is_caught(monkeypatch):
    real = interp._binary
    seen = {"n": 0}

    def bad(op, x, y, dt):
        # the second "* (1/n)" is the variance's: make it 1/(n-1)
        if op == "MUL" and x.shape == (4, 1) and np.all(np.asarray(y) == np.float32(1.0 / 8192)):
            seen["n"] += 1
            if seen["n"] == 2:
                return real(op, x, np.full_like(y, np.float32(1.0 / 8191)), dt)
        return real(op, x, y, dt)
    monkeypatch.setattr(interp, "_binary", bad)
    with pytest.raises(AssertionError) as e:
        test_layernorm_mean_is_exact_and_matches_torch_float64()
    assert seen["n"] >= 2


# ---------------------------------------------------------------------------
# fused attention forward (CUSTOM sdpa_fwd), evaluated as its primitives
# ---------------------------------------------------------------------------

def _attention_f64(q, k, v, scale, causal):
    """Textbook attention in float64, written independently of the oracle:
    softmax(scale q k^T) v with the row max subtracted, and the logsumexp."""
    qd, kd, vd = (interp.bf16_to_f32(a).astype(np.float64) for a in (q, k, v))
    s = np.einsum("hid,hjd->hij", qd, kd) * scale
    if causal:
        s = np.where(np.arange(s.shape[2])[None, None, :] <= np.arange(s.shape[1])[None, :, None], s, -np.inf)
    m = s.max(axis=2, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=2, keepdims=True)
    return (e / z) @ vd, m + np.log(z)


@pytest.mark.parametrize("h,tq,tk,d,causal", [(2, 37, 37, 32, True), (3, 20, 45, 64, False), (1, 64, 64, 16, True)])
def test_sdpa_matches_float64_attention(h, tq, tk, d, causal):
    spec = synth.attention(h, tq, tk, d, causal)
    inp = synth.inputs_attention(h, tq, tk, d)
    o, lse = oracle.run(spec, inp)
    o64, l64 = _attention_f64(inp["Q"], inp["K"], inp["V"], 1.0 / np.sqrt(d), causal)
    # float32 per primitive against float64: a few hundred ulps at most here
    assert np.abs(o - o64).max() <= 1e-5 * np.abs(o64).max()
    assert np.abs(lse - l64).max() <= 1e-5 * (np.abs(l64).max() + 1)


def test_sdpa_closed_forms():
    h, t, d = 2, 16, 32
    inp = synth.inputs_attention(h, t, t, d)
    o, lse = oracle.run(synth.attention(h, t, t, d, causal=True), inp)
    # causal row 0 sees key 0 only: O = V[0] and L = the one scaled score
    assert o[:, 0].tobytes() == interp.bf16_to_f32(inp["V"][:, 0]).tobytes()
    s00 = (interp.bf16_to_f32(inp["Q"][:, 0]) * interp.bf16_to_f32(inp["K"][:, 0])).astype(np.float32)
    s00 = np.array([interp._reduce("SUM", s00[i:i + 1], "f32", (1,))[0, 0] for i in range(h)], np.float32)
    assert lse[:, 0, 0].tobytes() == (s00 * np.float32(1.0 / np.sqrt(d))).astype(np.float32).tobytes()
    # all scores equal (K = 0): uniform weights, O is the mean of V's rows and
    # L is log(Tk) (sum of ones is exact, 1/Tk exact for a power of two)
    inp0 = dict(inp, K=np.zeros_like(inp["K"]))
    o, lse = oracle.run(synth.attention(h, t, t, d, causal=False), inp0)
    vm = interp.bf16_to_f32(inp["V"]).astype(np.float64).mean(axis=1)
    assert np.abs(o - vm[:, None, :]).max() <= 4 * gamma(t - 1) * np.abs(interp.bf16_to_f32(inp["V"])).sum(axis=1).max() / t
    assert np.all(lse == np.float32(np.log(np.float32(t))))


def test_sdpa_large_scores_need_the_max_shift():
    # scores near 1e4: exp without the max shift overflows; with it the
    # result is finite and matches float64
    h, t, d = 1, 24, 32
    inp = synth.inputs_attention(h, t, t, d)
    inp["Q"] = synth.to_bf16_bits(interp.bf16_to_f32(inp["Q"]) * np.float32(300.0))
    o, lse = oracle.run(synth.attention(h, t, t, d, causal=False), inp)
    o64, l64 = _attention_f64(inp["Q"], inp["K"], inp["V"], 1.0 / np.sqrt(d), False)
    assert np.all(np.isfinite(o)) and np.abs(o - o64).max() <= 1e-4 * np.abs(o64).max()
    assert np.abs(lse - l64).max() <= 1e-5 * np.abs(l64).max()


def test_planted_transposed_attention_scores_are_caught(monkeypatch):
    real = interp.sdpa_fwd

    def bad(q, k, v, scale, causal, out_dtype="f32", block=64):
        # softmax over the wrong axis: swap the roles of q and k
        return real(k, q, v, scale, causal, out_dtype, block) if q.shape == k.shape else real(q, k, v, scale, causal,
                                                                                               out_dtype, block)
    monkeypatch.setattr(interp, "sdpa_fwd", bad)
    with pytest.raises(AssertionError):
        test_sdpa_matches_float64_attention(2, 37, 37, 32, True)


def test_planted_missing_causal_mask_is_caught(monkeypatch):
    real = interp.sdpa_fwd
    monkeypatch.setattr(interp, "sdpa_fwd", lambda q, k, v, scale, causal, out_dtype="f32", block=64:
                        real(q, k, v, scale, False, out_dtype, block))
    with pytest.raises(AssertionError):
        test_sdpa_closed_forms()


# ---------------------------------------------------------------------------
# indexed primitives: GATHER and SCATTER (limn README, "The op set", indexed;
# "Backends": the C device folds a scatter's colliding adds serially)
# ---------------------------------------------------------------------------

def _gather_loops(data, index, axis):
    """Brute force over every output position, written from the definition."""
    out = np.zeros(index.shape, data.dtype)
    for p in np.ndindex(*index.shape):
        t = int(index[p])
        if 0 <= t < data.shape[axis]:
            q = list(p)
            q[axis] = t
            out[p] = data[tuple(q)]
    return out


def _scatter_loops(base, index, values, axis):
    """Brute force: positions in row-major order, one float32 add each."""
    out = base.copy()
    for p in np.ndindex(*index.shape):
        t = int(index[p])
        if 0 <= t < base.shape[axis]:
            q = list(p)
            q[axis] = t
            out[tuple(q)] = np.float32(out[tuple(q)] + values[p])
    return out


def _indexed_spec(kind, dshape, ishape, axis, dtype="f32"):
    g = synth.Spec()
    d = g.buffer("data", dshape, dtype)
    i = g.buffer("index", ishape, "i32")
    if kind == "gather":
        g.output(g.gather(d, i, axis))
    else:
        v = g.buffer("values", ishape, dtype)
        g.output(g.scatter(d, i, v, axis))
    return g


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_gather_brute_force_with_out_of_range(axis):
    rng = np.random.default_rng(40 + axis)
    data = rng.standard_normal((3, 4, 5)).astype(np.float32)
    ishape = [3, 4, 5]
    ishape[axis] = 7
    index = rng.integers(-2, data.shape[axis] + 2, ishape).astype(np.int32)
    got, = oracle.run(_indexed_spec("gather", data.shape, tuple(ishape), axis), {"data": data, "index": index})
    assert got.tobytes() == _gather_loops(data, index, axis).tobytes()
    assert np.all(got[(index < 0) | (index >= data.shape[axis])] == 0)


def test_gather_identity_index_is_the_data():
    data = np.arange(60, dtype=np.float32).reshape(3, 4, 5)
    for axis in range(3):
        shp = [1, 1, 1]
        shp[axis] = data.shape[axis]
        index = np.broadcast_to(np.arange(data.shape[axis], dtype=np.int32).reshape(shp), data.shape).copy()
        got, = oracle.run(_indexed_spec("gather", data.shape, data.shape, axis), {"data": data, "index": index})
        assert got.tobytes() == data.tobytes()


def test_embedding_gather_picks_rows():
    inp = synth.inputs_embedding(50, 6, 30)
    got, = oracle.run(synth.embedding_gather(50, 6, 30), {k: inp[k] for k in ("table", "ids")})
    for r in range(30):
        assert got[r].tobytes() == inp["table"][inp["ids"][r, 0]].tobytes()


@pytest.mark.parametrize("axis", [0, 1])
def test_scatter_brute_force_with_collisions(axis):
    rng = np.random.default_rng(50 + axis)
    base = rng.standard_normal((6, 5)).astype(np.float32)
    ishape = [6, 5]
    ishape[axis] = 9
    index = rng.integers(-1, base.shape[axis] + 1, ishape).astype(np.int32)
    values = rng.standard_normal(ishape).astype(np.float32)
    got, = oracle.run(_indexed_spec("scatter", base.shape, tuple(ishape), axis),
                      {"data": base, "index": index, "values": values})
    assert got.tobytes() == _scatter_loops(base, index, values, axis).tobytes()


def test_scatter_of_ones_is_a_histogram():
    rng = np.random.default_rng(60)
    ids = rng.integers(0, 40, (500, 1)).astype(np.int32)
    g = synth.Spec()
    i = g.buffer("index", (500, 1), "i32")
    g.output(g.scatter(g.const(0, (40, 1), "i32"), i, g.const(1, (500, 1), "i32"), 0))
    got, = oracle.run(g, {"index": ids})
    assert np.array_equal(got[:, 0], np.bincount(ids[:, 0], minlength=40))


def test_scatter_collisions_fold_in_index_order():
    """Three adds into one float32 cell: 1, then 1e8 (1e8 + 1 rounds to 1e8,
    the spacing there being 8), then -1e8: 0 exactly. Any other order that
    adds -1e8 before the 1 gives 1."""
    g = _indexed_spec("scatter", (2,), (3,), 0)
    got, = oracle.run(g, {"data": np.zeros(2, np.float32), "index": np.array([1, 1, 1], np.int32),
                          "values": np.array([1.0, 1e8, -1e8], np.float32)})
    assert got.tolist() == [0.0, 0.0]
    got, = oracle.run(g, {"data": np.zeros(2, np.float32), "index": np.array([1, 1, 1], np.int32),
                          "values": np.array([1e8, -1e8, 1.0], np.float32)})
    assert got.tolist() == [0.0, 1.0]


def test_scatter_drops_out_of_range_and_keeps_base():
    g = _indexed_spec("scatter", (3,), (4,), 0)
    got, = oracle.run(g, {"data": np.array([5, 6, 7], np.float32), "index": np.array([-1, 3, 99, 1], np.int32),
                          "values": np.array([100, 200, 300, 0.5], np.float32)})
    assert got.tolist() == [5.0, 6.5, 7.0]


def test_scatter_narrow_dtypes_round_and_wrap_per_add():
    """int8: 100 + 100 wraps to -56. float16: 2048 + 1 ties to even (2048),
    three times over; one rounding of 2048 + 3 would give 2052."""
    g = _indexed_spec("scatter", (1,), (2,), 0, "i8")
    got, = oracle.run(g, {"data": np.zeros(1, np.int8), "index": np.zeros(2, np.int32),
                          "values": np.array([100, 100], np.int8)})
    assert got.tolist() == [-56]
    g = _indexed_spec("scatter", (1,), (3,), 0, "f16")
    got, = oracle.run(g, {"data": np.array([2048], np.float16), "index": np.zeros(3, np.int32),
                          "values": np.ones(3, np.float16)})
    assert got.tolist() == [2048.0]


def test_gather_then_scatter_of_a_permutation_is_the_identity():
    rng = np.random.default_rng(61)
    data = rng.standard_normal((8, 3)).astype(np.float32)
    perm = rng.permutation(8).astype(np.int32)
    index = np.repeat(perm[:, None], 3, axis=1)
    gathered, = oracle.run(_indexed_spec("gather", (8, 3), (8, 3), 0), {"data": data, "index": index})
    back, = oracle.run(_indexed_spec("scatter", (8, 3), (8, 3), 0),
                       {"data": np.zeros((8, 3), np.float32), "index": index, "values": gathered})
    assert back.tobytes() == data.tobytes()


def test_planted_reversed_scatter_order_is_caught(monkeypatch):
    real = interp.scatter

    def bad(base, index, values, axis, dt):
        return real(base, np.flip(index, axis), np.flip(values, axis), axis, dt)
    monkeypatch.setattr(interp, "scatter", bad)
    with pytest.raises(AssertionError):
        test_scatter_collisions_fold_in_index_order()


def test_planted_gather_axis_mixup_is_caught(monkeypatch):
    real = interp.gather
    monkeypatch.setattr(interp, "gather", lambda data, index, axis, dt:
                        real(data, index, (axis + 1) % data.ndim, dt) if data.ndim > 1 else real(data, index, axis, dt))
    with pytest.raises(Exception):
        test_gather_brute_force_with_out_of_range(0)


def test_planted_scatter_without_base_is_caught(monkeypatch):
    real = interp.scatter
    monkeypatch.setattr(interp, "scatter", lambda base, index, values, axis, dt:
                        real(np.zeros_like(base), index, values, axis, dt))
    with pytest.raises(AssertionError):
        test_scatter_drops_out_of_range_and_keeps_base()
