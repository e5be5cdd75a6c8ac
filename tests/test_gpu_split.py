"""GPU parity for the split reduce (limn README, "Backends": a long reduce
over few cells splits into strided partial totals and a fold). A reduce
whose output cells are few for its length runs as a SPLIT kernel (each
workgroup folds one piece of the reduce range into a partial, in a fixed
order) and a FOLD kernel (each cell's partials in piece order, then the
region's elementwise tail).

Bounds: MAX and integer SUMs are bit-exact (order-free and exact wrapping).
A float SUM of N terms is within 4 gamma_{N-1} sum |x| of the oracle's
in-order fold (the reduction-order bound), and, stated in the depth form,
within gamma_h sum |x| + u |S| where h is the most additions any term passes
through in the kernel's tree (``sum_depth`` of the FOLD kernel); the oracle
keeps a total of 2^24 float32 terms in float64 (the gamma_{N-1} form is
vacuous there), so only the depth form applies to it. Two runs give the same
bits."""

import numpy as np
import pytest

import oracle
from reduce_view_amd import synth
from tests import test_gpu_parity as P
from tests.harness import U, gamma, report, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from reduce_view_amd import rv
    rv.rv_init(0)


def _plan(prog):
    ks = prog.describe()["kernels"]
    return [(k["class"], k["plan"]) for k in ks], ks


def _abs_sum(x, axes, dtype):
    if dtype == "bf16":
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.abs(x.astype(np.float64)).sum(axis=tuple(axes), keepdims=True)


def _check_sum(name, spec, inp, axes, dtype="f32", u=U, plan=None, runs=2):
    prog = P._prog(spec)
    classes, ks = _plan(prog)
    assert [c for c, _ in classes] == ["SPLIT", "FOLD"], classes
    if plan:
        assert classes[0][1] == plan, classes
    h = ks[1]["plan_detail"]["sum_depth"]
    outs = [run(prog, inp)[0] for _ in range(runs)]
    for o in outs[1:]:
        assert o.tobytes() == outs[0].tobytes(), "two runs differ"
    got, = outs[:1]
    ref, = oracle.run(spec, inp)
    assert got.shape == ref.shape and got.dtype == ref.dtype
    g64 = got.astype(np.float64) if dtype != "bf16" else (got.astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)
    r64 = ref.astype(np.float64) if dtype != "bf16" else (ref.astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)
    a = _abs_sum(inp["x"], axes, dtype).reshape(r64.shape)  # (the reduce may run over a permuted View)
    n = int(np.prod([inp["x"].shape[d] for d in axes]))
    err = np.abs(g64 - r64)
    out_u = 2.0 ** -8 if dtype == "bf16" else (2.0 ** -53 if dtype == "f64" else U)
    # depth form: the kernel's tree against the exact total (gamma_h), the
    # oracle's own in-order fold against it (gamma_{N-1}, or one rounding
    # when the oracle widened the total to float64), and for bfloat16 both
    # sides' final rounding to the output width
    widened = (n - 1) * u >= 1 / 3
    oracle_err = 2 * out_u * np.abs(r64) if widened else gamma(n - 1, u) * a
    depth_bound = gamma(h, u) * a + oracle_err + (2 * out_u * np.abs(r64) if dtype == "bf16" else 0)
    report(name + "_depth", err, depth_bound)
    assert np.all(err <= depth_bound)
    if (n - 1) * u < 1 / 3:
        ns_bound = 4 * gamma(n - 1, u) * a + (2 * out_u * np.abs(r64) if dtype == "bf16" else 0)
        report(name, err, ns_bound)
        assert np.all(err <= ns_bound)
    else:
        print("BOUND", name, "4*gamma_{N-1}: vacuous (DIVERGENT) at N =", n, flush=True)
    return got, ref


def test_full_sum_2pow24():
    """The full SUM of 2^24 float32 values to a scalar (one cell, 2^24
    terms): before the split it ran on one workgroup."""
    P._case("split full sum 2^24")
    shape = (1 << 24,)
    _check_sum("split_sum_2pow24", synth.reduce(shape, (0,)), synth.inputs_reduce(shape), (0,), plan="split_row")


def test_column_sum_16384x4096():
    """SUM over axis 0 of (16384, 4096): 4096 cells, each 16384 terms."""
    P._case("split column sum 16384x4096")
    shape = (16384, 4096)
    _check_sum("split_colsum_16384x4096", synth.reduce(shape, (0,)), synth.inputs_reduce(shape, seed=12), (0,),
               plan="split_cols")


@pytest.mark.parametrize("shape,axes,plan", [
    ((7, 200003), (1,), "split_row"),        # ragged chunks, few rows
    ((40009, 77), (0,), "split_cols"),       # ragged pieces, 77 cells
    ((6, 520, 700), (0, 2), "split_row"),    # two reduced dims around a kept one
    ((3, 1 << 20), (1,), "split_row"),
])
def test_split_sum_shapes(shape, axes, plan):
    P._case(f"split sum {shape} over {axes}")
    _check_sum(f"split_sum_{'x'.join(map(str, shape))}", synth.reduce(shape, axes), synth.inputs_reduce(shape, seed=13),
               axes, plan=plan)


def test_split_sum_through_views():
    """A transposed row reduce (lanes walk the kept, stride-1 dim) and a
    full SUM over a padded View (masked cells read zero)."""
    P._case("split sum through a permuted view")
    x = synth.inputs_reduce((1 << 20, 8), seed=14)
    _check_sum("split_sum_permuted", synth.reduce((1 << 20, 8), (1,), permute=(1, 0)), x, (0,), plan="split_cols")
    P._case("split sum through a padded view")
    x = synth.inputs_reduce((1000, 3000), seed=15)
    spec = synth.reduce((1000, 3000), (0, 1), pad=((3, 4), (5, 6)))
    _check_sum("split_sum_padded", spec, x, (0, 1), plan="split_row")


def test_split_sum_dtypes():
    P._case("split sum bf16 rows")
    shape = (3, 1 << 20)
    _check_sum("split_sum_bf16", synth.reduce(shape, (1,), dtype="bf16"), synth.inputs_reduce(shape, "bf16", seed=16),
               (1,), dtype="bf16")
    P._case("split sum f64")
    shape = (1 << 21,)
    _check_sum("split_sum_f64", synth.reduce(shape, (0,), dtype="f64"), synth.inputs_reduce(shape, "f64", seed=17), (0,),
               dtype="f64", u=2.0 ** -53)


@pytest.mark.parametrize("dtype,shape,axes", [("i32", (1 << 22,), (0,)), ("i8", (5000, 300), (0,)),
                                              ("i16", (4, 1 << 19), (1,))])
def test_split_int_sum_bit_exact(dtype, shape, axes):
    P._case(f"split int sum {dtype} {shape}")
    spec = synth.reduce(shape, axes, dtype=dtype)
    inp = synth.inputs_reduce(shape, dtype, seed=18)
    prog = P._prog(spec)
    assert [c for c, _ in _plan(prog)[0]] == ["SPLIT", "FOLD"]
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("dtype", ["f32", "i32", "f64"])
def test_split_max_bit_exact(dtype):
    P._case(f"split max {dtype}")
    shape = ((1 << 22) + 37,)
    spec = synth.reduce(shape, (0,), op="MAX", dtype=dtype)
    inp = synth.inputs_reduce(shape, dtype, seed=19)
    prog = P._prog(spec)
    assert [c for c, _ in _plan(prog)[0]] == ["SPLIT", "FOLD"]
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()
    if dtype == "f32":
        x = inp["x"].copy()
        x[:] = -np.abs(x) - 1.0  # all negative: MAX is not 0
        got, = run(prog, {"x": x})
        assert got[0] == x.max() and got[0] < 0
        x[3_000_001] = np.nan
        got, = run(prog, {"x": x})
        assert np.isnan(got[0])


def test_split_with_epilogue():
    """The FOLD kernel evaluates the region's tail: a row mean SUM * (1/n)."""
    P._case("split mean rows 8x500000")
    rows, n = 8, 500000
    spec = synth.mean_rows(rows, n)
    inp = synth.inputs_reduce((rows, n), seed=20)
    prog = P._prog(spec)
    classes, ks = _plan(prog)
    assert [c for c, _ in classes] == ["SPLIT", "FOLD"]
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    a = _abs_sum(inp["x"], (1,), "f32") / n
    bound = 4 * gamma(n - 1) * a + 2 * U * np.abs(ref.astype(np.float64))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    report("split_mean_rows", err, bound)
    assert np.all(err <= bound)


def test_split_softmax_few_long_rows():
    """Softmax over 4 rows of 300000: its MAX and its SUM each become a split
    reduce (cut so the whole chip works on 4 rows), then the outputs."""
    P._case("split softmax 4x300000")
    rows, n = 4, 300000
    spec = synth.softmax(rows, n)
    inp = synth.inputs_softmax(rows, n)
    prog = P._prog(spec)
    classes, _ = _plan(prog)
    assert [c for c, _ in classes] == ["SPLIT", "FOLD", "SPLIT", "FOLD", "EW"], classes
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    # the denominator's order term, each EXP (2 ulp), RECIP and MUL (u each),
    # and subnormal outputs
    rel = 4 * gamma(n - 1) + 4 * U + 2 * 2.0 ** -23 + 4 * U
    r64 = ref.astype(np.float64)
    bound = np.abs(r64) * rel + 3 * 2.0 ** -149
    err = np.abs(got.astype(np.float64) - r64)
    report("split_softmax_4x300000", err, bound)
    assert np.all(err <= bound)
