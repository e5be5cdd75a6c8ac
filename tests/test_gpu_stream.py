"""GPU parity for rows too long to keep in registers: the streaming ROW plan
(one pass per reduce plus one for the outputs, the softmax MAX and SUM
folded into one pass by the online max/denominator recurrence), against the
oracle's plain per-primitive softmax / RMSNorm / LayerNorm. Also the same
plan forced onto short rows, and masked rows (-inf entries): partly masked,
masked but for one entry, and fully masked (NaN, as the primitive graph
defines: -inf - (-inf))."""

import contextlib
import os

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


@contextlib.contextmanager
def _env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    os.environ.update({k: str(v) for k, v in kv.items()})
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _check_softmax(name, spec, inp):
    """Bound: the reduction-order term 4 gamma_{n-1} of the denominator, plus
    the online rescales: every term of the denominator passes through at most
    R products by exp(m_old - m_new) (one per later chunk of its lane whose
    maximum grew, one per butterfly level, one per later wave), each within
    2 ulp and rounded once, and its own EXP within 2 ulp: (5R + 4) u. Then y's
    own EXP (2 ulp), RECIP and MUL (u each), and 3 * 2^-149 for subnormal y."""
    prog = P._prog(spec)
    k = prog.describe()["kernels"][0]
    assert k["plan"] == "row_stream" and k["plan_detail"]["online"], k["plan"]
    T, nch = k["plan_detail"]["threads_per_row"], k["plan_detail"]["chunks"]
    R = nch + int(np.log2(min(T, 64))) + max(T // 64, 1) - 1
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    n = ref.shape[1]
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    rel = 4 * gamma(n - 1) + (5 * R + 4) * U + 2 * 2.0 ** -23 + 4 * U
    r64 = np.where(nan, 0, ref).astype(np.float64)
    bound = np.abs(r64) * rel + 3 * 2.0 ** -149
    err = np.abs(np.where(nan, 0, got).astype(np.float64) - r64)
    report(name, err, bound)
    assert np.all(err <= bound)
    return got, ref


@pytest.mark.parametrize("rows,n", [(4, 300000), (3, 65553)])
def test_softmax_long_rows_online(rows, n):
    # RV_SPLIT=0: few long rows would otherwise become split reduces
    P._case(f"softmax long rows {rows}x{n}")
    with _env(RV_SPLIT=0):
        _check_softmax(f"softmax_stream_{rows}x{n}", synth.softmax(rows, n), synth.inputs_softmax(rows, n))


def test_softmax_long_rows_masked():
    """-inf entries: random half of a row; all but one entry (y is exactly 1
    there and 0 elsewhere); all entries (NaN on both sides); the first 40000
    entries (the running maximum stays -inf through many chunks)."""
    P._case("softmax long rows with -inf entries 6x70000")
    rows, n = 6, 70000
    x = synth.inputs_softmax(rows, n)["x"].copy()
    rng = np.random.default_rng(21)
    x[0, rng.random(n) < 0.5] = -np.inf
    x[1, :] = -np.inf
    x[1, 31337] = 5.0
    x[2, :] = -np.inf
    x[3, :40000] = -np.inf
    got, ref = _check_softmax("softmax_stream_masked", synth.softmax(rows, n), {"x": x})
    assert got[1, 31337] == 1.0 and np.all(np.delete(got[1], 31337) == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(ref[2]))
    assert np.all(got[0][x[0] == -np.inf] == 0) and np.all(got[3, :40000] == 0)


def test_stream_plan_forced_on_short_rows():
    with _env(RV_ROW_STREAM=1):
        for rows, n in [(33, 1000), (5, 128), (64, 4096)]:
            P._case(f"softmax streamed {rows}x{n}")
            _check_softmax(f"softmax_forced_stream_{rows}x{n}", synth.softmax(rows, n), synth.inputs_softmax(rows, n))
        assert P._prog(synth.rmsnorm(33, 1000)).describe()["kernels"][0]["plan"] == "row_stream"
        P.test_rmsnorm(33, 1000)
        P.test_rmsnorm(5, 128)
        assert P._prog(synth.layernorm(9, 1000)).describe()["kernels"][0]["plan"] == "row_stream"
        P.test_layernorm(9, 1000)
        P.test_layernorm(3, 256)


def test_norms_long_rows_multipass():
    """RMSNorm and LayerNorm rows too long for registers: one streaming pass
    per reduce (LayerNorm: mean, centred square sum) and one for y. The
    LayerNorm row (65536 bf16 values near 100, multiples of 0.5) keeps every
    partial sum of x below 2^23, so the mean is exact in any order."""
    assert P._prog(synth.rmsnorm(4, 100000)).describe()["kernels"][0]["plan"] == "row_stream"
    P.test_rmsnorm(4, 100000)
    assert P._prog(synth.layernorm(4, 65536)).describe()["kernels"][0]["plan"] == "row_stream"
    P.test_layernorm(4, 65536)


def test_softmax_long_full_size():
    """The long-row workload the benchmark times: 256 rows of 262144 float32
    (1 MB per row, beyond a CU's registers and LDS)."""
    P._case("softmax long rows full 256x262144")
    _check_softmax("softmax_stream_256x262144", synth.softmax(256, 262144), synth.inputs_softmax(256, 262144))
