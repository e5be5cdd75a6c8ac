"""CAST between every pair of the seven dtypes on the GPU, bit for bit
against the oracle (limn README, "The op set", dtype paragraph), on the
pinned witnesses (ties of every float width, overflow, subnormals, values
that round twice on the way to a half width, truncation and wraparound) and
seeded fill of every class, including random bit patterns. NaN results only
have to be NaN; a float -> int cast of NaN, an infinity or a value whose
truncation leaves int32 is undefined and skipped."""

import numpy as np
import pytest

import oracle
from reduce_view_amd import rv, synth
from tests.harness import run

pytestmark = pytest.mark.gpu

DTS = synth.DTYPES
INTS = ("i32", "i16", "i8")


def _as_f64(arr, dt):
    if dt == "bf16":
        return (arr.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def _defined(x, src, dst):
    """Cells whose CAST is defined: all but float -> int of NaN, an infinity
    or a magnitude whose truncation leaves int32."""
    if dst not in INTS or src in INTS:
        return np.ones(x.shape, dtype=bool)
    v = _as_f64(x, src)
    with np.errstate(invalid="ignore"):
        t = np.trunc(v)
        return np.isfinite(v) & (t >= -2.0 ** 31) & (t < 2.0 ** 31)


@pytest.mark.parametrize("n", [1024, 77])
def test_cast_matrix_bit_exact(n):
    rv.rv_init(0)
    spec = synth.cast_matrix(n)
    inp = synth.inputs_cast(n)
    prog = rv.compile_spec(spec)
    assert {k["class"] for k in prog.describe()["kernels"]} == {"EW"}
    got = run(prog, inp)
    ref = oracle.run(spec, inp)
    i = 0
    for src in DTS:
        x = inp[f"x_{src}"]
        for dst in DTS:
            g, r = got[i], ref[i]
            i += 1
            assert g.dtype == r.dtype and g.shape == r.shape, (src, dst)
            keep = _defined(x, src, dst)
            if dst in INTS:
                bad = keep & (g != r)
            else:
                gn, rn = np.isnan(_as_f64(g, dst)), np.isnan(_as_f64(r, dst))
                width = {"f64": np.uint64, "f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}[dst]
                bad = keep & ((gn != rn) | (~rn & (g.view(width) != r.view(width))))
            assert not bad.any(), (src, dst, x[bad][:4], g[bad][:4], r[bad][:4])
