"""GPU parity of the indexed primitives against the oracle.

GATHER moves data: bit-exact for every dtype, out-of-range indices read
zero. Ordered SCATTER (stable radix sort of the index cells, then each run
of equal targets folded in index order) is bit-exact too, for every dtype:
it performs the oracle's additions in the oracle's order. Atomic SCATTER
(f32, f64, i32) is exact for i32; for floats the colliding adds land in any
order, so a target with c contributions differs from the ordered result by
at most 2 gamma_c (|base| + sum |v|) (each order is within gamma_c of the
exact sum), plus c * 2^-126 for a hardware add that might flush a subnormal
result."""

import numpy as np
import pytest

import oracle
from reduce_view_amd import synth
from tests.harness import gamma, report, run

pytestmark = pytest.mark.gpu

U64 = 2.0 ** -53


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


def _rand(rng, shape, dt):
    if dt in ("i32", "i16", "i8"):
        lim = {"i32": 2 ** 31 - 1, "i16": 2 ** 15 - 1, "i8": 127}[dt]
        return rng.integers(-lim, lim, shape).astype({"i32": np.int32, "i16": np.int16, "i8": np.int8}[dt])
    x = rng.standard_normal(shape)
    if dt == "bf16":
        return synth.to_bf16_bits(x.astype(np.float32))
    return x.astype({"f32": np.float32, "f64": np.float64, "f16": np.float16}[dt])


def _spec(kind, dshape, ishape, axis, dt, atomic=False):
    g = synth.Spec(f"{kind}_{dt}")
    d = g.buffer("data", dshape, dt)
    i = g.buffer("index", ishape, "i32")
    if kind == "gather":
        g.output(g.gather(d, i, axis))
    else:
        v = g.buffer("values", ishape, dt)
        g.output(g.scatter(d, i, v, axis, atomic))
    return g


def _exact(name, spec, inp):
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.shape == ref.shape and got.dtype == ref.dtype
    if got.tobytes() != ref.tobytes():
        bad = np.flatnonzero((got.view(np.uint8).reshape(got.size, -1) != ref.view(np.uint8).reshape(ref.size, -1))
                             .any(axis=1))
        raise AssertionError(f"{name}: {bad.size} cells differ, first {bad[:8]}: got {got.ravel()[bad[:4]]}, "
                             f"oracle {ref.ravel()[bad[:4]]}")
    print(f"EXACT {name} {got.size} cells", flush=True)
    return got


# ---------------------------------------------------------------------------
# GATHER
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "f64", "i32", "i16", "i8"])
def test_embedding_gather_dtypes(dt):
    _case(f"embedding gather {dt}")
    vocab, dim, n = 3001, 96, 2500
    inp = synth.inputs_embedding(vocab, dim, n)
    rng = np.random.default_rng(80)
    inp["table"] = _rand(rng, (vocab, dim), dt)
    inp["ids"][::97] = -1  # out of range: zero rows
    inp["ids"][5::101] = vocab
    _exact(f"embedding_gather_{dt}", synth.embedding_gather(vocab, dim, n, dt), inp)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_gather_general_axes(axis):
    """A varying index on every axis of a 3-D tensor, with a ragged last dim
    and out-of-range entries."""
    _case(f"gather general axis {axis}")
    rng = np.random.default_rng(81 + axis)
    dshape = (37, 45, 129)
    ishape = list(dshape)
    ishape[axis] = 53
    data = rng.standard_normal(dshape).astype(np.float32)
    index = rng.integers(-2, dshape[axis] + 2, ishape).astype(np.int32)
    _exact(f"gather_axis{axis}", _spec("gather", dshape, tuple(ishape), axis, "f32"), {"data": data, "index": index})


def test_gather_from_a_padded_permuted_view_with_computed_index():
    _case("gather through a View, computed index")
    g = synth.Spec("gather_view")
    d = g.buffer("D", (40, 70, 33), "f32")
    dv = g.view(d, ("permute", (2, 1, 0)), ("pad", ((0, 0), (3, 2), (0, 0))), ("permute", (2, 1, 0)),
                ("shrink", ((0, 40), (1, 74), (0, 33))))
    i = g.buffer("I", (40, 50, 33), "i32")
    idx = g.add(i, g.const(-1, (40, 50, 33), "i32"))
    g.output(g.mul(g.gather(dv, idx, 1), g.const(3.0, (40, 50, 33), "f32")))
    rng = np.random.default_rng(84)
    inp = {"D": rng.standard_normal((40, 70, 33)).astype(np.float32),
           "I": rng.integers(-2, 77, (40, 50, 33)).astype(np.int32)}
    _exact("gather_view", g, inp)


def test_gather_full_size():
    """The benchmark's workload: 32768 ids into a (65536, 1024) float32
    table."""
    _case("embedding gather full 65536x1024 by 32768")
    vocab, dim, n = 65536, 1024, 32768
    inp = synth.inputs_embedding(vocab, dim, n)
    _exact("embedding_gather_full", synth.embedding_gather(vocab, dim, n), {k: inp[k] for k in ("table", "ids")})


# ---------------------------------------------------------------------------
# ordered SCATTER: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "f64", "i32", "i16", "i8"])
def test_embedding_scatter_ordered_dtypes(dt):
    """Heavy collisions (2500 rows into 300) so each target folds ~8 values
    in order; some ids out of range."""
    _case(f"embedding scatter ordered {dt}")
    vocab, dim, n = 300, 96, 2500
    inp = synth.inputs_embedding(vocab, dim, n)
    rng = np.random.default_rng(85)
    inp["values"] = _rand(rng, (n, dim), dt)
    inp["ids"][::89] = -5
    inp["ids"][3::97] = vocab
    _exact(f"embedding_scatter_{dt}", synth.embedding_scatter(vocab, dim, n, dt),
           {k: inp[k] for k in ("values", "ids")})


@pytest.mark.parametrize("keys,cells", [(200, 5000), (70000, 9000), (300, 100000), (1000, 300000)])
def test_scatter_ordered_radix_passes_and_tiles(keys, cells):
    """One, three, two and two radix passes; 3, 5, 49 and 147 tiles of 2048
    cells, so equal keys cross tile boundaries and must keep their order
    (147 tiles: the digit counts are scanned by a kernel of their own)."""
    _case(f"scatter ordered keys={keys} cells={cells}")
    rng = np.random.default_rng(86)
    base = rng.standard_normal((keys, 3)).astype(np.float32)
    index = rng.integers(0, keys, (cells, 1)).astype(np.int32)
    values = rng.standard_normal((cells, 3)).astype(np.float32) * np.float32(1e3)
    g = synth.Spec("scatter_radix")
    d = g.buffer("data", (keys, 3), "f32")
    i = g.view(g.buffer("index", (cells, 1), "i32"), ("expand", (cells, 3)))
    g.output(g.scatter(d, i, g.buffer("values", (cells, 3), "f32"), 0))
    kd = _prog(g).describe()["kernels"]
    detail = kd[1]["plan_detail"]
    assert detail["keys"] == keys and detail["index_cells"] == cells  # the 3 columns are carried
    assert detail["radix_passes"] == (int(keys - 1).bit_length() + 7) // 8
    assert ("scatter_scan" in [x["plan"] for x in kd]) == (cells > 64 * 2048)
    _exact(f"scatter_k{keys}_c{cells}", g, {"data": base, "index": index, "values": values})


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_scatter_ordered_general_axes(axis):
    """An index varying along every dim (nothing carried): one thread per
    index cell."""
    _case(f"scatter ordered general axis {axis}")
    rng = np.random.default_rng(87 + axis)
    oshape = (23, 31, 65)
    ishape = list(oshape)
    ishape[axis] = 40
    base = rng.standard_normal(oshape).astype(np.float32)
    index = rng.integers(-1, oshape[axis] + 1, ishape).astype(np.int32)
    values = rng.standard_normal(ishape).astype(np.float32)
    _exact(f"scatter_axis{axis}", _spec("scatter", oshape, tuple(ishape), axis, "f32"),
           {"data": base, "index": index, "values": values})


def test_scatter_all_into_one_row():
    """Every id the same: one run of 6000 values, folded in order."""
    _case("scatter one hot row")
    inp = synth.inputs_embedding(64, 256, 6000)
    inp["ids"][:] = 17
    _exact("scatter_one_row", synth.embedding_scatter(64, 256, 6000), {k: inp[k] for k in ("values", "ids")})


def test_scatter_order_decides_the_result():
    """1, 1e8, -1e8 into one cell: 0 in index order (1 is absorbed), 1 in
    any order that cancels first; 513 copies so they span lanes and waves."""
    _case("scatter order decides")
    n = 3 * 513
    values = np.tile(np.array([1.0, 1e8, -1e8], np.float32), 513).reshape(n, 1)
    spec = _spec("scatter", (4, 1), (n, 1), 0, "f32")
    got = _exact("scatter_order", spec, {"data": np.zeros((4, 1), np.float32),
                                         "index": np.full((n, 1), 2, np.int32), "values": values})
    assert got[2, 0] == 0.0


def test_scatter_computed_base_and_values_and_two_outputs():
    _case("scatter computed base/values, output twice")
    g = synth.Spec("scatter_computed")
    d = g.buffer("D", (50, 40), "f32")
    i = g.buffer("I", (90, 40), "i32")
    v = g.buffer("V", (90, 40), "f32")
    # basic IEEE operations only (an EXP would differ by its ulps)
    s = g.scatter(g.add(g.mul(d, g.const(3.0, (50, 40), "f32")), d), i, g.mul(v, v), 0)
    g.output(s, s)
    rng = np.random.default_rng(90)
    inp = {"D": rng.standard_normal((50, 40)).astype(np.float32),
           "I": rng.integers(0, 50, (90, 40)).astype(np.int32),
           "V": rng.standard_normal((90, 40)).astype(np.float32)}
    prog = _prog(g)
    a, b = run(prog, inp)
    r1, r2 = oracle.run(g, inp)
    assert a.tobytes() == r1.tobytes() and b.tobytes() == r2.tobytes()


def test_scatter_empty_index_is_the_base():
    _case("scatter empty index")
    spec = _spec("scatter", (5, 7), (0, 7), 0, "f32")
    base = np.arange(35, dtype=np.float32).reshape(5, 7)
    _exact("scatter_empty", spec, {"data": base, "index": np.zeros((0, 7), np.int32),
                                   "values": np.zeros((0, 7), np.float32)})


def test_scatter_ordered_is_repeatable():
    _case("scatter ordered twice")
    inp = synth.inputs_embedding(500, 64, 20000)
    spec = synth.embedding_scatter(500, 64, 20000)
    prog = _prog(spec)
    a, = run(prog, {k: inp[k] for k in ("values", "ids")})
    b, = run(prog, {k: inp[k] for k in ("values", "ids")})
    assert a.tobytes() == b.tobytes()


def test_scatter_full_size():
    """The benchmark's workload: 32768 rows of 1024 float32 into a zero
    (65536, 1024) table."""
    _case("embedding scatter full 65536x1024 from 32768")
    vocab, dim, n = 65536, 1024, 32768
    inp = synth.inputs_embedding(vocab, dim, n)
    _exact("embedding_scatter_full", synth.embedding_scatter(vocab, dim, n), {k: inp[k] for k in ("values", "ids")})


# ---------------------------------------------------------------------------
# atomic SCATTER
# ---------------------------------------------------------------------------

def _atomic_check(name, vocab, dim, n, dt, seed=91):
    inp = synth.inputs_embedding(vocab, dim, n, seed=seed)
    rng = np.random.default_rng(seed)
    inp["values"] = _rand(rng, (n, dim), dt)
    inp["ids"][::50] = -1
    sub = {k: inp[k] for k in ("values", "ids")}
    got, = run(_prog(synth.embedding_scatter(vocab, dim, n, dt, atomic=True)), sub)
    ref, = oracle.run(synth.embedding_scatter(vocab, dim, n, dt), sub)
    if dt == "i32":
        assert got.tobytes() == ref.tobytes()
        return
    ids = inp["ids"][:, 0]
    ok = (ids >= 0) & (ids < vocab)
    c = np.bincount(ids[ok], minlength=vocab).astype(np.float64)[:, None]
    mag = np.zeros((vocab, dim))
    np.add.at(mag, ids[ok], np.abs(inp["values"][ok].astype(np.float64)))
    u = U64 if dt == "f64" else 2.0 ** -24
    g = np.where(c * u < 1, c * u / (1 - c * u), np.inf)
    bound = 2 * g * mag + c * (2.0 ** -1022 if dt == "f64" else 2.0 ** -126)
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    report(name, err, bound)
    assert np.all(err <= bound)


@pytest.mark.parametrize("dt", ["f32", "f64", "i32"])
def test_embedding_scatter_atomic(dt):
    _case(f"embedding scatter atomic {dt}")
    _atomic_check(f"scatter_atomic_{dt}", 300, 96, 2500, dt)


def test_scatter_atomic_full_size():
    _case("embedding scatter atomic full 65536x1024 from 32768")
    _atomic_check("scatter_atomic_full", 65536, 1024, 32768, "f32", seed=9)
