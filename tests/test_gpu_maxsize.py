"""GPU parity past 2^31 cells: every index and address the kernels form must
be 64-bit once a buffer holds more cells than an int32 counts (limn README,
"The op set": a View addresses its buffer through offset + sum of index times
stride, with no width stated; HBM of 288 GB holds such buffers easily).

int8 keeps the buffers at 2 GB each. Integer results are exact, so every
check is bit for bit against the oracle: sampled rows (including the rows on
both sides of cell 2^31) for the elementwise and row workloads, evaluated by
the oracle on those rows alone (their cells depend on nothing else), and the
whole input for the full SUM."""

import numpy as np
import pytest

import oracle
from reduce_view_amd import synth
from tests.harness import run

pytestmark = pytest.mark.gpu

ROWS, COLS = 65537, 32768  # (ROWS - 1) * COLS = 2^31: row 65536 starts at cell 2^31


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


def _i8(rng, shape):
    return rng.integers(-128, 128, shape, dtype=np.int8)


def test_chain_i8_past_2p31_cells():
    _case("chain_i8 65537x32768")
    rng = np.random.default_rng(31)
    inp = {k: _i8(rng, (ROWS, COLS)) for k in ("a", "b", "c")}
    spec = synth.chain_int(ROWS, COLS, "i8")
    got = run(_prog(spec), inp)[0]
    rows = [0, 1, 32768, ROWS - 2, ROWS - 1]
    ref = oracle.run(synth.chain_int(len(rows), COLS, "i8"), {k: v[rows] for k, v in inp.items()})[0]
    assert np.array_equal(got[rows], ref)


def test_row_sum_i8_past_2p31_cells():
    _case("row SUM i8 65537x32768")
    rng = np.random.default_rng(32)
    x = _i8(rng, (ROWS, COLS))
    prog = _prog(synth.reduce((ROWS, COLS), (1,), dtype="i8"))
    got = run(prog, {"x": x})[0]
    rows = [0, 32768, ROWS - 2, ROWS - 1]
    ref = oracle.run(synth.reduce((len(rows), COLS), (1,), dtype="i8"), {"x": x[rows]})[0]
    assert np.array_equal(got[rows], ref)


def test_full_sum_i8_past_2p31_cells():
    n = (1 << 31) + 4096
    _case(f"full SUM i8 of {n}")
    rng = np.random.default_rng(33)
    x = _i8(rng, (n,))
    spec = synth.reduce((n,), (0,), dtype="i8")
    prog = _prog(spec)
    assert [k["class"] for k in prog.describe()["kernels"]] == ["SPLIT", "FOLD"]
    got = run(prog, {"x": x})[0]
    ref = oracle.run(spec, {"x": x}, max_elems=1 << 32)[0]
    assert np.array_equal(got, ref)


def test_transpose_i8_past_2p31_cells():
    m = 46341  # m * m = 2^31 + 4633
    _case(f"transpose i8 {m}x{m}")
    rng = np.random.default_rng(34)
    x = _i8(rng, (m, m))
    got = run(_prog(synth.transpose(m, m, "i8")), {"X": x})[0]
    for lo in (0, m // 2 - 32, m - 64):
        ref = oracle.run(synth.transpose(m, 64, "i8"), {"X": np.ascontiguousarray(x[:, lo:lo + 64])})[0]
        assert np.array_equal(got[lo:lo + 64], ref), lo


def test_contraction_bf16_operand_past_2p31_cells():
    m, n, k = ROWS, 256, COLS  # A holds 2^31 + 32768 bf16 cells
    _case(f"contraction bf16 {m}x{n}x{k}")
    rng = np.random.default_rng(35)
    # integer-valued operands in [-2, 2]: every partial sum is an integer
    # below 2^24, exact in float32 in any order
    bits = synth.to_bf16_bits(np.arange(-2, 3, dtype=np.float32))
    a = bits[rng.integers(0, 5, (m, k), dtype=np.int8)]
    b = bits[rng.integers(0, 5, (k, n), dtype=np.int8)]
    prog = _prog(synth.gemm_bf16(m, n, k))
    assert [x["class"] for x in prog.describe()["kernels"]] == ["MFMA"]
    got = run(prog, {"A": a, "B": b})[0]
    rows = [0, 1, 32768, m - 257, m - 256, m - 2, m - 1]
    ref = oracle.run(synth.gemm_bf16(len(rows), n, k), {"A": a[rows], "B": b})[0]
    assert np.array_equal(got[rows], ref)
