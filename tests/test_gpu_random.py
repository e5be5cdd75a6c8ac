"""GPU parity over random small regions (the generator in test_lowering:
direct, transposed, broadcast-row and windowed operands, mixed elementwise
ops, reduce and row-reduce tails): the HIP kernels, through the C ABI,
reproduce the oracle bit for bit on integer-valued inputs."""

import pytest

import oracle
from tests.harness import run
from tests.test_lowering import random_region

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from reduce_view_amd import rv
    rv.rv_init(0)


@pytest.mark.parametrize("seed", range(40))
def test_random_region_matches_oracle(seed):
    from reduce_view_amd import rv
    print(f"CASE random region {seed}", flush=True)
    g, inputs = random_region(seed)
    got = run(rv.compile_spec(g), inputs)
    ref = oracle.run(g, inputs)
    assert got[0].tobytes() == ref[0].tobytes()


# the same regions stored in bfloat16, float16 and int32 (small integers:
# exact in every dtype; narrow floats round once at the store, as the oracle)
@pytest.mark.parametrize("dt", ["bf16", "f16", "i32"])
@pytest.mark.parametrize("seed", range(12))
def test_random_region_dtypes_match_oracle(dt, seed):
    from reduce_view_amd import rv
    print(f"CASE random region {dt} {seed}", flush=True)
    g, inputs = random_region(seed, dt)
    got = run(rv.compile_spec(g), inputs)
    ref = oracle.run(g, inputs)
    assert got[0].tobytes() == ref[0].tobytes()
