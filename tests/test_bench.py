"""bench.py on the CPU: every program it times compiles (hipRTC needs no
device) to the kernel classes the run asserts, each timed workload's work
figure matches its program's shape, and a request for more than one GPU
ends with a message instead of a run."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture(scope="module")
def rv():
    from reduce_view_amd import rv as _rv
    return _rv


def test_configuration_programs_compile_to_the_asserted_classes(rv):
    seen = set()
    for cfg, name, spec, _mk, work, unit, bound, classes in bench.config_programs():
        got = [k["class"] for k in rv.compile_spec(spec).describe()["kernels"]]
        assert got == classes, (name, got)
        assert work > 0 and unit in ("GB/s", "TFLOP/s") and bound in ("hbm", "mfma", "latency")
        seen.add(cfg)
    assert seen == {"c1", "c2", "c3", "c4", "c5"}


def test_workload_programs_compile(rv):
    wl = bench.workloads()
    for name, w in wl.items():
        for pname, spec, work in w["programs"]:
            d = rv.compile_spec(spec).describe()
            assert d["kernels"], (name, pname)
            assert work > 0
    # the zero-operand contraction is the same program as the timed one
    g = rv.compile_spec(wl["gemm"]["programs"][0][1]).describe()
    z = rv.compile_spec(wl["gemm_zero"]["programs"][0][1]).describe()
    assert [k["name"] for k in g["kernels"]] == [k["name"] for k in z["kernels"]]
    assert [k["class"] for k in g["kernels"]] == ["MFMA", "FOLD"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
