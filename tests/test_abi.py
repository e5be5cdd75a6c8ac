"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and every typed error of the contract can be forced without a GPU
(Tiki README, "Compile model code": unsupported ops, layouts or devices raise
a typed error naming the contract)."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

from reduce_view_amd import rv, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "rv.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = set(re.findall(r"\b(rv_[a-z_]+)\s*\(", header))
    assert declared == set(rv.EXPORTS)
    lib = ctypes.CDLL(rv.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (rv_[a-z_]+)", out))
    assert declared <= exported


def _status(fn, *a):
    with pytest.raises(rv.RVError) as e:
        fn(*a)
    return e.value.name


def test_view_errors():
    v = rv.rv_view_contiguous((4, 6))
    assert _status(rv.rv_view_expand, v, (8, 6)) == "RV_E_INVALID"
    assert _status(rv.rv_view_shrink, v, (0, 0), (5, 6)) == "RV_E_INVALID"
    assert _status(rv.rv_view_pad, v, (-1, 0), (0, 0)) == "RV_E_INVALID"
    assert _status(rv.rv_view_permute, v, (0, 0)) == "RV_E_INVALID"
    t = rv.rv_view_permute(v, (1, 0))
    assert _status(rv.rv_view_reshape, t, (24,)) == "RV_E_UNSUPPORTED_LAYOUT"
    m = rv.rv_view_pad(v, (1, 0), (0, 0))
    assert _status(rv.rv_view_reshape, m, (30,)) == "RV_E_UNSUPPORTED_LAYOUT"
    assert _status(rv.rv_view_reshape, v, (5, 5)) == "RV_E_INVALID"


def _compile_status(spec):
    return _status(rv.compile_spec, spec)


def test_graph_errors():
    g = synth.Spec()
    x = g.buffer("x", (4,), "f32")
    g.output(g.raw_view(x, (4,), (2,)))  # reads element 6 of 4
    assert _compile_status(g) == "RV_E_OUT_OF_BOUNDS"
    g = synth.Spec()
    x = g.buffer("x", (4,), "f32")
    g.output(g.raw_view(x, (2,), (-1,), offset=3))
    assert _compile_status(g) == "RV_E_UNSUPPORTED_LAYOUT"
    g = synth.Spec()
    x = g.buffer("x", (4,), "f32")
    g.output(g.raw_view(x, (4,), (1,), mask_lo=(0,), mask_hi=(5,)))
    assert _compile_status(g) == "RV_E_INVALID"
    g = synth.Spec()
    a = g.buffer("a", (4,), "f32")
    b = g.buffer("b", (4,), "bf16")
    g.output(g.add(a, b))
    assert _compile_status(g) == "RV_E_DTYPE"
    g = synth.Spec()
    a = g.buffer("a", (4,), "i32")
    g.output(g.exp(a))
    assert _compile_status(g) == "RV_E_DTYPE"
    g = synth.Spec()
    a = g.buffer("a", (4,), "f32")
    b = g.buffer("b", (5,), "f32")
    g.output(g.mul(a, b))
    assert _compile_status(g) == "RV_E_INVALID"
    for op in ("ASSIGN", "CUSTOM"):
        g = synth.Spec()
        a = g.buffer("a", (4,), "f32")
        g.output(g._add(op=op, src=(a,)))
        assert _compile_status(g) == "RV_E_UNSUPPORTED_OP", op


def _indexed(kind, dshape=(4, 5), ishape=(3, 5), axis=0, idt="i32", dt="f32", vdt=None, vshape=None, atomic=False):
    g = synth.Spec()
    d = g.buffer("d", dshape, dt)
    i = g.buffer("i", ishape, idt)
    if kind == "gather":
        g.output(g.gather(d, i, axis))
    else:
        v = g.buffer("v", vshape or ishape, vdt or dt)
        g.output(g.scatter(d, i, v, axis, atomic))
    return g


def _status_or_ok(spec):
    try:
        rv.compile_spec(spec)
    except rv.RVError as e:
        return e.name
    return "OK"


def test_indexed_op_contract_errors():
    for kind in ("gather", "scatter"):
        assert _status_or_ok(_indexed(kind)) == "OK"
        assert _status_or_ok(_indexed(kind, idt="i16")) == "RV_E_DTYPE"
        assert _status_or_ok(_indexed(kind, ishape=(3, 4))) == "RV_E_INVALID"  # differs off the axis
        assert _status_or_ok(_indexed(kind, ishape=(3, 5, 1))) == "RV_E_INVALID"  # rank
        assert _status_or_ok(_indexed(kind, axis=2)) == "RV_E_INVALID"  # axis outside the rank
    assert _status_or_ok(_indexed("scatter", vdt="f64")) == "RV_E_DTYPE"
    assert _status_or_ok(_indexed("scatter", vshape=(2, 5))) == "RV_E_INVALID"
    for dt in ("f32", "f64", "i32"):
        assert _status_or_ok(_indexed("scatter", dt=dt, atomic=True)) == "OK", dt
    for dt in ("f16", "bf16", "i16", "i8"):
        assert _status_or_ok(_indexed("scatter", dt=dt, atomic=True)) == "RV_E_UNSUPPORTED_OP", dt
        assert _status_or_ok(_indexed("scatter", dt=dt)) == "OK", dt


def test_no_device_is_a_typed_error():
    code = ("import sys; sys.path.insert(0, %r); from reduce_view_amd import rv\n"
            "try:\n    rv.rv_init(0)\n    print('OK')\nexcept rv.RVError as e:\n    print(e.name, str(e))\n") % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120).stdout
    assert out.startswith("RV_E_DEVICE"), out


def test_injected_compile_failure():
    code = ("import sys; sys.path.insert(0, %r); from reduce_view_amd import rv, synth\n"
            "try:\n    rv.compile_spec(synth.transpose(8, 8))\n    print('OK')\nexcept rv.RVError as e:\n"
            "    print(e.name)\n") % ROOT
    env = dict(os.environ, RV_DEBUG_BAD_SOURCE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300).stdout
    assert out.strip() == "RV_E_COMPILE", out


class _Fake:
    """A stand-in buffer (never dereferenced: launch validation fails first)."""

    def __init__(self, nelems, dtype):
        self.n, self.dt = nelems, dtype


def _bufs(prog, sizes, dtypes, base=1 << 20):
    out = []
    for i, (n, dt) in enumerate(zip(sizes, dtypes)):
        out.append(rv.rv_buffer(base * (i + 1) * 64, n, rv.DTYPE[dt], 0))
    return out


def test_launch_validation_errors_without_device():
    prog = rv.compile_spec(synth.gemm_relu2_sum(128, 128, 64))
    assert prog.ws_bytes > 0
    good = _bufs(prog, [128 * 64, 64 * 128, 1], ["bf16", "bf16", "f32"])
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch(prog.h, good, 0, 0, 0)
    assert e.value.name == "RV_E_WORKSPACE"
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch(prog.h, good, 1 << 30, 16, 0)
    assert e.value.name == "RV_E_WORKSPACE"
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch(prog.h, good[:2], 1 << 30, prog.ws_bytes, 0)
    assert e.value.name == "RV_E_INVALID"
    bad = _bufs(prog, [128 * 64, 64 * 128, 1], ["f32", "bf16", "f32"])
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch(prog.h, bad, 1 << 30, prog.ws_bytes, 0)
    assert e.value.name == "RV_E_DTYPE"
    small = _bufs(prog, [100, 64 * 128, 1], ["bf16", "bf16", "f32"])
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch(prog.h, small, 1 << 30, prog.ws_bytes, 0)
    assert e.value.name == "RV_E_INVALID"
    alias = [good[0], good[1], rv.rv_buffer(good[0].ptr, 1, rv.DTYPE["f32"], 0)]
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch(prog.h, alias, 1 << 30, prog.ws_bytes, 0)
    assert e.value.name == "RV_E_INVALID" and "overlaps" in str(e.value)


def test_program_io_and_describe():
    prog = rv.compile_spec(synth.softmax(32, 512))
    assert (prog.n_inputs, prog.n_outputs) == (1, 1)
    assert prog.out_desc == [((32, 512), "f32")]
    d = prog.describe()
    assert [k["class"] for k in d["kernels"]] == ["ROW"]
    assert d["kernels"][0]["name"].startswith("rv_row_row_") and d["kernels"][0]["name"] in prog.source()
    assert rv.rv_last_error() == ""


def test_attention_scale_must_be_positive():
    # the kernel's running maximum of the scaled scores is max(s) * scale and
    # masked keys are set to -inf before scaling: a scale <= 0 is refused
    for scale, want in ((0.25, "OK"), (0.0, "RV_E_INVALID"), (-0.25, "RV_E_INVALID"),
                        (float("inf"), "RV_E_INVALID"), (float("nan"), "RV_E_INVALID")):
        g = synth.Spec()
        q = g.buffer("q", (1, 16, 32), "bf16")
        k = g.buffer("k", (1, 16, 32), "bf16")
        v = g.buffer("v", (1, 16, 32), "bf16")
        g.output(g.sdpa(q, k, v, scale, causal=True)[0])
        assert _status_or_ok(g) == want, scale


def test_ordered_scatter_key_count_limit():
    # 65536 targets along the axis times 32768 index columns the index varies
    # along: 2^31 keys do not fit the 31-bit key words
    def spec(cols):
        g = synth.Spec()
        base = g.const(0.0, (65536, cols), "f32")
        i = g.buffer("i", (1, cols), "i32")
        v = g.buffer("v", (1, cols), "f32")
        g.output(g.scatter(base, i, v, 0))
        return g
    assert _status_or_ok(spec(32767)) == "OK"
    assert _status_or_ok(spec(32768)) == "RV_E_INVALID"


def test_caller_workspace_size_is_checked():
    # a caller-supplied workspace smaller than the program needs is refused
    # before anything reaches the device (host tensors stand in for buffers)
    import torch
    prog = rv.compile_spec(synth.gemm_relu2_sum(128, 128, 64))
    prog.slots = ["A", "B"]
    inputs = {"A": torch.zeros(128 * 64, dtype=torch.bfloat16), "B": torch.zeros(64 * 128, dtype=torch.bfloat16)}
    out = [torch.zeros(1, dtype=torch.float32)]

    class _Stream:
        cuda_stream = 0
    small = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(rv.RVError) as e:
        prog.launch(inputs, out, stream=_Stream(), workspace=small)
    assert e.value.name == "RV_E_WORKSPACE"
    with pytest.raises(rv.RVError) as e:
        prog.prepare(inputs, out, _Stream(), workspace=small)()
    assert e.value.name == "RV_E_WORKSPACE"
