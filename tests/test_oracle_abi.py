"""The oracle driven by the library's node descriptors (``oracle_run``): the
same graphs once from their movement chains (``oracle.run``) and once from
the (shape, strides, offset, mask) Views the library's View algebra
composed, bit for bit. CPU only."""

import numpy as np
import pytest

import oracle
from oracle import interp
from oracle.abi import oracle_run
from reduce_view_amd import rv, synth


def _run_both(spec, inputs):
    arr, slots = rv.nodes_from_spec(spec)
    ref = oracle.run(spec, inputs)
    outs = [np.zeros(r.shape, r.dtype) for r in ref]
    bufs = [np.ascontiguousarray(inputs[s]) for s in slots] + outs
    assert oracle_run(arr, len(arr), spec.outputs, len(spec.outputs), bufs, len(bufs)) == 0
    for a, b in zip(outs, ref):
        assert a.shape == b.shape and a.tobytes() == b.tobytes()


def _gather_scatter():
    g = synth.Spec("indexed")
    d = g.buffer("D", (6, 9, 5), "f32")
    dv = g.view(d, ("permute", (2, 1, 0)), ("pad", ((0, 0), (1, 1), (0, 0))), ("permute", (2, 1, 0)),
                ("shrink", ((0, 6), (0, 9), (0, 5))))
    i = g.buffer("I", (6, 7, 5), "i32")
    v = g.buffer("V", (6, 7, 5), "f32")
    g.output(g.gather(dv, i, 1), g.scatter(d, i, v, 1))
    rng = np.random.default_rng(3)
    return g, {"D": rng.standard_normal((6, 9, 5)).astype(np.float32),
               "I": rng.integers(-1, 10, (6, 7, 5)).astype(np.int32),
               "V": rng.standard_normal((6, 7, 5)).astype(np.float32)}


CASES = {
    "ew_chain_masked": lambda: (synth.ew_chain(37, 41, masked=True), synth.inputs_ew(37, 41)),
    "transpose": lambda: (synth.transpose(13, 29), {"X": synth.inputs_ew(13, 29)["X"]}),
    "softmax": lambda: (synth.softmax(5, 300), synth.inputs_softmax(5, 300)),
    "rmsnorm": lambda: (synth.rmsnorm(4, 256), synth.inputs_rmsnorm(4, 256)),
    "layernorm": lambda: (synth.layernorm(3, 256), synth.inputs_layernorm(3, 256)),
    "matmul": lambda: (synth.matmul_broadcast(9, 7, 11), synth.inputs_matmul(9, 7, 11)),
    "gemm": lambda: (synth.gemm_relu2_sum(16, 24, 32, emit_y=True), synth.inputs_gemm(16, 24, 32)),
    "chain_i8": lambda: (synth.chain_int(9, 17, "i8"), synth.inputs_chain_int(9, 17, "i8")),
    "attention": lambda: (synth.attention(2, 40, 56, 32, True, outputs="ol"), synth.inputs_attention(2, 40, 56, 32)),
    "indexed": _gather_scatter,
}


@pytest.mark.parametrize("name", list(CASES))
def test_descriptors_evaluate_like_the_movement_chains(name):
    spec, inputs = CASES[name]()
    _run_both(spec, inputs)


def test_wrong_buffer_count_is_refused():
    spec = synth.transpose(4, 4)
    arr, slots = rv.nodes_from_spec(spec)
    with pytest.raises(interp.OracleError):
        oracle_run(arr, len(arr), spec.outputs, 1, [np.zeros((4, 4), np.float32)], 1)
