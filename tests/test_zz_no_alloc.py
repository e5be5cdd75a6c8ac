"""rv_launch_noalloc, for callers that cannot allocate: the same programs
launched with the library's own workspace give the bits rv_launch gives with
a caller's, on consecutive calls (the second smaller than the first, so the
shared array holds the first call's leftovers), for every kernel class that
uses workspace: contraction partials, operand copies, split-reduce partials,
the ordered scatter's sort buffers, attention key-chunk partials, a cut
value."""

import ctypes

import numpy as np
import pytest

from reduce_view_amd import rv, synth
from tests.harness import to_device, to_host

pytestmark = pytest.mark.gpu


def _cut(rows, cols):
    # a permuted View of a computed value is a cut: the value goes to workspace
    g = synth.Spec(f"cut_{rows}x{cols}")
    a = g.buffer("a", (rows, cols), "f32")
    b = g.buffer("b", (rows, cols), "f32")
    s = g.add(a, b)
    g.output(g.mul(g.view(s, ("permute", (1, 0))), g.view(s, ("permute", (1, 0)))))
    return g


def _cut_inputs(rows, cols):
    rng = np.random.default_rng(31)
    return {"a": rng.standard_normal((rows, cols)).astype(np.float32),
            "b": rng.standard_normal((rows, cols)).astype(np.float32)}


# (large, small) pairs: the second call of each pair is the smaller input
PAIRS = [
    ((synth.gemm_relu2_sum(1024, 1024, 1024), synth.inputs_gemm(1024, 1024, 1024)),
     (synth.gemm_relu2_sum(512, 512, 256), synth.inputs_gemm(512, 512, 256))),
    ((synth.gemm_relu2_sum(600, 520, 200), synth.inputs_gemm(600, 520, 200)),
     (synth.gemm_relu2_sum(257, 129, 65), synth.inputs_gemm(257, 129, 65))),
    ((synth.reduce((1 << 22,), (0,)), synth.inputs_reduce((1 << 22,))),
     (synth.reduce((40009, 77), (0,)), synth.inputs_reduce((40009, 77)))),
    ((synth.embedding_scatter(4096, 64, 9000), synth.inputs_embedding(4096, 64, 9000)),
     (synth.embedding_scatter(20, 6, 100), synth.inputs_embedding(20, 6, 100))),
    ((synth.attention(1, 8192, 8192, 32, True), synth.inputs_attention(1, 8192, 8192, 32)),
     (synth.attention(1, 4100, 4100, 32, True), synth.inputs_attention(1, 4100, 4100, 32))),
    ((_cut(300, 500), _cut_inputs(300, 500)), (_cut(17, 33), _cut_inputs(17, 33))),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rv.rv_init(0)


def _bufs(prog, dev_in, outs):
    b = [rv.rv_buffer(dev_in[n].data_ptr(), dev_in[n].numel(), rv.DTYPE[rv._dtype_name(dev_in[n].dtype)], 0)
         for n in prog.slots]
    b += [rv.rv_buffer(t.data_ptr(), t.numel(), rv.DTYPE[rv._dtype_name(t.dtype)], 0) for t in outs]
    return b


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_launch_on_consecutive_calls(pair):
    import torch
    stream = torch.cuda.current_stream()
    for spec, inp in PAIRS[pair]:
        print(f"CASE no-alloc {spec.name}", flush=True)
        prog = rv.compile_spec(spec)
        assert prog.ws_bytes > 0, spec.name
        dev_in = {k: to_device(v) for k, v in inp.items() if k in prog.slots}
        ref = prog.launch(dev_in)
        torch.cuda.synchronize()
        ref = [to_host(t) for t in ref]
        outs = prog.alloc_outputs()
        for t in outs:
            t.fill_(7)
        rv.rv_launch_noalloc(prog.h, _bufs(prog, dev_in, outs), stream.cuda_stream)
        torch.cuda.synchronize()
        got = [to_host(t) for t in outs]
        for a, b in zip(ref, got):
            assert a.tobytes() == b.tobytes(), spec.name


def test_noalloc_refuses_a_program_not_loaded_on_the_device():
    # loading a code object allocates device memory: rv_launch_noalloc runs
    # only programs one rv_launch has loaded on the device
    import torch
    spec, inp = PAIRS[2][1]
    prog = rv.compile_spec(spec)
    dev_in = {k: to_device(v) for k, v in inp.items() if k in prog.slots}
    outs = prog.alloc_outputs()
    stream = torch.cuda.current_stream().cuda_stream
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch_noalloc(prog.h, _bufs(prog, dev_in, outs), stream)
    assert e.value.name == "RV_E_INVALID"
    ref = prog.launch(dev_in)
    rv.rv_launch_noalloc(prog.h, _bufs(prog, dev_in, outs), stream)
    torch.cuda.synchronize()
    for a, b in zip(ref, outs):
        assert to_host(a).tobytes() == to_host(b).tobytes()


def test_noalloc_refuses_a_program_beyond_its_size():
    import torch
    prog = rv.compile_spec(_cut(8192, 4096))  # a 128 MiB cut value
    assert prog.ws_bytes > rv.RV_SCRATCH_BYTES
    dev_in = {k: to_device(v) for k, v in {"a": np.zeros((8192, 4096), np.float32),
                                           "b": np.zeros((8192, 4096), np.float32)}.items()}
    outs = prog.alloc_outputs()
    with pytest.raises(rv.RVError) as e:
        rv.rv_launch_noalloc(prog.h, _bufs(prog, dev_in, outs), torch.cuda.current_stream().cuda_stream)
    assert e.value.name == "RV_E_WORKSPACE"
