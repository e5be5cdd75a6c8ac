"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, at sizes that span several tiles and
a ragged tail, with each config's tolerance written here and its bound
printed. Bit-exact where the pages' semantics leave one answer (movement,
transpose, in-order folds, CMPLT/WHERE branches without transcendentals)."""

import numpy as np
import pytest

import oracle
from oracle import interp
from reduce_view_amd import synth
from tests.harness import U, contraction_sum_depth, gamma, report, run, ulp32, ulp_bf16

pytestmark = pytest.mark.gpu


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


# ---- config 1: broadcast MUL + SUM over k ------------------------------------

@pytest.mark.parametrize("m,n,k", [(64, 64, 64), (4, 3, 5), (37, 70, 19), (1, 300, 7)])
def test_matmul_broadcast_in_order_is_bit_exact(m, n, k):
    _case(f"matmul {m}x{n}x{k}")
    spec = synth.matmul_broadcast(m, n, k)
    inp = synth.inputs_matmul(m, n, k, seed=0)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    absprod = np.abs(inp["A"]).astype(np.float64) @ np.abs(inp["B"]).astype(np.float64)
    report(f"matmul_{m}x{n}x{k}", np.abs(got - ref)[:, :, 0], 4 * gamma(k - 1) * absprod)
    assert got.tobytes() == ref.tobytes()


def test_matmul_raw_descriptors():
    spec = synth.matmul_broadcast_raw(33, 17, 29)
    inp = synth.inputs_matmul(33, 17, 29, seed=3)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


# ---- config 2: elementwise chain, masked chain, transpose --------------------

def _chain_check(spec, inp, name):
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.shape == ref.shape
    # where the EXP branch is not taken the chain is MUL then ADD: bit-exact;
    # elsewhere one float32 expf (2 ulp) then the ADD's rounding
    it = oracle.Interpreter(spec, inp)
    e_node = [i for i, nd in enumerate(spec.nodes) if nd["op"] == "EXP"][0]
    c_node = [i for i, nd in enumerate(spec.nodes) if nd["op"] == "CMPLT"][0]
    e = it.value(e_node)
    took_exp = it.value(c_node) == 0
    bound = np.where(took_exp, 2 * ulp32(e) + ulp32(ref), 0.0)
    report(name, np.abs(got.astype(np.float64) - ref), bound)
    assert (got[~took_exp] == ref[~took_exp]).all()
    assert np.all(np.abs(got.astype(np.float64) - ref) <= bound)


@pytest.mark.parametrize("r,c", [(256, 320), (131, 77), (4096, 4096)])
def test_ew_chain(r, c):
    _case(f"ew_chain {r}x{c}")
    inp = synth.inputs_ew(r, c, seed=1)
    _chain_check(synth.ew_chain(r, c), inp, f"ew_chain_{r}x{c}")


@pytest.mark.parametrize("r,c", [(256, 320), (131, 77), (4096, 4096)])
def test_ew_chain_masked(r, c):
    _case(f"ew_chain masked {r}x{c}")
    inp = synth.inputs_ew(r, c, seed=1)
    _chain_check(synth.ew_chain(r, c, masked=True), inp, f"ew_chain_masked_{r}x{c}")


@pytest.mark.parametrize("r,c", [(64, 64), (100, 37), (4096, 4096), (1, 513)])
def test_transpose_bit_exact(r, c):
    _case(f"transpose {r}x{c}")
    x = synth.inputs_ew(r, c, seed=1)["X"]
    got, = run(_prog(synth.transpose(r, c)), {"X": x})
    assert got.tobytes() == np.ascontiguousarray(x.T).tobytes()


# ---- config 3: softmax, RMSNorm ------------------------------------------------

@pytest.mark.parametrize("rows,n", [(64, 4096), (33, 1000), (5, 128)])
def test_softmax(rows, n):
    _case(f"softmax {rows}x{n}")
    spec = synth.softmax(rows, n)
    inp = synth.inputs_softmax(rows, n)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    bound = ref * (4 * gamma(n - 1) + 2 * 2.0 ** -23 + 4 * U) + 3 * 2.0 ** -149
    report(f"softmax_{rows}x{n}", np.abs(got - ref), bound)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= bound)


@pytest.mark.parametrize("rows,n", [(64, 4096), (33, 1000), (5, 128)])
def test_rmsnorm(rows, n):
    _case(f"rmsnorm {rows}x{n}")
    spec = synth.rmsnorm(rows, n)
    inp = synth.inputs_rmsnorm(rows, n)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    bound = np.abs(ref).astype(np.float64) * (0.5 * 4 * gamma(n - 1) + 6 * U)
    report(f"rmsnorm_{rows}x{n}", np.abs(got - ref), bound)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= bound)


@pytest.mark.parametrize("rows,n,dt", [(64, 4096, "f16"), (33, 1000, "f16"), (64, 4096, "f64"), (33, 1000, "f64")])
def test_rmsnorm_dtype_variants(rows, n, dt):
    """f64: the same bound in float64's unit. f16: every primitive rounds to
    float16, so only the float32 square sum's order differs; it can move the
    rounded sum by one float16 ulp (2^-10 relative), halved by SQRT, then
    the few per-node roundings: 4 float16 ulps of y plus |y| 2^-10."""
    _case(f"rmsnorm {dt} {rows}x{n}")
    spec = synth.rmsnorm(rows, n, dtype=dt)
    inp = synth.inputs_rmsnorm(rows, n, dtype=dt)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    g, r = got.astype(np.float64), ref.astype(np.float64)
    if dt == "f64":
        u = 2.0 ** -53
        bound = np.abs(r) * (0.5 * 4 * gamma(n - 1, u) + 6 * u)
    else:
        ulp16 = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        bound = 4 * ulp16 + np.abs(r) * 2.0 ** -10
    report(f"rmsnorm_{dt}_{rows}x{n}", np.abs(g - r), bound)
    assert np.all(np.abs(g - r) <= bound)


@pytest.mark.parametrize("rows,cols,dt", [(256, 320, "i8"), (131, 77, "i16"), (64, 1000, "i32"), (8192, 8192, "i8")])
def test_chain_int_wraps_bit_exact(rows, cols, dt):
    _case(f"chain {dt} {rows}x{cols}")
    spec = synth.chain_int(rows, cols, dt)
    inp = synth.inputs_chain_int(rows, cols, dt)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.dtype == ref.dtype and got.tobytes() == ref.tobytes()


# ---- config 4: LayerNorm (bf16 in/out) -----------------------------------------

@pytest.mark.parametrize("rows,n", [(16, 8192), (9, 1000), (3, 256)])
def test_layernorm(rows, n):
    _case(f"layernorm {rows}x{n}")
    spec = synth.layernorm(rows, n)
    inp = synth.inputs_layernorm(rows, n)
    got, = run(_prog(spec), inp)
    it = oracle.Interpreter(spec, inp)
    ref = it.value(spec.outputs[0])
    g = interp.bf16_to_f32(got).astype(np.float64)
    r = interp.bf16_to_f32(ref).astype(np.float64)
    # tolerance: the variance's reduction-order term propagates through
    # xc * r * gamma (its magnitude, not y's: y = xc*r*gamma + beta may cancel),
    # two more float32 roundings, and one bfloat16 ulp for the final CAST
    nodes = spec.nodes
    cast_out = spec.outputs[0]
    y32 = it.value(nodes[cast_out]["src"][0]).astype(np.float64)
    add_y = nodes[cast_out]["src"][0]
    prod = np.abs(it.value(nodes[add_y]["src"][0]).astype(np.float64))
    sums = [i for i, nd in enumerate(nodes) if nd["op"] == "SUM"]
    ssq = it.value(sums[1]).astype(np.float64)
    ratio = ssq / (ssq + n * 1e-5)
    bound = prod * (0.5 * 4 * gamma(n - 1) * ratio + 4 * U) + 2 * U * np.abs(y32) + ulp_bf16(np.maximum(np.abs(r), np.abs(g))) + 2.0 ** -133
    report(f"layernorm_{rows}x{n}", np.abs(g - r), bound)
    assert np.all(np.abs(g - r) <= bound)


# ---- config 5: bf16 contraction on MFMA + relu^2 + full SUM ----------------------

# the 256 x 256 four-wave kernel (five 32-deep LDS stages): k of 64, 192, 128
# (and 256, 320 below) leave 2, 1, 4, 3 and 0 k-tiles after its whole rounds
# of five; an output dim under 256 has its operand copied, zero-padded, first
@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (256, 384, 192), (256, 512, 128), (256, 256, 64),
                                   (512, 256, 192)])
def test_gemm_integer_valued_bit_exact(m, n, k):
    _case(f"gemm int {m}x{n}x{k}")
    inp = synth.inputs_gemm_integer(m, n, k)
    spec = synth.gemm_bf16(m, n, k)
    prog = _prog(spec)
    cls = [kk["class"] for kk in prog.describe()["kernels"]]
    assert cls[-1] == "MFMA" and set(cls[:-1]) <= {"EW"}, cls
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()
    # relu(y)^2 summed: exact in any order while the total stays below 2^24
    # (every partial sum of non-negative integers is then a float32 integer)
    inp = synth.inputs_gemm_integer(m, n, k, lo=-1, hi=1)
    yi = (interp.bf16_to_f32(inp["A"]).astype(np.int64) @ interp.bf16_to_f32(inp["B"]).astype(np.int64))
    assert (np.maximum(yi, 0) ** 2).sum() < 2 ** 24
    spec = synth.gemm_relu2_sum(m, n, k)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


def _gemm_strided(m, n, k, pa, pb, oa, ob):
    """A and B as windows of wider buffers: A rows of pitch k + pa starting
    at column oa, B rows of pitch n + pb starting at column ob."""
    g = synth.Spec(f"gemm_strided_{m}x{n}x{k}")
    a = g.buffer("A", (m, k + pa), "bf16")
    b = g.buffer("B", (k, n + pb), "bf16")
    aw = g.view(a, ("shrink", ((0, m), (oa, oa + k))))
    bw = g.view(b, ("shrink", ((0, k), (ob, ob + n))))
    a3 = g.cast(g.view(aw, ("reshape", (m, 1, k)), ("expand", (m, n, k))), "f32")
    b3 = g.cast(g.view(bw, ("permute", (1, 0)), ("reshape", (1, n, k)), ("expand", (m, n, k))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    return g


# operand windows with row pitches wider than the rows and nonzero offsets:
# the copy addresses' row pitch and base offsets are the View's, not k or n
@pytest.mark.parametrize("m,n,k,pa,pb,oa,ob", [(256, 256, 192, 64, 256, 8, 16), (512, 512, 320, 8, 24, 0, 8),
                                               (256, 512, 64, 1000, 8, 992, 0)])
def test_gemm_operand_windows_bit_exact(m, n, k, pa, pb, oa, ob):
    _case(f"gemm windows {m}x{n}x{k} pitches +{pa} +{pb} offsets {oa} {ob}")
    spec = _gemm_strided(m, n, k, pa, pb, oa, ob)
    prog = _prog(spec)
    kd = prog.describe()["kernels"][0]
    assert kd["class"] == "MFMA" and kd["plan"] == "gemm_w6"
    rng = np.random.default_rng(17)
    inp = {"A": synth.to_bf16_bits(rng.integers(-2, 3, (m, k + pa)).astype(np.float32)),
           "B": synth.to_bf16_bits(rng.integers(-2, 3, (k, n + pb)).astype(np.float32))}
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


# the pipeline settings the plan's environment knobs select (the default: 3 +
# 1 early copies, pinned interleaving): every one stays bit-exact on
# integer-valued operands, with B stored [k][n] and [n][k]
@pytest.mark.parametrize("knobs", [
    {"RV_GEMM_W6_PE": "0", "RV_GEMM_W6_PO": "0"},
    {"RV_GEMM_W6_PE": "12", "RV_GEMM_W6_PO": "4"},
    {"RV_GEMM_PIN": "0"},
    {"RV_GEMM_PIN": "2"},
])
def test_gemm_kernel_variants_bit_exact(monkeypatch, knobs):
    m, n, k = 512, 256, 448
    _case(f"gemm variant {knobs} {m}x{n}x{k}")
    for key, val in knobs.items():
        monkeypatch.setenv(key, val)
    inp = synth.inputs_gemm_integer(m, n, k)
    spec = synth.gemm_bf16(m, n, k)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()
    inp = {"A": inp["A"], "Bt": np.ascontiguousarray(inp["B"].T)}
    spec = synth.gemm_bf16_bt(m, n, k)
    got, = run(_prog(spec), inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (512, 384, 640), (512, 768, 320)])
def test_gemm_relu2_sum(m, n, k):
    _case(f"gemm relu2 sum {m}x{n}x{k}")
    inp = synth.inputs_gemm(m, n, k)
    spec = synth.gemm_bf16(m, n, k)
    y_gpu, = run(_prog(spec), inp)
    y_ref, = oracle.run(spec, inp)
    a = np.abs(interp.bf16_to_f32(inp["A"]).astype(np.float64))
    b = np.abs(interp.bf16_to_f32(inp["B"]).astype(np.float64))
    dy = 4 * gamma(k - 1) * (a @ b)
    report(f"gemm_y_{m}x{n}x{k}", np.abs(y_gpu - y_ref)[:, :, 0], dy)
    assert np.all(np.abs(y_gpu - y_ref)[:, :, 0] <= dy)
    spec = synth.gemm_relu2_sum(m, n, k)
    prog = _prog(spec)
    desc = prog.describe()
    s_gpu, = run(prog, inp)
    s_ref, = oracle.run(spec, inp)
    y = y_ref[:, :, 0].astype(np.float64)
    q = np.maximum(y, 0) ** 2
    depth = contraction_sum_depth(desc)
    ds = (np.sum((2 * np.abs(y) * dy + dy ** 2) * (y > -dy)) + U * q.sum() + 4 * gamma(depth) * q.sum()
          + U * abs(float(s_ref.ravel()[0])))
    report(f"gemm_S_{m}x{n}x{k}", np.array([abs(float(s_gpu.ravel()[0]) - float(s_ref.ravel()[0]))]), np.array([ds]))
    assert abs(float(s_gpu.ravel()[0]) - float(s_ref.ravel()[0])) <= ds


@pytest.mark.parametrize("m,n,k", [(256, 256, 128), (128, 256, 64), (512, 256, 320)])
def test_gemm_k_contiguous_second_operand_bit_exact(m, n, k):
    _case(f"gemm bt int {m}x{n}x{k}")
    inp = synth.inputs_gemm_integer(m, n, k)
    inp = {"A": inp["A"], "Bt": np.ascontiguousarray(inp["B"].T)}
    spec = synth.gemm_bf16_bt(m, n, k)
    prog = _prog(spec)
    cls = [kk["class"] for kk in prog.describe()["kernels"]]
    assert cls[-1] == "MFMA" and set(cls[:-1]) <= {"EW"}, cls
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


# ---- full sizes, in the launch configuration the benchmark times -------------

def test_softmax_full_size():
    _case("softmax full 16384x4096")
    test_softmax(16384, 4096)


def test_rmsnorm_full_size():
    _case("rmsnorm full 16384x4096")
    test_rmsnorm(16384, 4096)


def test_rmsnorm_dtype_variants_full_size():
    _case("rmsnorm f16 and f64 full 16384x4096")
    test_rmsnorm_dtype_variants(16384, 4096, "f16")
    test_rmsnorm_dtype_variants(16384, 4096, "f64")


def test_layernorm_full_size():
    _case("layernorm full 8192x8192")
    test_layernorm(8192, 8192)


def test_gemm_full_size_sampled_rows_and_scalar():
    """4096^3: y on sampled rows against the oracle computed for those rows
    only, and S = SUM(relu(y)^2) against the stored oracle value."""
    import json
    import os
    _case("gemm full 4096^3")
    m = n = k = 4096
    inp = synth.inputs_gemm(m, n, k, seed=5)
    y_gpu, = run(_prog(synth.gemm_bf16(m, n, k)), inp)
    rows = [0, 1, 2047, 4095]
    sub = {"A": inp["A"][rows], "B": inp["B"]}
    y_ref, = oracle.run(synth.gemm_bf16(len(rows), n, k), sub)
    a = np.abs(interp.bf16_to_f32(sub["A"]).astype(np.float64))
    b = np.abs(interp.bf16_to_f32(inp["B"]).astype(np.float64))
    dy = 4 * gamma(k - 1) * (a @ b)
    err = np.abs(y_gpu[rows, :, 0].astype(np.float64) - y_ref[:, :, 0])
    report("gemm_full_y_rows", err, dy)
    assert np.all(err <= dy)
    path = os.path.join(os.path.dirname(__file__), "golden", "gemm_relu2_sum_4096.json")
    gold = json.load(open(path))
    prog = _prog(synth.gemm_relu2_sum(m, n, k))
    desc = prog.describe()
    s_gpu, = run(prog, inp)
    depth = contraction_sum_depth(desc)
    ds = gold["propagated_y_term"] + U * gold["sum_q"] + 4 * gamma(depth) * gold["sum_q"] + U * abs(gold["S"])
    e = abs(float(s_gpu.ravel()[0]) - gold["S"])
    report("gemm_full_S", np.array([e]), np.array([ds]))
    assert e <= ds


def test_graph_replay_matches_eager():
    """Launches captured in a HIP graph (torch.cuda.CUDAGraph on a side
    stream) and replayed several times, with eager launches and
    synchronisations between the replays, give the eager result every time
    (the contraction's program includes its partials + fold)."""
    import torch
    from tests.harness import to_device, to_host
    stream = torch.cuda.Stream()
    cases = [(synth.ew_chain(256, 320, masked=True), synth.inputs_ew(256, 320)),
             (synth.gemm_relu2_sum(256, 256, 128), synth.inputs_gemm(256, 256, 128)),
             (synth.softmax(64, 1024), synth.inputs_softmax(64, 1024))]
    for spec, inp in cases:
        _case(f"graph replay {spec.name}")
        prog = _prog(spec)
        dev = {k: to_device(v) for k, v in inp.items() if k in prog.slots}
        with torch.cuda.stream(stream):
            eager_out = prog.alloc_outputs()
            graph_out = prog.alloc_outputs()
            ws = prog.workspace()
            ws2 = torch.empty_like(ws) if ws is not None else None
            go_eager = prog.prepare(dev, eager_out, stream, ws)
            go_graph = prog.prepare(dev, graph_out, stream, ws2)
            go_eager()
            go_graph()  # loads the module before capture
            torch.cuda.synchronize()
            ref = [to_host(t) for t in eager_out]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                go_graph()
            for rep in range(3):
                for t in graph_out:
                    t.zero_()
                go_eager()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                for a, b in zip(ref, graph_out):
                    assert a.tobytes() == to_host(b).tobytes(), (spec.name, rep)


# ---- ragged contractions: still on the matrix cores ----------------------------

@pytest.mark.parametrize("m,n,k,bt", [(257, 129, 65, False), (255, 257, 31, False), (300, 257, 64, False),
                                      (520, 300, 96, True), (1, 1, 1, False), (33, 300, 200, True),
                                      (256, 256, 32, False)])
def test_gemm_ragged_integer_bit_exact(m, n, k, bt):
    """Every tile width and tail (limn README, "Correctness"): a last tile
    shifted back inside the operands, operands copied zero-padded into
    workspace; integer-valued operands are exact in any order."""
    _case(f"gemm ragged int {m}x{n}x{k} bt={bt}")
    from tests.test_lowering import _gemm_views
    spec = _gemm_views(m, n, k, bt=bt)
    prog = _prog(spec)
    assert [kk["class"] for kk in prog.describe()["kernels"]].count("MFMA") == 1
    inp = synth.inputs_gemm_integer(m, n, k)
    if bt:
        inp = {"A": inp["A"], "B": np.ascontiguousarray(inp["B"].T)}
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


def test_gemm_ragged_full_rows_sampled():
    """4095 x 4096 x 4096: the last row tile starts at 3839 and leaves its
    first row to the tile before it; sampled rows on both sides of the seam
    against the oracle (integer-valued operands: exact in any order)."""
    _case("gemm ragged 4095x4096x4096")
    m = 4095
    n = k = 4096
    inp = synth.inputs_gemm_integer(m, n, k)
    prog = _prog(synth.gemm_bf16(m, n, k))
    pd = [kk for kk in prog.describe()["kernels"] if kk["class"] == "MFMA"][0]["plan_detail"]
    assert pd["ragged"] and pd["copied"] == {"A": False, "B": False}
    got, = run(prog, inp)
    rows = [0, 3838, 3839, 3840, 4094]
    ref, = oracle.run(synth.gemm_bf16(len(rows), n, k), {"A": inp["A"][rows], "B": inp["B"]})
    assert got[rows].tobytes() == ref.tobytes()


def test_gemm_transposed_padded_operands_bit_exact():
    """A read through a transposing View and B through a padding View: both
    are copied (transposed / zero-padded) into workspace, then contracted."""
    _case("gemm transposed + padded operands")
    g = synth.Spec("gemm_t")
    a = g.buffer("A", (96, 300), "bf16")
    b = g.buffer("B", (90, 260), "bf16")
    a2 = g.view(a, ("permute", (1, 0)))
    b2 = g.view(b, ("pad", ((3, 3), (0, 0))))
    a3 = g.cast(g.view(a2, ("reshape", (300, 1, 96)), ("expand", (300, 260, 96))), "f32")
    b3 = g.cast(g.view(b2, ("permute", (1, 0)), ("reshape", (1, 260, 96)), ("expand", (300, 260, 96))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    rng = np.random.default_rng(29)
    inp = {"A": synth.to_bf16_bits(rng.integers(-2, 3, (96, 300)).astype(np.float32)),
           "B": synth.to_bf16_bits(rng.integers(-2, 3, (90, 260)).astype(np.float32))}
    got, = run(_prog(g), inp)
    ref, = oracle.run(g, inp)
    assert got.tobytes() == ref.tobytes()


def _split_k(desc):
    mf = [kk for kk in desc["kernels"] if kk["class"] == "MFMA"]
    return mf[0]["plan_detail"]["split_k"], [kk["plan"] for kk in mf]


# few output tiles over a deep k: the contraction is split into k-slices
# whose raw planes a second kernel folds in slice order before the
# epilogue; integer-valued operands are exact in any order. Ragged tiles,
# copied operands, B stored [n][k], and forced slice counts.
@pytest.mark.parametrize("m,n,k,bt,force", [(256, 512, 2048, False, None), (300, 520, 2048, False, None),
                                            (256, 768, 1024, True, None), (40, 24, 1024, False, None),
                                            (256, 512, 2048, False, "2"), (256, 256, 4096, True, "16"),
                                            (1000, 700, 1536, False, "4")])
def test_gemm_split_k_integer_bit_exact(monkeypatch, m, n, k, bt, force):
    _case(f"gemm split-k int {m}x{n}x{k} bt={bt} force={force}")
    if force:
        monkeypatch.setenv("RV_GEMM_SPLITK", force)
    from tests.test_lowering import _gemm_views
    spec = _gemm_views(m, n, k, bt=bt)
    prog = _prog(spec)
    S, plans = _split_k(prog.describe())
    assert plans == ["gemm_w6", "gemm_slices"] and S == (int(force) if force else S) and S > 1, (S, plans)
    inp = synth.inputs_gemm_integer(m, n, k)
    if bt:
        inp = {"A": inp["A"], "B": np.ascontiguousarray(inp["B"].T)}
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("m,n,k", [(256, 512, 2048), (300, 520, 2048)])
def test_gemm_split_k_relu2_sum_integer_bit_exact(m, n, k):
    """The relu^2 + SUM epilogue on the slices' fold: its per-workgroup
    partials and their fold, exact while the total stays below 2^24."""
    _case(f"gemm split-k relu2 sum int {m}x{n}x{k}")
    # sparse -1 / 0 / 1 operands keep the deep sums small
    rng = np.random.default_rng(31)
    inp = {"A": synth.to_bf16_bits(rng.choice([-1.0, 0.0, 1.0], (m, k), p=[0.05, 0.9, 0.05]).astype(np.float32)),
           "B": synth.to_bf16_bits(rng.choice([-1.0, 0.0, 1.0], (k, n), p=[0.05, 0.9, 0.05]).astype(np.float32))}
    yi = (interp.bf16_to_f32(inp["A"]).astype(np.int64) @ interp.bf16_to_f32(inp["B"]).astype(np.int64))
    assert (np.maximum(yi, 0) ** 2).sum() < 2 ** 24
    spec = synth.gemm_relu2_sum(m, n, k)
    prog = _prog(spec)
    desc = prog.describe()
    assert _split_k(desc)[0] > 1 and [kk["class"] for kk in desc["kernels"]][-3:] == ["MFMA", "MFMA", "FOLD"]
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


def test_gemm_split_k_1024x1024x8192_sampled():
    """1024 x 1024 x 8192 (16 output tiles, split over k) on random operands:
    sampled rows, on both sides of a tile seam, within the contraction's
    rounding bound against the oracle."""
    _case("gemm split-k 1024x1024x8192")
    m, n, k = 1024, 1024, 8192
    inp = synth.inputs_gemm(m, n, k, seed=9)
    prog = _prog(synth.gemm_bf16(m, n, k))
    assert _split_k(prog.describe())[0] > 1
    y_gpu, = run(prog, inp)
    rows = [0, 255, 256, 1023]
    sub = {"A": inp["A"][rows], "B": inp["B"]}
    y_ref, = oracle.run(synth.gemm_bf16(len(rows), n, k), sub)
    a = np.abs(interp.bf16_to_f32(sub["A"]).astype(np.float64))
    b = np.abs(interp.bf16_to_f32(inp["B"]).astype(np.float64))
    dy = 4 * gamma(k - 1) * (a @ b)
    err = np.abs(y_gpu[rows, :, 0].astype(np.float64) - y_ref[:, :, 0])
    report("gemm_split_y_rows", err, dy)
    assert np.all(err <= dy)


# the generated epilogue reading operands of its own at (m, n), one through a
# masked View, in place, over ragged tiles and on the slices' fold:
# integer-valued, so y * s + c is exact and the bf16 rounding is the oracle's
@pytest.mark.parametrize("m,n,k,plans", [(1024, 768, 256, ["gemm_w6"]), (300, 260, 192, ["gemm_w6"]),
                                         (256, 512, 2048, ["gemm_w6", "gemm_slices"])])
def test_gemm_epilogue_operands_bit_exact(m, n, k, plans):
    _case(f"gemm epilogue operands {m}x{n}x{k}")
    from tests.test_lowering import _gemm_affine, _gemm_affine_inputs
    spec = _gemm_affine(m, n, k)
    prog = _prog(spec)
    assert [kk["plan"] for kk in prog.describe()["kernels"] if kk["class"] == "MFMA"] == plans
    inp = _gemm_affine_inputs(m, n, k)
    got, = run(prog, inp)
    ref, = oracle.run(spec, inp)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("m,n,k", [(520, 300, 96), (257, 129, 65)])
def test_gemm_ragged_relu2_sum(m, n, k):
    """The relu^2 + SUM epilogue over ragged tiles: cells a shifted tile
    shares with the tile before it, and padded rows and columns, are left out
    of the partials."""
    _case(f"gemm ragged relu2 sum {m}x{n}x{k}")
    inp = synth.inputs_gemm(m, n, k)
    spec = synth.gemm_relu2_sum(m, n, k)
    prog = _prog(spec)
    desc = prog.describe()
    assert [kk["class"] for kk in desc["kernels"]][-2:] == ["MFMA", "FOLD"]
    s_gpu, = run(prog, inp)
    s_ref, = oracle.run(spec, inp)
    y_gpu, = run(_prog(synth.gemm_bf16(m, n, k)), inp)
    y_ref, = oracle.run(synth.gemm_bf16(m, n, k), inp)
    a = np.abs(interp.bf16_to_f32(inp["A"]).astype(np.float64))
    b = np.abs(interp.bf16_to_f32(inp["B"]).astype(np.float64))
    dy = 4 * gamma(k - 1) * (a @ b)
    assert np.all(np.abs(y_gpu - y_ref)[:, :, 0] <= dy)
    y = y_ref[:, :, 0].astype(np.float64)
    q = np.maximum(y, 0) ** 2
    depth = contraction_sum_depth(desc)
    ds = (np.sum((2 * np.abs(y) * dy + dy ** 2) * (y > -dy)) + U * q.sum() + 4 * gamma(depth) * q.sum()
          + U * abs(float(s_ref.ravel()[0])))
    e = abs(float(s_gpu.ravel()[0]) - float(s_ref.ravel()[0]))
    report(f"gemm_ragged_S_{m}x{n}x{k}", np.array([e]), np.array([ds]))
    assert e <= ds
