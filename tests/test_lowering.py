"""Scheduler and lowering on the CPU (no GPU): the kernel classes each
workload is cut into, the limn IR dump's structure for (4, 5) @ (5, 3), and
a lowered-plan interpreter (tests/plan_interp.py) that executes what
rv_describe says the kernels do and diffs it against the oracle."""

import os

import numpy as np
import pytest

import oracle
from oracle import interp as O
from reduce_view_amd import rv, synth
from tests.harness import U, gamma
from tests.plan_interp import run_plan

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name):
    facts = {}
    for line in open(os.path.join(HERE, "golden", name)):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        facts[k] = v
    return facts


def test_limn_ir_dump_structure():
    f = _golden("limn_ir_matmul_4x5x3.txt")
    prog = rv.compile_spec(synth.matmul_broadcast(4, 3, 5))
    d = prog.describe()
    assert len(d["kernels"]) == int(f["kernels"][0])
    k = d["kernels"][0]
    assert k["class"] == "REDUCE"
    assert k["domain"] == [int(x) for x in f["domain"]]
    assert k["reduce_dims"] == [int(x) for x in f["reduce_dims"]]
    strides = sorted(tuple(L["view"]["strides"]) for L in k["leaves"])
    assert strides == sorted([tuple(int(x) for x in f["in0_strides"]), tuple(int(x) for x in f["in1_strides"])])
    assert tuple(k["stores"][0]["view"]["strides"]) == tuple(int(x) for x in f["out_strides"])
    assert prog.out_desc[0][0] == tuple(int(x) for x in f["out_shape"])
    assert k["lane_dim"] == int(f["innermost_dim"][0])
    ops = [o["op"] for o in k["ops"]]
    assert ops.count("SUM") == 1 and "MUL" in ops
    src = prog.source()
    assert "float acc = 0.0f;" in src  # identity fill 0.0, then ACCUM ADD


def _interp(spec, inputs):
    prog = rv.compile_spec(spec)
    d = prog.describe()
    flat = [np.ascontiguousarray(inputs[s]).ravel() for s in prog.slots]
    outs = run_plan(d, flat, prog.out_desc)
    return d, outs


CLASSES = {
    "matmul": (lambda: synth.matmul_broadcast(7, 5, 9), lambda: synth.inputs_matmul(7, 5, 9), ["REDUCE"]),
    "ew": (lambda: synth.ew_chain(19, 23), lambda: synth.inputs_ew(19, 23), ["EW"]),
    "ew_masked": (lambda: synth.ew_chain(19, 23, masked=True), lambda: synth.inputs_ew(19, 23), ["EW"]),
    "transpose": (lambda: synth.transpose(13, 29), lambda: {"X": synth.inputs_ew(13, 29)["X"]}, ["EW"]),
    "softmax": (lambda: synth.softmax(6, 300), lambda: synth.inputs_softmax(6, 300), ["ROW"]),
    "rmsnorm": (lambda: synth.rmsnorm(6, 300), lambda: synth.inputs_rmsnorm(6, 300), ["ROW"]),
    "layernorm": (lambda: synth.layernorm(5, 256), lambda: synth.inputs_layernorm(5, 256), ["ROW"]),
    "gemm": (lambda: synth.gemm_relu2_sum(256, 256, 64), lambda: synth.inputs_gemm(256, 256, 64),
             ["MFMA", "FOLD"]),
    "gemm_y": (lambda: synth.gemm_bf16(256, 256, 128), lambda: synth.inputs_gemm(256, 256, 128), ["MFMA"]),
    # narrow and ragged extents: the operands are copied, zero-padded, first
    "gemm_copied": (lambda: synth.gemm_relu2_sum(100, 130, 70), lambda: synth.inputs_gemm(100, 130, 70),
                    ["EW", "EW", "MFMA", "FOLD"]),
    "gemm_y_ragged": (lambda: synth.gemm_bf16(257, 260, 128), lambda: synth.inputs_gemm(257, 260, 128),
                      ["EW", "MFMA"]),
    # K no multiple of the 64-deep k-step: both operands padded along K
    "gemm_k96": (lambda: synth.gemm_bf16(257, 260, 96), lambda: synth.inputs_gemm(257, 260, 96),
                 ["EW", "EW", "MFMA"]),
    # operands as windows of wider buffers, each a View of a View: the two
    # compose into one View of the buffer, so nothing is copied first
    "gemm_windows": (lambda: _gemm_windows(), lambda: _gemm_windows_inputs(), ["MFMA"]),
    # one output tile, k deep enough to split: k-slices (raw planes), then
    # their fold with the epilogue; small integers make every sum exact, so
    # the slices' order matches the oracle's bit for bit
    "gemm_splitk": (lambda: synth.gemm_relu2_sum(40, 24, 1024), lambda: synth.inputs_gemm(40, 24, 1024),
                    ["EW", "EW", "MFMA", "MFMA", "FOLD"]),
    "gemm_y_splitk": (lambda: synth.gemm_bf16(40, 24, 512), lambda: synth.inputs_gemm_integer(40, 24, 512),
                      ["EW", "EW", "MFMA", "MFMA"]),
    # an epilogue reading operands of its own, one through a padding View
    "gemm_affine": (lambda: _gemm_affine(40, 24, 64), lambda: _gemm_affine_inputs(40, 24, 64), ["EW", "EW", "MFMA"]),
    "gemm_affine_splitk": (lambda: _gemm_affine(40, 24, 1024), lambda: _gemm_affine_inputs(40, 24, 1024),
                           ["EW", "EW", "MFMA", "MFMA"]),
    "gather": (lambda: synth.embedding_gather(50, 6, 30), lambda: synth.inputs_embedding(50, 6, 30), ["EW"]),
    "gather_general": (lambda: _gather_general(), lambda: _indexed_inputs(), ["EW", "EW"]),
    "scatter": (lambda: synth.embedding_scatter(20, 6, 100), lambda: synth.inputs_embedding(20, 6, 100),
                ["SCATTER"] * 3),
    "scatter_atomic": (lambda: synth.embedding_scatter(20, 6, 100, atomic=True),
                       lambda: synth.inputs_embedding(20, 6, 100), ["EW", "SCATTER"]),
    "scatter_general": (lambda: _scatter_general(), lambda: _indexed_inputs(), ["SCATTER"] * 3),
}


def _indexed_inputs():
    rng = np.random.default_rng(70)
    return {"D": rng.standard_normal((4, 9, 5)).astype(np.float32),
            "I": rng.integers(-3, 12, (4, 7, 5)).astype(np.int32),
            "V": rng.standard_normal((4, 7, 5)).astype(np.float32)}


def _gather_general():
    """GATHER along axis 1 of a permuted, padded View of the data, by a
    computed index (index + 1), then an elementwise consumer."""
    g = synth.Spec("gather_general")
    d = g.buffer("D", (4, 9, 5), "f32")
    dv = g.view(d, ("permute", (2, 1, 0)), ("pad", ((0, 0), (1, 1), (0, 0))), ("permute", (2, 1, 0)),
                ("shrink", ((0, 4), (0, 9), (0, 5))))
    i = g.buffer("I", (4, 7, 5), "i32")
    idx = g.add(i, g.const(1, (4, 7, 5), "i32"))
    g.output(g.mul(g.gather(dv, idx, 1), g.const(2.0, (4, 7, 5), "f32")))
    return g


def _scatter_general():
    """SCATTER along axis 1 with an index that varies along every dim (no
    carried dims), a computed base and computed values."""
    g = synth.Spec("scatter_general")
    d = g.buffer("D", (4, 9, 5), "f32")
    i = g.buffer("I", (4, 7, 5), "i32")
    v = g.buffer("V", (4, 7, 5), "f32")
    g.output(g.scatter(g.exp(d), i, g.mul(v, v), 1))
    return g


def _gemm_windows():
    g = synth.Spec("gemm_windows")
    a = g.buffer("A", (256, 96), "bf16")
    b = g.buffer("B", (64, 320), "bf16")
    aw = g.view(a, ("shrink", ((0, 256), (16, 80))))
    bw = g.view(b, ("shrink", ((0, 64), (8, 264))))
    a3 = g.cast(g.view(aw, ("reshape", (256, 1, 64)), ("expand", (256, 256, 64))), "f32")
    b3 = g.cast(g.view(bw, ("permute", (1, 0)), ("reshape", (1, 256, 64)), ("expand", (256, 256, 64))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    return g


def _gemm_windows_inputs():
    rng = np.random.default_rng(23)
    return {"A": synth.to_bf16_bits(rng.integers(-2, 3, (256, 96)).astype(np.float32)),
            "B": synth.to_bf16_bits(rng.integers(-2, 3, (64, 320)).astype(np.float32))}


@pytest.mark.parametrize("name", list(CLASSES))
def test_plan_interpreter_matches_oracle(name):
    mk_spec, mk_in, classes = CLASSES[name]
    spec, inp = mk_spec(), mk_in()
    d, got = _interp(spec, inp)
    assert [k["class"] for k in d["kernels"]] == classes
    ref = oracle.run(spec, inp)
    for g, r in zip(got, ref):
        assert g.shape == r.shape
        if name in ("gemm", "gemm_copied", "gemm_splitk"):
            # the plan folds the epilogue in one order, the oracle widens: close
            assert abs(float(g.ravel()[0]) - float(r.ravel()[0])) <= 1e-4 * abs(float(r.ravel()[0]))
        else:
            # the plan folds every reduce in ascending order, as the oracle does
            assert g.tobytes() == r.tobytes(), name


def test_cuts_and_workspace():
    # a permute of a computed value is a cut: the value goes to workspace
    g = synth.Spec()
    a = g.buffer("a", (8, 12), "f32")
    b = g.buffer("b", (8, 12), "f32")
    s = g.add(a, b)
    g.output(g.mul(g.view(s, ("permute", (1, 0))), g.view(s, ("permute", (1, 0)))))
    inp = {"a": np.arange(96, dtype=np.float32).reshape(8, 12), "b": np.ones((8, 12), np.float32)}
    d, got = _interp(g, inp)
    assert [k["class"] for k in d["kernels"]] == ["EW", "EW"]
    assert d["workspace_bytes"] >= 96 * 4
    assert got[0].tobytes() == oracle.run(g, inp)[0].tobytes()
    # reduces over different axes cannot share a row space: each is cut
    g = synth.Spec()
    x = g.buffer("x", (6, 7, 5), "f32")
    s1 = g.sum(x, (2,))
    s2 = g.max(s1, (0,))
    g.output(s2)
    xi = np.random.default_rng(1).standard_normal((6, 7, 5)).astype(np.float32)
    d, got = _interp(g, {"x": xi})
    assert [k["class"] for k in d["kernels"]] == ["REDUCE", "REDUCE"]
    assert got[0].tobytes() == oracle.run(g, {"x": xi})[0].tobytes()
    # an input returned as an output is a copy; several outputs
    g = synth.Spec()
    x = g.buffer("x", (5, 3), "f32")
    m = g.max(x, (1,))
    g.output(x, m, m)
    xi = np.random.default_rng(2).standard_normal((5, 3)).astype(np.float32)
    d, got = _interp(g, {"x": xi})
    ref = oracle.run(g, {"x": xi})
    for a, b in zip(got, ref):
        assert a.tobytes() == b.tobytes()


def test_empty_and_size_one_dims():
    g = synth.Spec()
    x = g.buffer("x", (0, 5), "f32")
    g.output(g.exp(x))
    d, got = _interp(g, {"x": np.zeros((0, 5), np.float32)})
    assert d["kernels"][0]["plan"] == "empty" and got[0].shape == (0, 5)
    g = synth.Spec()
    x = g.buffer("x", (1, 7, 1, 3), "f32")
    g.output(g.sum(x, (1, 3)))
    xi = np.random.default_rng(3).standard_normal((1, 7, 1, 3)).astype(np.float32)
    d, got = _interp(g, {"x": xi})
    assert got[0].tobytes() == oracle.run(g, {"x": xi})[0].tobytes()


@pytest.mark.parametrize("shape,axes", [((3, 0), (1,)), ((0, 4), (0,)), ((2, 3, 0), (1, 2)), ((2, 0, 3), (1,))])
def test_reduce_over_empty_range_writes_identity(shape, axes):
    # the kernel still runs for its output cells, which get 0 (SUM) / -inf (MAX)
    g = synth.Spec()
    x = g.buffer("x", shape, "f32")
    g.output(g.sum(x, axes), g.max(x, axes))
    inp = {"x": np.zeros(shape, np.float32)}
    d, got = _interp(g, inp)
    assert all(k["plan"] != "empty" for k in d["kernels"])
    ref = oracle.run(g, inp)
    assert np.all(ref[0] == 0) and np.all(ref[1] == -np.inf)
    for a, b in zip(got, ref):
        assert a.shape == b.shape and a.tobytes() == b.tobytes()


def test_dims_merge_for_contiguous_chains():
    prog = rv.compile_spec(synth.rmsnorm(64, 512))
    k = prog.describe()["kernels"][0]
    assert k["domain"] == [64, 512] and k["reduce_dims"] == [1]
    g = synth.Spec()
    a = g.buffer("a", (8, 16, 32), "f32")
    g.output(g.exp(a))
    k = rv.compile_spec(g).describe()["kernels"][0]
    assert k["domain"] == [8 * 16 * 32] and k["plan"] == "rowmajor"


def test_dtype_variants_through_the_plan():
    rng = np.random.default_rng(4)
    for dt, mk in (("i8", lambda s: rng.integers(-128, 128, s).astype(np.int8)),
                   ("i32", lambda s: rng.integers(-2 ** 31, 2 ** 31, s, dtype=np.int64).astype(np.int32)),
                   ("f64", lambda s: rng.standard_normal(s)),
                   ("f16", lambda s: rng.standard_normal(s).astype(np.float16))):
        g = synth.Spec()
        a = g.buffer("a", (9, 11), dt)
        b = g.buffer("b", (9, 11), dt)
        s = g.add(g.mul(a, b), g.neg(b))
        g.output(s, g.sum(s, (1,)), g.max(s, (0,)))
        inp = {"a": mk((9, 11)), "b": mk((9, 11))}
        d, got = _interp(g, inp)
        ref = oracle.run(g, inp)
        for x, y in zip(got, ref):
            assert x.tobytes() == y.tobytes(), dt


def test_attention_is_one_custom_kernel():
    # the two CUSTOM sdpa_fwd nodes (output and logsumexp) share one launch
    prog = rv.compile_spec(synth.attention(3, 200, 333, 64, causal=False, out_dtype="bf16"))
    ks = prog.describe()["kernels"]
    assert [k["class"] for k in ks] == ["ATTN"]
    k = ks[0]
    assert k["grid"] == [2, 3, 1] and k["block"] == [256, 1, 1]
    assert k["plan_detail"]["head_dim"] == 64 and k["plan_detail"]["keys"] == 333
    # 64-key K and V tiles, 3 stages at head width 64 (48 KB), no VGPR staging
    assert k["plan_detail"]["stages"] == 3 and k["lds_bytes"] == 3 * 2 * 64 * 64 * 2
    assert sorted(s["loc"]["index"] for s in k["stores"]) == [0, 1]
    assert prog.out_desc == [((3, 200, 64), "bf16"), ((3, 200, 1), "f32")]


def test_attention_key_chunk_choice():
    """Keys split over workgroups only when one workgroup per 128-query block
    leaves the chip's slots empty (256 CUs x 4, 3, 2 workgroups at head width
    32, 64, 128), in the smallest of 1024 / 2048 / 4096-key chunks that keeps
    the workgroups within twice the slots; a row no longer than one chunk is
    never split."""
    cases = [((6, 8192, 32, True), 1024, 288), ((6, 8192, 32, False), 2048, 256), ((6, 8192, 128, True), 2048, 160),
             ((6, 8192, 128, False), 4096, 128), ((16, 2048, 128, True), 1024, 24), ((96, 4096, 32, False), 0, 32),
             ((2, 300, 64, True), 0, 3)]
    for (h, t, d, causal), ck, grid in cases:
        ks = rv.compile_spec(synth.attention(h, t, t, d, causal)).describe()["kernels"]
        assert ks[0]["plan_detail"]["key_chunk"] == ck and ks[0]["grid"][:2] == [grid, h], (h, t, d, causal, ks[0])
        assert [k["plan"] for k in ks] == (["attn_fwd", "attn_merge"] if ck else ["attn_fwd"])


def test_contraction_split_choice(monkeypatch):
    """A contraction splits over k only while its tiles leave CUs idle: the
    slice count is the power of two with the smallest estimated time, every
    slice at least 256 deep, at most 256 workgroups, planes within 32 MiB;
    RV_GEMM_SPLITK forces a count that fits (1, or one that does not fit,
    leaves the contraction whole)."""
    def plan(m, n, k):
        ks = rv.compile_spec(synth.gemm_bf16(m, n, k)).describe()["kernels"]
        mf = [kk for kk in ks if kk["class"] == "MFMA"]
        return mf[0]["plan_detail"]["split_k"], [kk["plan"] for kk in mf], mf[0]["grid"][0], ks
    cases = [((4096, 4096, 4096), 1), ((4096, 4096, 1024), 1), ((1024, 1024, 8192), 8), ((512, 512, 16384), 32),
             ((1024, 1024, 2048), 4), ((768, 768, 4096), 8), ((2048, 2048, 4096), 2), ((256, 256, 256), 1),
             ((256, 256, 512), 2)]
    for (m, n, k), want in cases:
        S, plans, grid, ks = plan(m, n, k)
        tiles = -(-m // 256) * -(-n // 256)
        assert S == want and grid == tiles * S, ((m, n, k), S, grid)
        assert plans == (["gemm_w6", "gemm_slices"] if S > 1 else ["gemm_w6"])
        if S > 1:
            pd = ks[-1]["plan_detail"]
            assert pd["split_k"] == S and pd["plane"] % 64 == 0 and pd["plane"] >= m * n
            assert pd["plane"] * S * 4 <= 32 << 20
    monkeypatch.setenv("RV_GEMM_SPLITK", "16")
    assert plan(1024, 1024, 8192)[0] == 16  # forced past the plane limit
    monkeypatch.setenv("RV_GEMM_SPLITK", "64")
    assert plan(1024, 1024, 8192)[0] == 1   # 16 tiles x 64 > 256 workgroups
    monkeypatch.setenv("RV_GEMM_SPLITK", "3")
    assert plan(1024, 1024, 8192)[0] == 1   # not a power of two
    monkeypatch.setenv("RV_GEMM_SPLITK", "1")
    assert plan(512, 512, 16384)[:2] == (1, ["gemm_w6"])


def test_attention_operand_view_is_materialised():
    # k given as a permuted View of a (H, D, Tk) buffer: copied to workspace first
    g = synth.Spec()
    q = g.buffer("Q", (2, 40, 32), "bf16")
    kt = g.buffer("Kt", (2, 32, 50), "bf16")
    v = g.buffer("V", (2, 50, 32), "bf16")
    o, _ = g.sdpa(q, g.view(kt, ("permute", (0, 2, 1))), v, 0.25, causal=False)
    g.output(o)
    ks = rv.compile_spec(g).describe()
    assert [k["class"] for k in ks["kernels"]] == ["EW", "ATTN"]
    assert ks["workspace_bytes"] >= 2 * 50 * 32 * 2


def test_attention_contract_errors():
    def status(spec, patch=None):
        nodes, _ = rv.nodes_from_spec(spec)
        if patch:
            patch(nodes)
        with pytest.raises(rv.RVError) as e:
            rv.rv_compile(nodes, list(spec.outputs))
        return e.value.name

    g = synth.Spec()
    q = g.buffer("Q", (1, 8, 32), "f32")
    k = g.buffer("K", (1, 8, 32), "f32")
    o, _ = g.sdpa(q, k, k, 0.1)
    g.output(o)
    assert status(g) == "RV_E_DTYPE"
    g = synth.Spec()
    q = g.buffer("Q", (1, 8, 48), "bf16")
    o, _ = g.sdpa(q, q, q, 0.1)
    g.output(o)
    assert status(g) == "RV_E_UNSUPPORTED_LAYOUT"
    g = synth.attention(1, 8, 8, 32, outputs="o")
    assert status(g, lambda n: setattr(n[3], "buf", 7)) == "RV_E_UNSUPPORTED_OP"
    g = synth.attention(1, 8, 8, 32, outputs="o")
    assert status(g, lambda n: setattr(n[3], "reduce_axes", 5 << 16)) == "RV_E_INVALID"


def test_contraction_plans():
    """Every bf16 contraction takes the four-wave 256 x 256 kernel with A
    staged 64 deep (3 stages) and B 32 deep (4 stages): 160 KB of LDS.
    float16 rows give each ROW lane 32 cells, float32 rows 16."""
    big = rv.compile_spec(synth.gemm_relu2_sum(4096, 4096, 4096)).describe()["kernels"][0]
    assert big["plan"] == "gemm_w6" and big["block"][0] == 256 and big["grid"][0] == 256
    pd = big["plan_detail"]
    assert pd["tile"] == [256, 256, 32] and pd["wave_tiles"] == [4, 4]
    assert pd["stages"] == {"A": 3, "B": 4} and pd["stage_depth"] == {"A": 64, "B": 32}
    assert pd["early_copies"] == [3, 1] and big["lds_bytes"] == 3 * 256 * 64 * 2 + 4 * 256 * 32 * 2 == 160 * 1024
    assert pd["ragged"] is False and pd["copied"] == {"A": False, "B": False}
    small = rv.compile_spec(synth.gemm_bf16(256, 384, 192)).describe()["kernels"][0]
    assert small["plan"] == "gemm_w6" and small["grid"][0] == 2 and small["plan_detail"]["ragged"] is True
    # K = 96 is no multiple of 64: the 64-deep kernel reads zero-padded copies
    odd = rv.compile_spec(synth.gemm_bf16(256, 256, 96)).describe()
    assert odd["kernels"][-1]["plan"] == "gemm_w6" and odd["kernels"][-1]["plan_detail"]["extent"][2] == 128
    f16 = rv.compile_spec(synth.rmsnorm(64, 4096, dtype="f16")).describe()["kernels"][0]
    f32 = rv.compile_spec(synth.rmsnorm(64, 4096)).describe()["kernels"][0]
    assert f16["plan_detail"]["threads_per_row"] == 128 and f32["plan_detail"]["threads_per_row"] == 256


def _random_view(rng, shape):
    """A View over row-major `shape` from 1-4 random movements (the
    library's own View algebra), as raw (shape, strides, offset, mask)."""
    v = rv.rv_view_contiguous(shape)
    for _ in range(int(rng.integers(1, 5))):
        cur = [v.shape[d] for d in range(v.ndim)]
        kind = rng.choice(["permute", "shrink", "pad", "expand", "reshape"])
        try:
            if kind == "permute":
                v = rv.rv_view_permute(v, list(rng.permutation(len(cur))))
            elif kind == "shrink":
                lo = [int(rng.integers(0, max(1, c // 2))) for c in cur]
                hi = [int(rng.integers(l + 1, c + 1)) if c > l else c for l, c in zip(lo, cur)]
                v = rv.rv_view_shrink(v, lo, hi)
            elif kind == "pad":
                v = rv.rv_view_pad(v, [int(rng.integers(0, 3)) for _ in cur], [int(rng.integers(0, 3)) for _ in cur])
            elif kind == "expand":
                ones = [d for d, c in enumerate(cur) if c == 1]
                if ones:
                    new = list(cur)
                    new[ones[0]] = int(rng.integers(2, 4))
                    v = rv.rv_view_expand(v, new)
            else:
                n = int(np.prod(cur))
                for cand in ([n], [1] + cur, cur + [1], [cur[0] * cur[1]] + cur[2:] if len(cur) > 1 else cur):
                    try:
                        v = rv.rv_view_reshape(v, cand)
                        break
                    except rv.RVError:
                        continue
        except rv.RVError:
            pass
    d = v.to_dict()
    return d


@pytest.mark.parametrize("seed", range(40))
def test_view_of_view_composes_exactly(seed):
    """Random raw Views of random raw Views over one buffer (movement only):
    the scheduler composes each pair into one View of the buffer where a
    single View expresses it, else materialises the inner value; either way
    the planned kernels reproduce the oracle bit for bit."""
    rng = np.random.default_rng(seed)
    shape = [int(x) for x in rng.integers(1, 7, int(rng.integers(1, 4)))]
    inner = _random_view(rng, shape)
    outer = _random_view(rng, list(inner["shape"]))
    g = synth.Spec(f"view_of_view_{seed}")
    x = g.buffer("X", tuple(shape), "f32")
    a = g.raw_view(x, inner["shape"], inner["strides"], inner["offset"], inner["mask_lo"], inner["mask_hi"])
    b = g.raw_view(a, outer["shape"], outer["strides"], outer["offset"], outer["mask_lo"], outer["mask_hi"])
    g.output(g.contiguous(b))
    inp = {"X": rng.standard_normal(shape).astype(np.float32) + 3.0}
    d, got = _interp(g, inp)
    ref = oracle.run(g, inp)
    assert got[0].tobytes() == ref[0].tobytes()
    assert len(d["kernels"]) in (1, 2)


def test_view_of_view_window_is_one_kernel():
    """A column window of a permuted buffer, then a broadcast of it: one View
    of the buffer, one kernel."""
    g = synth.Spec("window")
    x = g.buffer("X", (6, 10), "f32")
    a = g.raw_view(x, (10, 6), (1, 10), 0)                   # permute
    b = g.raw_view(a, (4, 2, 6), (6, 0, 1), 12, None, None)  # rows 2..5, a broadcast dim
    g.output(g.contiguous(b))
    inp = {"X": np.arange(60, dtype=np.float32).reshape(6, 10)}
    d, got = _interp(g, inp)
    assert len(d["kernels"]) == 1
    assert got[0].tobytes() == oracle.run(g, inp)[0].tobytes()


def _random_values(rng, shape, dt):
    """Small integers in the storage of dtype ``dt`` (bfloat16 as bits)."""
    v = rng.integers(-3, 4, shape)
    if dt == "bf16":
        return synth.to_bf16_bits(v.astype(np.float32))
    return v.astype({"f32": np.float32, "f16": np.float16, "f64": np.float64, "i32": np.int32}[dt])


def random_region(seed, dt="f32"):
    """A random small region: two or three buffers read directly,
    transposed, as a broadcast row, or through a shrunk (and partly padded)
    window of a larger buffer; a random mix of ADD / MUL / NEG / CMPLT /
    WHERE; then nothing, a SUM or MAX over one axis, or a row reduce expanded
    back and combined with the region. Integer-valued float32 inputs make
    every order of additions give the same bits. Returns (spec, inputs)."""
    rng = np.random.default_rng(1000 + seed)
    rank = 2 if rng.random() < 0.6 else 3
    shape = tuple(int(x) for x in rng.integers(8, 21, rank))
    g = synth.Spec(f"random_{dt}_{seed}")
    inputs, vals = {}, []
    for b in range(int(rng.integers(2, 4))):
        name = f"B{b}"
        mode = ["direct", "transposed", "row", "window"][int(rng.integers(0, 4))]
        if mode == "direct":
            bshape = shape
            v = g.buffer(name, bshape, dt)
        elif mode == "transposed":
            bshape = shape[::-1]
            v = g.view(g.buffer(name, bshape, dt), ("permute", tuple(range(rank))[::-1]))
        elif mode == "row":
            bshape = (shape[-1],)
            v = g.view(g.buffer(name, bshape, dt), ("reshape", (1,) * (rank - 1) + (shape[-1],)), ("expand", shape))
        else:
            bshape = tuple(d + 3 for d in shape)
            lo = tuple(int(rng.integers(0, 4)) for _ in shape)
            v = g.view(g.buffer(name, bshape, dt), ("shrink", tuple((l, l + d) for l, d in zip(lo, shape))))
            if rng.random() < 0.5:  # and pad one side back with zeros
                pad = tuple((1, 0) if dd == 0 else (0, 0) for dd in range(rank))
                v = g.view(v, ("pad", pad), ("shrink", tuple((0, d) for d in shape)))
        inputs[name] = _random_values(rng, bshape, dt)
        vals.append(v)
    x = vals[0]
    for v in vals[1:]:
        op = rng.choice(["add", "mul", "where"])
        if op == "add":
            x = g.add(x, v)
        elif op == "mul":
            x = g.mul(x, v)
        else:
            x = g.where(g.cmplt(x, v), x, g.neg(v))
    tail = rng.choice(["none", "reduce", "row"])
    if tail == "reduce":
        ax = int(rng.integers(0, rank))
        x = g.sum(x, (ax,)) if rng.random() < 0.5 else g.max(x, (ax,))
    elif tail == "row":
        r = g.max(x, (rank - 1,)) if rng.random() < 0.5 else g.sum(x, (rank - 1,))
        x = g.add(x, g.neg(g.view(r, ("expand", shape))))
        if rng.random() < 0.5:
            x = g.sum(g.mul(x, x), (rank - 1,))
    g.output(x)
    return g, inputs


@pytest.mark.parametrize("seed", range(40))
def test_random_graphs_plan_matches_oracle(seed):
    """Random regions (random_region) planned and run through the CPU plan
    interpreter reproduce the oracle exactly."""
    g, inputs = random_region(seed)
    d, got = _interp(g, inputs)
    ref = oracle.run(g, inputs)
    assert got[0].tobytes() == ref[0].tobytes()


@pytest.mark.parametrize("spec,classes", [
    (synth.reduce((1 << 24,), (0,)), ["SPLIT", "FOLD"]),
    (synth.reduce((16384, 4096), (0,)), ["SPLIT", "FOLD"]),
    (synth.reduce((6, 520, 700), (0, 2)), ["SPLIT", "FOLD"]),
    (synth.mean_rows(8, 500000), ["SPLIT", "FOLD"]),
    (synth.softmax(4, 300000), ["SPLIT", "FOLD", "SPLIT", "FOLD", "EW"]),
    (synth.softmax(16384, 4096), ["ROW"]),               # many rows: one ROW kernel
    (synth.softmax(256, 262144), ["ROW"]),               # a row per CU: the streaming ROW plan
    (synth.reduce((64, 64, 64), (2,)), ["REDUCE"]),      # little work: one launch
    (synth.reduce((1000, 100), (0,)), ["REDUCE"]),
])
def test_split_reduce_classes(spec, classes):
    """A long reduce over few output cells splits into partials and a fold
    (limn README, "Backends"); reduces with enough cells, or too little
    work to pay for a second launch, keep one kernel."""
    d = rv.compile_spec(spec).describe()
    assert [k["class"] for k in d["kernels"]] == classes
    for a, b in zip(d["kernels"], d["kernels"][1:]):
        if a["class"] == "SPLIT":
            assert b["class"] == "FOLD" and b["plan"] == "fold_cells"
            pa, pb = a["plan_detail"], b["plan_detail"]
            assert pb["partials"] == pa["pieces"] and pb["sum_depth"] > pa["sum_depth"]
            assert a["grid"][0] * a["grid"][1] >= 256  # the chip is filled


def test_split_off_switch(monkeypatch):
    monkeypatch.setenv("RV_SPLIT", "0")
    d = rv.compile_spec(synth.reduce((1 << 24,), (0,))).describe()
    assert [k["plan"] for k in d["kernels"]] == ["row_stream"]


def _gemm_affine(m, n, k):
    """z = CAST_bf16(y * s[n] + c'[m]) on the contraction y: a column scale and
    a row bias read by the epilogue, the bias through a padding View (rows
    before 3 and from m - 7 on read zero)."""
    g = synth.Spec(f"gemm_affine_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), "bf16")
    b = g.buffer("B", (k, n), "bf16")
    sc = g.buffer("S", (n,), "f32")
    c = g.buffer("C", (m - 10,), "f32")
    a3 = g.cast(g.view(a, ("reshape", (m, 1, k)), ("expand", (m, n, k))), "f32")
    b3 = g.cast(g.view(b, ("permute", (1, 0)), ("reshape", (1, n, k)), ("expand", (m, n, k))), "f32")
    y = g.sum(g.mul(a3, b3), (2,))
    sv = g.view(sc, ("reshape", (1, n, 1)), ("expand", (m, n, 1)))
    cv = g.view(c, ("pad", ((3, 7),)), ("reshape", (m, 1, 1)), ("expand", (m, n, 1)))
    g.output(g.cast(g.add(g.mul(y, sv), cv), "bf16"))
    return g


def _gemm_affine_inputs(m, n, k):
    rng = np.random.default_rng(41)
    inp = dict(synth.inputs_gemm_integer(m, n, k))
    inp["S"] = rng.integers(-3, 4, n).astype(np.float32)
    inp["C"] = rng.integers(-50, 51, m - 10).astype(np.float32)
    return inp


def _gemm_views(m, n, k, a_mv=(), b_mv=(), bt=False):
    """y = SUM_k CAST(A) * CAST(B) with A (m, k) and B (k, n) reached through
    extra movements of their buffers (B stored [n][k] when ``bt``)."""
    g = synth.Spec(f"gemm_views_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), "bf16")
    a2 = g.view(a, *a_mv) if a_mv else a
    b = g.buffer("B", (n, k) if bt else (k, n), "bf16")
    b2 = g.view(b, *b_mv) if b_mv else b
    bkn = g.view(b2, ("permute", (1, 0))) if bt else b2
    a3 = g.cast(g.view(a2, ("reshape", (m, 1, k)), ("expand", (m, n, k))), "f32")
    b3 = g.cast(g.view(bkn, ("permute", (1, 0)), ("reshape", (1, n, k)), ("expand", (m, n, k))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    return g


RAGGED_GEMMS = [
    ((4095, 4096, 4096), {}, False, False),      # one row short: the last tile shifts, no copy
    ((257, 129, 65), {}, True, True),            # every extent ragged: both operands copied
    ((255, 257, 31), {}, True, True),
    ((300, 257, 64), {}, False, True),           # N not a multiple of 8: B copied
    ((520, 300, 128), {"bt": True}, False, False),  # B stored [n][k], ragged N in place
    ((520, 300, 96), {"bt": True}, True, True),   # K no multiple of the 64-deep step: both padded
    ((1, 1, 1), {}, True, True),
    ((256, 256, 64), {}, False, False),
    ((256, 256, 32), {}, True, True),
]


@pytest.mark.parametrize("mnk,kw,ca,cb", RAGGED_GEMMS)
def test_every_bf16_contraction_runs_on_mfma(mnk, kw, ca, cb):
    """No bf16 CAST * MUL * SUM contraction leaves the matrix cores: ragged
    extents shift the last tile or copy an operand, zero-padded, into
    workspace first (limn README, "Correctness": matmuls across every tile
    width and tail)."""
    m, n, k = mnk
    d = rv.compile_spec(_gemm_views(m, n, k, **kw)).describe()
    cls = [kk["class"] for kk in d["kernels"]]
    assert cls.count("MFMA") == 1 and set(cls) <= {"MFMA", "EW"}, cls
    mf = [kk for kk in d["kernels"] if kk["class"] == "MFMA"][0]["plan_detail"]
    assert mf["copied"] == {"A": ca, "B": cb}
    assert cls.count("EW") == ca + cb


def test_transposed_and_padded_operands_run_on_mfma():
    # A read transposed (stored [k][m]) and B through a pad: both copied
    g = synth.Spec("gemm_t")
    a = g.buffer("A", (96, 300), "bf16")
    b = g.buffer("B", (90, 260), "bf16")
    a2 = g.view(a, ("permute", (1, 0)))
    b2 = g.view(b, ("pad", ((3, 3), (0, 0))))
    a3 = g.cast(g.view(a2, ("reshape", (300, 1, 96)), ("expand", (300, 260, 96))), "f32")
    b3 = g.cast(g.view(b2, ("permute", (1, 0)), ("reshape", (1, 260, 96)), ("expand", (300, 260, 96))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    d = rv.compile_spec(g).describe()
    assert [kk["class"] for kk in d["kernels"]] == ["EW", "EW", "MFMA"]


@pytest.mark.parametrize("spec", [
    synth.ew_chain(4096, 4096), synth.ew_chain(4096, 4096, masked=True), synth.transpose(4096, 4096),
    synth.softmax(16384, 4096), synth.rmsnorm(16384, 4096), synth.layernorm(8192, 8192),
    synth.matmul_broadcast(64, 64, 64), synth.gemm_relu2_sum(4096, 4096, 4096), synth.gemm_relu2_sum(257, 129, 65),
    synth.softmax(256, 262144), synth.attention(6, 8192, 8192, 32, True), synth.reduce((1 << 24,), (0,)),
    synth.reduce((16384, 4096), (0,)), synth.embedding_gather(65536, 1024, 32768),
    synth.embedding_scatter(65536, 1024, 32768), synth.rmsnorm(16384, 4096, dtype="f64"),
], ids=lambda s: s.name)
def test_kernel_budgets_visible_and_spill_free(spec):
    """rv_describe reports each compiled kernel's registers, scratch and LDS
    (Tiki README, "The architecture we want": budgets visible before
    launch); the kernels of every workload keep everything in registers and
    LDS: no scratch, no vector spills, LDS within the CU's 160 KB. Only the
    contraction spills scalar registers, and those land in lanes of a vector
    register (no memory traffic; read back after its k-loop)."""
    d = rv.compile_spec(spec).describe()
    for k in d["kernels"]:
        r = k["resources"]
        assert r["scratch_bytes"] == 0 and r["vgpr_spill"] == 0, (k["name"], r)
        assert r["sgpr_spill"] == 0 or k["class"] == "MFMA", (k["name"], r)
        assert 0 < r["vgpr"] <= 512 and r["lds_bytes"] <= 160 * 1024, (k["name"], r)
        if k["class"] == "MFMA":
            assert r["agpr"] == 256  # the 256 accumulators per lane stay in the accumulation registers
