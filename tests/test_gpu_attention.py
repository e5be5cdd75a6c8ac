"""GPU parity of the fused attention forward (CUSTOM sdpa_fwd) against the
oracle's primitive composition: scores folded in order over the head dim,
max-shifted softmax, contraction over keys, L = max + log(sum).

Bound, per output cell (i, d), from the steps where the kernel rounds
differently from the composition (all relative to sum_j P_ij |v_jd|, the
magnitude the contraction adds up):
  * each probability enters the second contraction rounded to bfloat16
    (the matrix cores' operand type): 2^-8;
  * the denominator and the contraction fold in another order: 4 gamma_Tk;
  * a score differs by at most 2 gamma_D scale sum_d |q k| (both sides fold
    the head dim in some order) plus the base-2 conversion (scale * log2 e
    rounded, one multiply) 4 u (1 + |s| log2 e), moving exp(s) relatively by
    as much;
  * each rescale of the running sums by exp2(m_old - m_new) and each
    exponential: (5 R + 4) u with R the key tiles.
L: the denominator's relative error (4 gamma_Tk + (5 R + 4) u) plus the
score error and 4 u |m| for the base conversion, plus 2 ulp of L.
A bfloat16 output adds one bfloat16 ulp of the result."""

import numpy as np
import pytest

import oracle
from oracle import interp
from reduce_view_amd import synth
from tests.harness import U, gamma, report, run, ulp_bf16

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


def _f64_parts(q, k, v, scale, causal):
    """float64 P, sum_j P |v| and max_j sum_d |q k| per query (bound terms)."""
    qd, kd, vd = (interp.bf16_to_f32(a).astype(np.float64) for a in (q, k, v))
    s = np.einsum("hid,hjd->hij", qd, kd) * scale
    aqk = np.einsum("hid,hjd->hij", np.abs(qd), np.abs(kd))
    if causal:
        hide = np.arange(s.shape[2])[None, None, :] > np.arange(s.shape[1])[None, :, None]
        s = np.where(hide, -np.inf, s)
        aqk = np.where(hide, 0, aqk)
    m = s.max(axis=2, keepdims=True)
    e = np.exp(s - m)
    P = e / e.sum(axis=2, keepdims=True)
    return P @ np.abs(vd), aqk.max(axis=2, keepdims=True), np.abs(s).max(axis=2, where=np.isfinite(s),
                                                                       initial=0.0, keepdims=True), m


def _check(name, spec, inp, h, tq, tk, d, causal, out_dtype="f32", outputs="ol"):
    prog = _prog(spec)
    kd = prog.describe()["kernels"]
    assert {k["class"] for k in kd} == {"ATTN"}, kd
    got = run(prog, inp)
    ref = oracle.run(spec, inp)
    scale = 1.0 / np.sqrt(d)
    pv, aqk, smax, m = _f64_parts(inp["Q"], inp["K"], inp["V"], scale, causal)
    R = -(-tk // 32) + 1
    score = 2 * gamma(d) * scale * aqk + 4 * U * (1 + smax * np.log2(np.e))
    rel = 2.0 ** -8 + 4 * gamma(tk) + score + (5 * R + 4) * U
    i = 0
    if "o" in outputs:
        g, r = got[i], ref[i]
        if out_dtype == "bf16":
            g, r = interp.bf16_to_f32(g).astype(np.float64), interp.bf16_to_f32(r).astype(np.float64)
            extra = ulp_bf16(np.maximum(np.abs(g), np.abs(r)))
        else:
            g, r = g.astype(np.float64), r.astype(np.float64)
            extra = 0.0
        bound = rel * pv + extra + 2.0 ** -126
        err = np.abs(g - r)
        report(f"{name}_O", err, bound)
        assert np.all(err <= bound)
        i += 1
    if "l" in outputs:
        g, r = got[i].astype(np.float64), ref[i].astype(np.float64)
        bound = 4 * gamma(tk) + (5 * R + 4) * U + score + 4 * U * np.abs(m) + 4 * U * np.abs(r) + 2.0 ** -126
        err = np.abs(g - r)
        report(f"{name}_L", err, bound)
        assert np.all(err <= bound)


@pytest.mark.parametrize("h,tq,tk,d,causal,odt", [
    (2, 128, 128, 32, True, "f32"),
    (2, 200, 333, 64, False, "bf16"),
    (1, 130, 130, 128, True, "f32"),
    (3, 64, 1000, 32, False, "f32"),
    (2, 300, 300, 64, True, "bf16"),
    (1, 1, 1, 32, False, "f32"),
    (1, 5, 37, 128, False, "f32"),
    # causal with more queries than keys: rows past the last key see all keys
    (2, 300, 200, 32, True, "f32"),
    (1, 70, 5, 64, True, "bf16"),
])
def test_attention_matches_composition(h, tq, tk, d, causal, odt):
    _case(f"attention {h}x{tq}x{tk}x{d} causal={causal} out={odt}")
    spec = synth.attention(h, tq, tk, d, causal, odt)
    inp = synth.inputs_attention(h, tq, tk, d)
    _check(f"attention_{h}x{tq}x{tk}x{d}", spec, inp, h, tq, tk, d, causal, odt)


@pytest.mark.parametrize("chunk", [128, 256])
@pytest.mark.parametrize("h,tq,tk,d,causal,odt", [
    (2, 300, 300, 64, True, "bf16"),
    (3, 64, 1000, 32, False, "f32"),
    (1, 513, 700, 128, True, "f32"),
    (2, 1024, 1024, 32, True, "f32"),
])
def test_attention_key_chunks_merge(monkeypatch, chunk, h, tq, tk, d, causal, odt):
    """Keys split over workgroups in chunks of 128 or 256 (the long-row
    split, forced onto small shapes): partials (m, l, accumulator) per chunk,
    folded in chunk order by the merge kernel."""
    monkeypatch.setenv("RV_ATTN_CHUNK", str(chunk))
    _case(f"attention chunks of {chunk}: {h}x{tq}x{tk}x{d} causal={causal} out={odt}")
    spec = synth.attention(h, tq, tk, d, causal, odt)
    plans = [k["plan"] for k in _prog(spec).describe()["kernels"]]
    assert plans == ["attn_fwd", "attn_merge"], plans
    inp = synth.inputs_attention(h, tq, tk, d)
    _check(f"attention_chunk{chunk}_{h}x{tq}x{tk}x{d}", spec, inp, h, tq, tk, d, causal, odt)


@pytest.mark.parametrize("outputs", ["o", "l"])
def test_attention_single_output(outputs):
    _case(f"attention one output {outputs}")
    spec = synth.attention(2, 96, 96, 64, True, outputs=outputs)
    inp = synth.inputs_attention(2, 96, 96, 64)
    _check(f"attention_only_{outputs}", spec, inp, 2, 96, 96, 64, True, outputs=outputs)


def test_attention_causal_first_row_is_first_value():
    """Query 0 sees key 0 only: O[:, 0] is V[:, 0] (probability exactly 1,
    rounded to bfloat16 exactly) and L[:, 0] is that one scaled score."""
    _case("attention causal first row")
    h, t, d = 2, 64, 32
    inp = synth.inputs_attention(h, t, t, d)
    o, lse = run(_prog(synth.attention(h, t, t, d, True)), inp)
    assert o[:, 0].tobytes() == interp.bf16_to_f32(inp["V"][:, 0]).tobytes()


def test_attention_full_size_sampled_rows():
    """6 heads x 8192 tokens x 32, causal (the benchmark's workload): sampled
    query rows against the oracle evaluated for that row alone (a causal row
    i is the non-causal attention of q_i over the first i + 1 keys)."""
    _case("attention full 6x8192x8192x32 causal, sampled rows")
    h, t, d = 6, 8192, 32
    inp = synth.inputs_attention(h, t, t, d)
    o, lse = run(_prog(synth.attention(h, t, t, d, True)), inp)
    rng = np.random.default_rng(31)
    rows = sorted(set([0, 1, 31, 32, 127, 128, 4095, 8191] + list(rng.integers(0, t, 24))))
    worst = 0.0
    for hh in (0, h - 1):
        for i in rows:
            sub = {"Q": inp["Q"][hh:hh + 1, i:i + 1], "K": inp["K"][hh:hh + 1, :i + 1], "V": inp["V"][hh:hh + 1, :i + 1]}
            spec = synth.attention(1, 1, i + 1, d, False)
            ro, rl = oracle.run(spec, sub)
            pv, aqk, smax, m = _f64_parts(sub["Q"], sub["K"], sub["V"], 1.0 / np.sqrt(d), False)
            R = -(-(i + 1) // 32) + 1
            score = 2 * gamma(d) * aqk / np.sqrt(d) + 4 * U * (1 + smax * np.log2(np.e))
            rel = 2.0 ** -8 + 4 * gamma(i + 1) + score + (5 * R + 4) * U
            err = np.abs(o[hh, i].astype(np.float64) - ro[0, 0].astype(np.float64))
            bound = rel[0, 0] * pv[0, 0] + 2.0 ** -126
            worst = max(worst, float((err / bound).max()))
            assert np.all(err <= bound), (hh, i)
            lb = 4 * gamma(i + 1) + (5 * R + 4) * U + score[0, 0, 0] + 4 * U * abs(m[0, 0, 0]) + \
                4 * U * abs(float(rl[0, 0, 0])) + 2.0 ** -126
            assert abs(float(lse[hh, i, 0]) - float(rl[0, 0, 0])) <= lb, (hh, i)
    print(f"BOUND attention full sampled rows max err/bound {worst:.4f}", flush=True)
