"""The library's View algebra (rv_view_* through the C ABI) on the CPU:
descriptors against hand-computed ones, and every composed View against the
oracle's VIEW of the same movement chain (the oracle applies numpy's own
movement routines, the library composes strides: two independent
implementations of limn README, "Architecture", third rule)."""

import numpy as np
import pytest

import oracle
from reduce_view_amd import rv, synth


def _desc(v):
    return v.to_dict()


def _materialise(flat, d):
    shape = d["shape"]
    out = np.zeros(shape, flat.dtype)
    for idx in np.ndindex(*shape):
        if all(d["mask_lo"][k] <= idx[k] < d["mask_hi"][k] for k in range(len(shape))):
            out[idx] = flat[d["offset"] + sum(i * s for i, s in zip(idx, d["strides"]))]
    return out


def _compose(shape, movement):
    v = rv.rv_view_contiguous(shape)
    for name, a in movement:
        if name == "reshape":
            v = rv.rv_view_reshape(v, a)
        elif name == "permute":
            v = rv.rv_view_permute(v, a)
        elif name == "expand":
            v = rv.rv_view_expand(v, a)
        elif name == "pad":
            v = rv.rv_view_pad(v, [w[0] for w in a], [w[1] for w in a])
        elif name == "shrink":
            v = rv.rv_view_shrink(v, [w[0] for w in a], [w[1] for w in a])
    return _desc(v)


def test_hand_computed_descriptors():
    # the masked operand of the elementwise workload: shrink then pad cancels
    # the offset and leaves a mask
    d = _compose((4096, 4096), [("shrink", ((3, 4093), (5, 4091))), ("pad", ((3, 3), (5, 5)))])
    assert d == dict(shape=(4096, 4096), strides=(4096, 1), offset=0, mask_lo=(3, 5), mask_hi=(4093, 4091))
    # permuted operand
    assert _compose((4096, 4096), [("permute", (1, 0))])["strides"] == (1, 4096)
    # stride-0 row vector
    d = _compose((4096,), [("reshape", (1, 4096)), ("expand", (4096, 4096))])
    assert d["strides"] == (0, 1)
    # the broadcast matmul operands of the limn IR dump: (5, 0, 1) and (0, 1, 3)
    assert _compose((4, 5), [("reshape", (4, 1, 5)), ("expand", (4, 3, 5))])["strides"] == (5, 0, 1)
    assert _compose((5, 3), [("permute", (1, 0)), ("reshape", (1, 3, 5)), ("expand", (4, 3, 5))])["strides"] == (0, 1, 3)
    # reshape merges chained dims and splits one
    assert _compose((2, 3, 4), [("reshape", (6, 4))])["strides"] == (4, 1)
    d = _compose((6, 4), [("permute", (1, 0)), ("reshape", (2, 2, 6))])
    assert d["strides"] == (2, 1, 4)
    # pad only shifts the offset by before * stride
    d = _compose((5, 7), [("pad", ((2, 1), (0, 3)))])
    assert d["offset"] == -14 and d["mask_lo"] == (2, 0) and d["mask_hi"] == (7, 7)


MOVEMENT_CASES = [
    ((6, 7), [("permute", (1, 0))]),
    ((6, 7), [("shrink", ((1, 5), (2, 7))), ("pad", ((1, 1), (2, 0)))]),
    ((6, 7), [("pad", ((2, 0), (1, 3))), ("shrink", ((1, 8), (0, 9))), ("permute", (1, 0))]),
    ((1, 7), [("expand", (5, 7)), ("permute", (1, 0))]),
    ((4, 6), [("reshape", (2, 2, 6)), ("permute", (2, 0, 1)), ("shrink", ((1, 5), (0, 2), (1, 2)))]),
    ((4, 6), [("permute", (1, 0)), ("reshape", (3, 2, 4)), ("pad", ((0, 1), (1, 1), (0, 0)))]),
    ((3, 1, 5), [("expand", (3, 4, 5)), ("reshape", (3, 4, 5)), ("permute", (2, 1, 0))]),
    ((2, 3, 4), [("reshape", (6, 4)), ("shrink", ((1, 6), (0, 4))), ("pad", ((0, 0), (2, 2)))]),
]


@pytest.mark.parametrize("shape,movement", MOVEMENT_CASES)
def test_composed_view_equals_oracle_movement(shape, movement):
    x = np.random.default_rng(7).standard_normal(shape).astype(np.float32)
    d = _compose(shape, movement)
    got = _materialise(x.ravel(), d)
    g = synth.Spec()
    b = g.buffer("x", shape, "f32")
    g.output(g.contiguous(g.view(b, *movement)))
    ref, = oracle.run(g, {"x": x})
    assert got.shape == ref.shape
    assert got.tobytes() == ref.tobytes()


def test_masked_views_refuse_merging_reshape():
    v = rv.rv_view_pad(rv.rv_view_contiguous((4, 4)), (1, 0), (0, 0))
    with pytest.raises(rv.RVError) as e:
        rv.rv_view_reshape(v, (20,))
    assert e.value.name == "RV_E_UNSUPPORTED_LAYOUT"
    # a masked dim passing through unchanged composes
    d = _desc(rv.rv_view_reshape(v, (5, 1, 4)))
    assert d["mask_lo"] == (1, 0, 0) and d["mask_hi"] == (5, 1, 4)
