"""A CPU interpreter of the library's lowered kernels, read from rv_describe:
every leaf is loaded through its lowered View (offset + sum_d i_d * stride_d
over the kernel's iteration domain, zero outside the mask), the ops run in
the listed order over the whole domain, reductions fold in ascending order
over the reduced dims, and stores write through their lowered Views.

This is the limn README's "Correctness" pattern for the scheduler and codegen
layer: interpret the lowered program instruction by instruction and diff the
numbers, so the plan means what it says. Primitive semantics come from the
oracle's per-primitive helpers (test infrastructure)."""

from __future__ import annotations

import numpy as np

from oracle import interp as O

STORAGE = O.STORAGE


def _gather(flat: np.ndarray, view: dict, shape) -> np.ndarray:
    shape = tuple(shape)
    idx = np.full(shape, int(view["offset"]), dtype=np.int64)
    inside = np.ones(shape, dtype=bool)
    for d, g in enumerate(np.indices(shape, dtype=np.int64) if shape else []):
        idx = idx + g * int(view["strides"][d])
        inside &= (g >= view["mask_lo"][d]) & (g < view["mask_hi"][d])
    assert not np.any(inside & ((idx < 0) | (idx >= flat.size))), "lowered view reads out of bounds"
    vals = flat[np.where(inside, idx, 0)] if flat.size else np.zeros(shape, flat.dtype)
    return np.where(inside, vals, np.zeros((), flat.dtype)).astype(flat.dtype)


def _scatter(flat: np.ndarray, view: dict, shape, vals: np.ndarray) -> None:
    shape = tuple(shape)
    idx = np.full(shape, int(view["offset"]), dtype=np.int64)
    for d, g in enumerate(np.indices(shape, dtype=np.int64) if shape else []):
        idx = idx + g * int(view["strides"][d])
    assert idx.min() >= 0 and idx.max() < flat.size, "lowered store out of bounds"
    flat[idx.ravel()] = np.broadcast_to(vals, shape).ravel()


def run_plan(desc: dict, inputs: list, out_specs: list) -> list:
    """``inputs``: flat storage arrays per input slot; ``out_specs``: (shape,
    dtype) per output. Returns the outputs (shaped)."""
    outs = [np.zeros(int(np.prod(s)), dtype=STORAGE[dt]) for s, dt in out_specs]
    ws: dict[int, np.ndarray] = {}

    def mem(loc, dtype, size_hint=0):
        if loc["kind"] == "input":
            return inputs[loc["index"]]
        if loc["kind"] == "output":
            return outs[loc["index"]]
        r = loc["index"]
        if r not in ws or ws[r].size < size_hint:
            ws[r] = np.zeros(max(size_hint, 1), dtype=STORAGE[dtype])
        return ws[r]

    for k in desc["kernels"]:
        dom = tuple(k["domain"])
        red = tuple(k["reduce_dims"])
        ops = k["ops"]
        if k["class"] == "FOLD":
            part = ws[k["plan_detail"]["src_region"]]
            s = np.float32(0.0)
            for v in part[: k["plan_detail"]["partials"]]:
                s = np.float32(s + v)
            st = k["stores"][0]
            o = mem(st["loc"], st["dtype"])
            val = O._narrow(np.array([s], np.float32), st["dtype"]) if st["dtype"] in ("bf16", "f16") else \
                np.array([s]).astype(STORAGE[st["dtype"]])
            o[st["view"]["offset"]] = val[0]
            continue
        if k["plan"] == "empty":
            continue
        vals: dict[int, np.ndarray] = {}
        if k["class"] == "MFMA" and k["plan"] == "gemm_w6" and k["plan_detail"]["split_k"] > 1:
            _mfma_slices(k, dom, mem)
            continue
        if k["class"] == "SCATTER":
            _scatter_step(k, dom, mem)
            continue
        _evaluate(k, dom, red, mem, vals)
        for st in k["stores"]:
            v = vals[st_ex(k, st)]
            if k["class"] == "MFMA" and st["loc"]["kind"] == "workspace":
                # one partial: the epilogue summed over the whole (m, n) plane
                plane = np.ascontiguousarray(v[:, :, :1]).astype(np.float32).ravel()
                s = np.float32(0.0)
                for x in plane:
                    s = np.float32(s + x)
                buf = mem(st["loc"], "f32", 1)
                buf[:] = 0
                buf[0] = s
                continue
            # a reduced dim the store does not walk (stride 0) is written once
            sshape = tuple(1 if (d in red and st["view"]["strides"][d] == 0) else dom[d] for d in range(len(dom)))
            if any(sshape[d] == 1 and v.shape[d] != 1 for d in range(len(dom))):
                v = v[tuple(slice(0, 1) if (sshape[d] == 1 and v.shape[d] != 1) else slice(None)
                            for d in range(len(dom)))]
            v = np.broadcast_to(v, sshape)
            if int(np.prod(sshape)) == 0:
                continue
            size = 1 + int(np.dot(np.array(sshape) - 1, np.array(st["view"]["strides"]))) + st["view"]["offset"]
            o = mem(st["loc"], st["dtype"], size)
            if st["loc"]["kind"] == "workspace" and o.dtype != STORAGE[st["dtype"]]:
                ws[st["loc"]["index"]] = o = np.zeros(size, STORAGE[st["dtype"]])
            _scatter(o, st["view"], sshape, v.astype(STORAGE[st["dtype"]]))
    return [o.reshape(s) for o, (s, _) in zip(outs, out_specs)]


def _evaluate(k, dom, red, mem, vals, only=None):
    """Every op of kernel ``k`` (or those in ``only``) over the domain
    ``dom``, in order."""
    ops, leaves = k["ops"], k["leaves"]
    for i, op in enumerate(ops):
        if only is not None and i not in only:
            continue
        name, dt = op["op"], op["dtype"]
        if name == "LOAD":
            L = leaves[op["leaf"]]
            if L["zero"]:
                vals[i] = np.zeros(dom, STORAGE[dt])
            else:
                # constant along a reduced dim (stride 0, unmasked): one
                # copy there, broadcast where used (a cell whose reduce
                # range is empty still sees it)
                v = L["view"]
                gshape = tuple(1 if (d in red and v["strides"][d] == 0 and v["mask_lo"][d] == 0
                                     and v["mask_hi"][d] == dom[d]) else dom[d] for d in range(len(dom)))
                vals[i] = _gather(mem(L["loc"], L["dtype"]), v, gshape)
        elif name == "CONST":
            v = np.array([float(op["cval"])], np.float64)
            if dt == "bf16":
                c = O.f32_to_bf16(v.astype(np.float32))
            elif dt in O.INTS:
                c = v.astype(np.int64).astype(STORAGE[dt])
            else:
                c = v.astype(STORAGE[dt])
            vals[i] = np.broadcast_to(c.reshape((1,) * len(dom)), dom)
        elif name == "MFMA_ACC" and k["plan"] == "gemm_slices":
            # the k-slices' planes summed in slice order
            pd = k["plan_detail"]
            ws = mem({"kind": "workspace", "index": pd["slices_region"]}, "f32")
            cells = dom[0] * dom[1]
            acc = ws[:cells].copy()
            for sl in range(1, pd["split_k"]):
                acc = (acc + ws[sl * pd["plane"]: sl * pd["plane"] + cells]).astype(np.float32)
            vals[i] = np.broadcast_to(acc.reshape(dom[0], dom[1], 1), dom)
        elif name == "MFMA_ACC":
            a_leaf = leaves[_mfma_leaf(k, "a")]
            b_leaf = leaves[_mfma_leaf(k, "b")]
            A = O.bf16_to_f32(_gather(mem(a_leaf["loc"], "bf16"), a_leaf["view"], dom))
            B = O.bf16_to_f32(_gather(mem(b_leaf["loc"], "bf16"), b_leaf["view"], dom))
            acc = np.zeros(dom[:2] + (1,), np.float32)
            for kk in range(dom[2]):
                acc = (acc + (A[:, :, kk:kk + 1] * B[:, :, kk:kk + 1]).astype(np.float32)).astype(np.float32)
            vals[i] = np.broadcast_to(acc, dom)
        elif name in ("SUM", "MAX"):
            x = np.ascontiguousarray(np.broadcast_to(vals[op["a"]], dom))
            vals[i] = O._reduce(name, x, ops[op["a"]]["dtype"], tuple(red))  # reduced dims kept as 1
        elif name == "CAST":
            vals[i] = O._cast(np.ascontiguousarray(vals[op["a"]]), ops[op["a"]]["dtype"], dt)
        elif name in ("NEG", "EXP", "LOG", "SQRT", "RECIP"):
            vals[i] = O._unary(name, np.ascontiguousarray(vals[op["a"]]), dt)
        elif name in ("ADD", "MUL", "CMPLT"):
            vals[i] = O._binary(name, np.ascontiguousarray(vals[op["a"]]), np.ascontiguousarray(vals[op["b"]]),
                                ops[op["a"]]["dtype"])
        elif name == "WHERE":
            vals[i] = np.where(vals[op["a"]] != 0, vals[op["b"]], vals[op["c"]]).astype(STORAGE[dt])
        elif name == "GATHER":
            L, gp = leaves[op["leaf"]], op["gather"]
            t = np.broadcast_to(vals[op["a"]], dom).astype(np.int64)
            if L["zero"]:
                vals[i] = np.zeros(dom, STORAGE[dt])
                continue
            v = L["view"]
            idx = np.full(dom, int(v["offset"]), dtype=np.int64) + (t - int(gp["lo"])) * int(gp["stride"])
            inside = (t >= gp["lo"]) & (t < gp["hi"])
            for d, g in enumerate(np.indices(dom, dtype=np.int64) if dom else []):
                idx = idx + g * int(v["strides"][d])
                inside &= (g >= v["mask_lo"][d]) & (g < v["mask_hi"][d])
            flat = mem(L["loc"], L["dtype"])
            assert not np.any(inside & ((idx < 0) | (idx >= flat.size))), "gathered read out of bounds"
            vals[i] = np.where(inside, flat[np.where(inside, idx, 0)], np.zeros((), flat.dtype)).astype(flat.dtype)
        else:
            raise AssertionError(name)


def _reach(ops, root):
    out, stack = set(), [root]
    while stack:
        i = stack.pop()
        if i is None or i < 0 or i in out:
            continue
        out.add(i)
        stack += [ops[i]["a"], ops[i]["b"], ops[i]["c"]]
    return out


def _scatter_step(k, dom, mem):
    """A scatter step as the additions it stands for: the ordered fold is the
    base plus every value at its target in index order; the atomic step the
    same adds into the target, which already holds the base. Keys and radix
    passes only order the adds."""
    part = k["plan_detail"]["part"]
    if part not in ("fold", "atomic"):
        return
    sc = k["scatter"]
    axis = k["plan_detail"]["axis"]
    oshape = tuple(sc["out_shape"])
    o = mem(sc["out"], sc["dtype"], int(np.prod(oshape))).reshape(oshape)
    ops = k["ops"]
    vals: dict[int, np.ndarray] = {}
    if part == "fold":
        _evaluate(k, oshape, (), mem, vals, only=_reach(ops, sc["base"]))
        o[...] = np.broadcast_to(vals[sc["base"]], oshape)
        vals = {}
    _evaluate(k, dom, (), mem, vals, only=_reach(ops, sc["index"]) | _reach(ops, sc["values"]))
    index = np.broadcast_to(vals[sc["index"]], dom)
    values = np.broadcast_to(vals[sc["values"]], dom)
    rest = np.indices(tuple(dom[d] for d in range(len(dom)) if d != axis))
    for kk in range(dom[axis]):
        t = np.take(index, kk, axis=axis)
        v = np.take(values, kk, axis=axis)
        sel = (t >= 0) & (t < oshape[axis])
        tgt = list(rest)
        tgt.insert(axis, np.where(sel, t, 0))
        cur = np.asarray(o[tuple(tgt)])
        new = np.reshape(O._binary("ADD", np.ascontiguousarray(cur), np.ascontiguousarray(v), sc["dtype"]), cur.shape)
        o[tuple(tgt)] = np.where(sel, new, cur)


def st_ex(k, st):
    """The op a store writes."""
    return st["ex"]


def _mfma_slices(k, dom, mem):
    """A contraction's k-slice kernel: slice s covers k in [s Ks, (s + 1) Ks)
    of the padded depth (the cells past the output's depth are zero padding);
    each slice's float32 accumulators, k in order, go to plane s of the
    slices region ([slice][m][n], planes ``plane`` floats apart)."""
    pd, leaves = k["plan_detail"], k["leaves"]
    S, Ke = pd["split_k"], pd["extent"][2]
    Ks = Ke // S
    a_leaf = leaves[_mfma_leaf(k, "a")]
    b_leaf = leaves[_mfma_leaf(k, "b")]
    A = O.bf16_to_f32(_gather(mem(a_leaf["loc"], "bf16"), a_leaf["view"], dom))
    B = O.bf16_to_f32(_gather(mem(b_leaf["loc"], "bf16"), b_leaf["view"], dom))
    cells = dom[0] * dom[1]
    plane = (cells + 63) // 64 * 64
    ws = mem({"kind": "workspace", "index": pd["slices_region"]}, "f32", S * plane)
    for sl in range(S):
        acc = np.zeros(dom[:2], np.float32)
        for kk in range(sl * Ks, min((sl + 1) * Ks, dom[2])):
            acc = (acc + (A[:, :, kk] * B[:, :, kk]).astype(np.float32)).astype(np.float32)
        ws[sl * plane: sl * plane + cells] = acc.ravel()


def _mfma_leaf(k, which):
    # the leaves the contraction reads (an operand copied into workspace
    # first is read from its copy)
    return k["plan_detail"]["operand_leaves"][0 if which == "a" else 1]
