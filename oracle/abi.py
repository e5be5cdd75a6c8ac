"""``oracle_run``: the oracle driven by the library's own node descriptors.

TEST INFRASTRUCTURE (see the package docstring). The descriptors are read as
plain data in the layout the C ABI header documents (``rv_view``,
``rv_node``; units are elements, masks half-open per dim); nothing from the
library is imported or called. Each descriptor becomes one oracle node: a
VIEW is evaluated from its composed (shape, strides, offset, mask), so
running the same graph once from its movement chain (``oracle.run``) and
once from the descriptors the library composed checks the library's View
algebra against the oracle's movement rules.
"""

from __future__ import annotations

import ctypes

import numpy as np

from .interp import STORAGE, OracleError, run

MAX_DIMS = 8
_OPS = ["BUFFER", "CONST", "VIEW", "NEG", "EXP", "LOG", "SQRT", "RECIP", "CAST", "ADD", "MUL", "CMPLT", "WHERE",
        "SUM", "MAX", "CONTIGUOUS", "GATHER", "SCATTER", "ASSIGN", "CUSTOM"]
_DTYPES = ["f32", "bf16", "f16", "f64", "i32", "i16", "i8"]
_CUSTOM_SDPA_FWD = 1


class View(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("strides", ctypes.c_int64 * MAX_DIMS),
                ("offset", ctypes.c_int64), ("mask_lo", ctypes.c_int64 * MAX_DIMS),
                ("mask_hi", ctypes.c_int64 * MAX_DIMS)]


class Node(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("dtype", ctypes.c_int32), ("src", ctypes.c_int32 * 3),
                ("buf", ctypes.c_int32), ("reduce_axes", ctypes.c_uint32), ("reserved", ctypes.c_int32),
                ("cval", ctypes.c_double), ("view", View)]


class _Graph:
    def __init__(self):
        self.nodes: list[dict] = []
        self.outputs: list[int] = []


def _as_nodes(nodes, n: int) -> list:
    """The n descriptors as this module's Node structs (from any ctypes
    array or pointer with the documented layout)."""
    raw = ctypes.string_at(ctypes.addressof(nodes) if not isinstance(nodes, int) else nodes,
                           n * ctypes.sizeof(Node))
    return [Node.from_buffer_copy(raw, i * ctypes.sizeof(Node)) for i in range(n)]


def _graph(nodes: list, outputs) -> tuple[_Graph, dict]:
    g = _Graph()
    slots: dict[int, tuple] = {}
    for i, x in enumerate(nodes):
        if not (0 <= x.op < len(_OPS)):
            raise OracleError(f"node {i}: op {x.op}")
        op = _OPS[x.op]
        arity = {"BUFFER": 0, "CONST": 0, "ADD": 2, "MUL": 2, "CMPLT": 2, "GATHER": 2, "WHERE": 3,
                 "SCATTER": 3, "CUSTOM": 3}.get(op, 1)
        src = tuple(int(x.src[k]) for k in range(arity))
        shape = tuple(int(x.view.shape[d]) for d in range(x.view.ndim))
        nd: dict = dict(op=op, src=src)
        if op == "BUFFER":
            nd.update(slot=f"s{x.buf}", shape=shape, dtype=_DTYPES[x.dtype])
            slots[x.buf] = (shape, _DTYPES[x.dtype])
        elif op == "CONST":
            nd.update(value=float(x.cval), shape=shape, dtype=_DTYPES[x.dtype])
        elif op == "VIEW":
            v = x.view
            nd["raw"] = dict(shape=shape, strides=tuple(int(v.strides[d]) for d in range(v.ndim)),
                             offset=int(v.offset), mask_lo=tuple(int(v.mask_lo[d]) for d in range(v.ndim)),
                             mask_hi=tuple(int(v.mask_hi[d]) for d in range(v.ndim)))
        elif op == "CAST":
            nd["dtype"] = _DTYPES[x.dtype]
        elif op in ("SUM", "MAX"):
            nd["axes"] = tuple(d for d in range(32) if (x.reduce_axes >> d) & 1)
        elif op in ("GATHER", "SCATTER"):
            ax = [d for d in range(32) if (x.reduce_axes >> d) & 1]
            if len(ax) != 1:
                raise OracleError(f"node {i}: {op} needs exactly one axis bit")
            nd["axis"] = ax[0]
            if op == "SCATTER":
                nd["atomic"] = x.buf == 1
        elif op == "CUSTOM":
            if x.buf != _CUSTOM_SDPA_FWD:
                raise OracleError(f"node {i}: CUSTOM kernel {x.buf}")
            nd.update(kind="sdpa_fwd", scale=float(x.cval), causal=bool(x.reduce_axes & 1),
                      out=int((x.reduce_axes >> 16) & 0xFF), dtype=_DTYPES[x.dtype])
        elif op == "ASSIGN":
            raise OracleError(f"node {i}: ASSIGN is not evaluated by this oracle")
        g.nodes.append(nd)
    g.outputs = [int(o) for o in outputs]
    return g, slots


def oracle_run(nodes, n: int, outputs, nout: int, bufs: list, nbufs: int) -> int:
    """Evaluate the n descriptors; ``bufs`` holds host arrays, the inputs by
    slot then one writable array per output (the buffer order the library's
    launch takes). The outputs are written in storage form. Returns 0."""
    descs = _as_nodes(nodes, n)
    g, slots = _graph(descs, list(outputs)[:nout])
    n_in = max(slots) + 1 if slots else 0
    if nbufs != n_in + nout:
        raise OracleError(f"expected {n_in + nout} buffers, got {nbufs}")
    inputs = {}
    for s, (shape, dt) in slots.items():
        a = np.asarray(bufs[s])
        if a.dtype != STORAGE[dt] or a.size < int(np.prod(shape)):
            raise OracleError(f"input {s}: {a.dtype}/{a.size}, need {dt}/{int(np.prod(shape))}")
        inputs[f"s{s}"] = a.ravel()[: int(np.prod(shape))].reshape(shape)
    outs = run(g, inputs)
    for k, o in enumerate(outs):
        dst = bufs[n_in + k]
        if dst.dtype != o.dtype or dst.size != o.size:
            raise OracleError(f"output {k}: {dst.dtype}/{dst.size}, the graph gives {o.dtype}/{o.size}")
        dst.reshape(-1)[:] = o.reshape(-1)
    return 0
