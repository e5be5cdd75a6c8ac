"""The CPU oracle: a plain interpreter that evaluates one primitive per graph
node, materialising every node's value, with no fusion.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or run anything under ``oracle/``. The library's
compute path never does, and this module imports nothing from the library.

What it follows:
  * limn README, "Architecture": the numpy device interprets the graph one
    numpy call per node with no fusion and is the reference every compiled
    backend is diffed against; a matmul is a broadcast multiply and a reduce,
    so the (m, n, k) intermediate is built rather than walked.
  * limn README, "Architecture" (third rule) and "Reading the schedule": a
    View is (shape, strides, offset, mask); reshape, permute, expand, pad and
    shrink compose into it; a padded read is a range check on a loop
    variable that yields a literal zero outside the range.
  * limn README, "The op set": the primitive set and the dtype rules
    (float16/bfloat16 are storage widths widened to compute; a reduce keeps a
    float32 running total and rounds back once; narrow ints wrap modulo
    2**width).
  * limn README, "Reading the schedule" and "Backends": a reduce walks its
    axis in order from the reduce identity.

Readings where the pages leave a step open (each is listed in the design
notes of the repository):
  * float32 arithmetic is IEEE round-to-nearest-even per primitive; EXP and
    LOG are evaluated in float64 and rounded once to float32 (correctly
    rounded but for ties closer than 2**-29 ulp); SQRT and RECIP are the
    correctly rounded float32 operations.
  * a reduce folds in ascending row-major order over its reduce indices.
  * a float32 running total whose length n has (n - 1) * 2**-24 >= 1/3 (the
    point where the reduction-order bound gamma_{n-1} stops meaning
    anything; Litmus README, "Support map and limits", item 7) is kept in
    float64 instead and rounded once.
  * CMPLT produces int8 0/1; WHERE treats any nonzero condition as true.
  * MAX starts from -inf (ints: the smallest value of the width), a NaN
    anywhere in the row gives NaN, and -0 orders below +0 (IEEE 754-2019
    maximum), so the result's bits do not depend on the fold order.
  * CAST rounds to nearest even and keeps NaN a NaN; a value cast to a half
    width (float16, bfloat16) is a float32 first, so a float64 or a large
    int32 source is rounded twice; float -> int truncates toward zero and
    wraps modulo 2**width (undefined beyond int32, for NaN and infinities);
    int -> int wraps.
  * GATHER along an axis reads data at the position with that axis
    coordinate replaced by the index (the index has the output's shape); an
    index outside the axis reads zero, as a read outside a View's mask does.
  * SCATTER along an axis adds each value into a copy of base at the
    position with that axis coordinate replaced by the index; colliding adds
    fold in ascending row-major order of the index positions, each one the
    dtype's ADD (rounded to the dtype, wrapping for ints); an index outside
    the axis drops its value.
  * a node too large to hold (the limn README warns that the reference runs
    out of memory on a large matmul) is evaluated in slabs along dim 0 when
    its consumer is a reduce that keeps dim 0. This changes no value: each
    output cell is still produced by the same in-order fold.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_fold.so")

STORAGE = {
    "f32": np.float32, "f64": np.float64, "f16": np.float16, "bf16": np.uint16,
    "i32": np.int32, "i16": np.int16, "i8": np.int8,
}
FLOATS = ("f32", "f64", "f16", "bf16")
INTS = ("i32", "i16", "i8")
ELEMENTWISE = ("NEG", "EXP", "LOG", "SQRT", "RECIP", "CAST", "ADD", "MUL", "CMPLT", "WHERE")


class OracleError(Exception):
    """A graph the oracle refuses (shape, dtype or op contract)."""


# ---------------------------------------------------------------------------
# the C folds
# ---------------------------------------------------------------------------
_lib = None


def _fold_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise OracleError(f"{_LIB_PATH} is not built; run oracle/build.py")
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        for name in ("fold_sum_f32", "fold_sum_f32_wide", "fold_sum_f32_to_f64", "fold_sum_f64",
                     "fold_sum_i32", "fold_max_f32", "fold_max_f64"):
            getattr(lib, name).argtypes = [p, i64, i64, p]
            getattr(lib, name).restype = None
        lib.fold_max_i32.argtypes = [p, i64, i64, ctypes.c_int32, p]
        lib.fold_max_i32.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# bfloat16 <-> float32 (bfloat16 is the top half of a float32)
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: the 16 bits become the high half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest with ties to even; NaN stays NaN
    (quiet bit set), overflow rounds to infinity."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    r = np.where(is_nan, ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF), r)
    return r.astype(np.uint16)


def _widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage -> compute width: float32 for the half widths, else itself."""
    if dtype == "bf16":
        return bf16_to_f32(arr)
    if dtype == "f16":
        return arr.astype(np.float32)
    return arr


def _narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """Compute width -> storage (one rounding for the half widths)."""
    if dtype == "bf16":
        return f32_to_bf16(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    return np.asarray(x).astype(STORAGE[dtype], copy=False)


def _to_dtype_from_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """CAST of float values (float32 or float64 array) to ``dtype``.

    * to an int: truncate toward zero, then wrap modulo 2**width (defined
      where the truncated value fits in int32; NaN, infinities and larger
      magnitudes are left undefined);
    * to float32 / float64: one rounding to nearest even;
    * to a half width (float16, bfloat16): the value is a float32 first and
      is rounded once from there (limn README, "The op set": the half widths
      are storage computed in float32), so a float64 source is rounded twice,
      to float32 and then to the half width."""
    if dtype in INTS:
        with np.errstate(invalid="ignore"):
            t = np.trunc(x.astype(np.float64))
            return t.astype(np.int64).astype(STORAGE[dtype])
    with np.errstate(over="ignore", invalid="ignore"):
        if dtype in ("bf16", "f16"):
            return _narrow(x.astype(np.float32), dtype)
        return x.astype(STORAGE[dtype])


# ---------------------------------------------------------------------------
# shape / dtype inference
# ---------------------------------------------------------------------------

def _movement_shape(shape, mv):
    name, arg = mv
    shape = tuple(shape)
    if name == "reshape":
        new = tuple(arg)
        if any(s < 0 for s in new) or int(np.prod(new, dtype=np.int64)) != int(np.prod(shape, dtype=np.int64)):
            raise OracleError(f"reshape {shape} -> {new}")
        return new
    if name == "permute":
        perm = tuple(arg)
        if sorted(perm) != list(range(len(shape))):
            raise OracleError(f"permute {perm} of rank {len(shape)}")
        return tuple(shape[p] for p in perm)
    if name == "expand":
        new = tuple(arg)
        if len(new) != len(shape) or any(o != 1 and o != n for o, n in zip(shape, new)):
            raise OracleError(f"expand {shape} -> {new}")
        return new
    if name == "pad":
        widths = tuple(tuple(w) for w in arg)
        if len(widths) != len(shape) or any(b < 0 or a < 0 for b, a in widths):
            raise OracleError(f"pad {widths}")
        return tuple(s + b + a for s, (b, a) in zip(shape, widths))
    if name == "shrink":
        rng = tuple(tuple(r) for r in arg)
        if len(rng) != len(shape) or any(not (0 <= lo <= hi <= s) for s, (lo, hi) in zip(shape, rng)):
            raise OracleError(f"shrink {rng} of {shape}")
        return tuple(hi - lo for lo, hi in rng)
    raise OracleError(f"unknown movement {name}")


def infer(spec) -> list:
    """(shape, dtype) of every node, checking the op contracts."""
    out = []
    for i, nd in enumerate(spec.nodes):
        op = nd["op"]
        src = nd.get("src", ())
        for s in src:
            if not (0 <= s < i):
                raise OracleError(f"node {i}: source {s} is not an earlier node")
        if op in ("BUFFER", "CONST"):
            out.append((tuple(nd["shape"]), nd["dtype"]))
        elif op == "VIEW":
            shp, dt = out[src[0]]
            if "raw" in nd and nd["raw"] is not None:
                shp = tuple(nd["raw"]["shape"])
            else:
                for mv in nd["movement"]:
                    shp = _movement_shape(shp, mv)
            out.append((shp, dt))
        elif op in ("NEG", "EXP", "LOG", "SQRT", "RECIP"):
            shp, dt = out[src[0]]
            if op != "NEG" and dt not in FLOATS:
                raise OracleError(f"node {i}: {op} needs a float dtype")
            out.append((shp, dt))
        elif op == "CAST":
            out.append((out[src[0]][0], nd["dtype"]))
        elif op in ("ADD", "MUL", "CMPLT"):
            (s0, d0), (s1, d1) = out[src[0]], out[src[1]]
            if s0 != s1 or d0 != d1:
                raise OracleError(f"node {i}: {op} of {s0}/{d0} and {s1}/{d1}")
            out.append((s0, "i8" if op == "CMPLT" else d0))
        elif op == "WHERE":
            (sc, _), (s1, d1), (s2, d2) = out[src[0]], out[src[1]], out[src[2]]
            if not (sc == s1 == s2) or d1 != d2:
                raise OracleError(f"node {i}: WHERE shapes/dtypes")
            out.append((s1, d1))
        elif op in ("SUM", "MAX"):
            shp, dt = out[src[0]]
            axes = tuple(nd["axes"])
            if any(not (0 <= a < len(shp)) for a in axes) or len(set(axes)) != len(axes):
                raise OracleError(f"node {i}: axes {axes} of rank {len(shp)}")
            out.append((tuple(1 if d in axes else s for d, s in enumerate(shp)), dt))
        elif op == "CONTIGUOUS":
            out.append(out[src[0]])
        elif op == "GATHER":
            (sd, dd), (si, di) = out[src[0]], out[src[1]]
            ax = nd["axis"]
            if di != "i32" or len(sd) != len(si) or not (0 <= ax < len(sd)) or \
                    any(sd[d] != si[d] for d in range(len(sd)) if d != ax):
                raise OracleError(f"node {i}: GATHER of {sd}/{dd} by {si}/{di} along {ax}")
            out.append((si, dd))
        elif op == "SCATTER":
            (sb, db), (si, di), (sv, dv) = out[src[0]], out[src[1]], out[src[2]]
            ax = nd["axis"]
            if di != "i32" or sv != si or dv != db or len(sb) != len(si) or not (0 <= ax < len(sb)) or \
                    any(sb[d] != si[d] for d in range(len(sb)) if d != ax):
                raise OracleError(f"node {i}: SCATTER into {sb}/{db} of {sv}/{dv} by {si}/{di} along {ax}")
            out.append((sb, db))
        elif op == "CUSTOM" and nd.get("kind") == "sdpa_fwd":
            (sq, dq), (sk, dk), (sv, dv) = out[src[0]], out[src[1]], out[src[2]]
            if len(sq) != 3 or sk != sv or len(sk) != 3 or sq[0] != sk[0] or sq[2] != sk[2] or \
                    (dq, dk, dv) != ("bf16", "bf16", "bf16"):
                raise OracleError(f"node {i}: sdpa_fwd of {sq}/{dq}, {sk}/{dk}, {sv}/{dv}")
            if nd["out"] == 0:
                out.append((sq, nd["dtype"]))
            else:
                out.append(((sq[0], sq[1], 1), "f32"))
        else:
            raise OracleError(f"node {i}: op {op} is not evaluated by this oracle")
    return out


# ---------------------------------------------------------------------------
# primitive evaluation
# ---------------------------------------------------------------------------

def _apply_movement(arr: np.ndarray, mv) -> np.ndarray:
    """One movement op with numpy's own routine; the result may be a
    non-contiguous or broadcast numpy view (no copy is made where numpy can
    avoid one)."""
    name, arg = mv
    if name == "reshape":
        return arr.reshape(tuple(arg))
    if name == "permute":
        return np.transpose(arr, tuple(arg))
    if name == "expand":
        return np.broadcast_to(arr, tuple(arg))
    if name == "pad":
        return np.pad(arr, tuple(tuple(w) for w in arg), mode="constant", constant_values=0)
    if name == "shrink":
        return arr[tuple(slice(lo, hi) for lo, hi in arg)]
    raise OracleError(name)


def _raw_view(src: np.ndarray, raw: dict) -> np.ndarray:
    """Explicit View descriptor: cell i reads src.flat[offset + sum_d i_d*s_d]
    when lo_d <= i_d < hi_d for every d, else zero."""
    flat = np.ascontiguousarray(src).reshape(-1)
    shape = tuple(raw["shape"])
    idx = np.full(shape, int(raw["offset"]), dtype=np.int64)
    inside = np.ones(shape, dtype=bool)
    grids = np.indices(shape, dtype=np.int64) if len(shape) else []
    for d, g in enumerate(grids):
        idx = idx + g * int(raw["strides"][d])
        inside &= (g >= int(raw["mask_lo"][d])) & (g < int(raw["mask_hi"][d]))
    if np.any(inside & ((idx < 0) | (idx >= flat.size))):
        raise OracleError("raw view reads outside its buffer")
    vals = flat[np.where(inside, idx, 0)] if flat.size else np.zeros(shape, flat.dtype)
    return np.where(inside, vals, np.zeros((), flat.dtype)).astype(flat.dtype)


def _unary(op: str, x: np.ndarray, dt: str) -> np.ndarray:
    if dt in INTS:
        if op == "NEG":
            return np.negative(x).astype(x.dtype)
        raise OracleError(f"{op} of an int")
    w = _widen(x, dt)
    with np.errstate(all="ignore"):
        if op == "NEG":
            r = np.negative(w)
        elif op in ("EXP", "LOG"):
            fn = np.exp if op == "EXP" else np.log
            if w.dtype == np.float64:
                r = fn(w)
            else:
                r = fn(w.astype(np.float64)).astype(np.float32)
        elif op == "SQRT":
            r = np.sqrt(w)
        elif op == "RECIP":
            r = np.asarray(1.0, dtype=w.dtype) / w
        else:
            raise OracleError(op)
    return _narrow(r, dt)


def _binary(op: str, x: np.ndarray, y: np.ndarray, dt: str) -> np.ndarray:
    if dt in INTS:
        with np.errstate(all="ignore"):
            if op == "ADD":
                return np.add(x, y, dtype=x.dtype)
            if op == "MUL":
                return np.multiply(x, y, dtype=x.dtype)
            return (x < y).astype(np.int8)
    a, b = _widen(x, dt), _widen(y, dt)
    with np.errstate(all="ignore"):
        if op == "ADD":
            return _narrow(a + b, dt)
        if op == "MUL":
            return _narrow(a * b, dt)
        return (a < b).astype(np.int8)


def _cast(x: np.ndarray, src_dt: str, dst_dt: str) -> np.ndarray:
    """CAST (limn README, "The op set", dtype paragraph). int -> int wraps
    modulo 2**width; int -> float64 is exact; int -> float32 rounds once to
    nearest even; int -> a half width goes through float32 (two roundings);
    float sources follow ``_to_dtype_from_float``."""
    if src_dt == dst_dt:
        return x.copy()
    if src_dt in INTS:
        if dst_dt in INTS:
            return x.astype(np.int64).astype(STORAGE[dst_dt])
        if dst_dt == "f64":
            return x.astype(np.float64)
        r = x.astype(np.float64).astype(np.float32) if dst_dt != "f32" else x.astype(np.float32)
        with np.errstate(over="ignore"):
            return _narrow(r, dst_dt) if dst_dt in ("bf16", "f16") else r
    w = _widen(x, src_dt)
    return _to_dtype_from_float(w, dst_dt)


def _reduce(op: str, x: np.ndarray, dt: str, axes) -> np.ndarray:
    """Fold ``x`` over ``axes`` (kept as size 1) in ascending row-major order."""
    shape = x.shape
    nd = len(shape)
    keep = [d for d in range(nd) if d not in axes]
    moved = np.transpose(x, keep + list(axes))
    cells = int(np.prod([shape[d] for d in keep], dtype=np.int64))
    n = int(np.prod([shape[d] for d in axes], dtype=np.int64))
    out_shape = tuple(1 if d in axes else shape[d] for d in range(nd))
    lib = _fold_lib()
    if dt in INTS:
        flat = np.ascontiguousarray(moved.astype(np.int32)).reshape(cells, n)
        res = np.empty(cells, dtype=np.int32)
        if op == "SUM":
            lib.fold_sum_i32(_ptr(flat), cells, n, _ptr(res))
        else:
            lib.fold_max_i32(_ptr(flat), cells, n, int(np.iinfo(STORAGE[dt]).min), _ptr(res))
        return res.astype(STORAGE[dt]).reshape(out_shape)
    if dt == "f64":
        flat = np.ascontiguousarray(moved, dtype=np.float64).reshape(cells, n)
        res = np.empty(cells, dtype=np.float64)
        (lib.fold_sum_f64 if op == "SUM" else lib.fold_max_f64)(_ptr(flat), cells, n, _ptr(res))
        return res.reshape(out_shape)
    flat = np.ascontiguousarray(_widen(np.ascontiguousarray(moved), dt), dtype=np.float32).reshape(cells, n)
    res = np.empty(cells, dtype=np.float32)
    if op == "MAX":
        lib.fold_max_f32(_ptr(flat), cells, n, _ptr(res))
    elif (n - 1) * 2.0 ** -24 >= 1.0 / 3.0:
        lib.fold_sum_f32_wide(_ptr(flat), cells, n, _ptr(res))
    else:
        lib.fold_sum_f32(_ptr(flat), cells, n, _ptr(res))
    return _narrow(res, dt).reshape(out_shape)


def gather(data: np.ndarray, index: np.ndarray, axis: int, dt: str) -> np.ndarray:
    """GATHER (limn README, "The op set", indexed): out[p] = data[p with its
    ``axis`` coordinate replaced by index[p]]; an index outside the axis
    reads the zero of the dtype (the reading for an out-of-range index, as
    an out-of-mask View cell reads zero)."""
    n = data.shape[axis]
    ok = (index >= 0) & (index < n)
    picked = np.take_along_axis(data, np.where(ok, index, 0).astype(np.int64), axis=axis)
    return np.where(ok, picked, np.zeros((), data.dtype)).astype(data.dtype)


def scatter(base: np.ndarray, index: np.ndarray, values: np.ndarray, axis: int, dt: str) -> np.ndarray:
    """SCATTER (limn README, "The op set", indexed; "Backends": the C device
    folds a scatter's colliding adds serially): a copy of base, then for
    every position p of index in ascending row-major order, values[p] is
    ADDed (the dtype's ADD, one rounding each) at p with its ``axis``
    coordinate replaced by index[p]; an index outside the axis drops its
    value. Positions that differ only off ``axis`` never collide, so the
    loop runs over the ``axis`` coordinate in order with the rest at once."""
    out = np.array(base, copy=True)
    n = base.shape[axis]
    idx = np.moveaxis(index, axis, 0)
    val = np.moveaxis(values, axis, 0)
    o = np.moveaxis(out, axis, 0)  # a view: writes land in out
    rest = np.indices(idx.shape[1:]) if idx.ndim > 1 else np.zeros((0,), np.int64)
    for k in range(idx.shape[0]):
        sel = (idx[k] >= 0) & (idx[k] < n)
        tgt = (np.where(sel, idx[k], 0),) + tuple(rest)
        cur = np.asarray(o[tgt])
        new = np.reshape(_binary("ADD", np.ascontiguousarray(cur), np.ascontiguousarray(val[k]), dt), cur.shape)
        o[tgt] = np.where(sel, new, cur)
    return out


def sdpa_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool, out_dtype: str = "f32",
             block: int = 64):
    """Fused attention forward evaluated as the composition of primitives it
    stands for (limn README, "The op set": a device without the CUSTOM
    kernel composes it from primitives, and the numpy device's evaluation
    is the reference). bfloat16 q (H, Tq, D), k and v (H, Tk, D); per head
    and block of query rows, every step one primitive with its rounding:
      S = SUM_d CAST(q) * CAST(k)        (products exact, folded in order)
      S = S * CONST(scale)               (scale rounded to float32)
      S = S where key j <= query i, else -inf   (causal only; exact)
      m = MAX_j S;  e = EXP(S + NEG(m));  s = SUM_j e;  P = e * RECIP(s)
      O = SUM_j P * CAST(v)              (folded over keys in order)
      L = m + LOG(s)                     (the row's logsumexp)
    Returns (O in ``out_dtype``, L float32 (H, Tq, 1))."""
    H, Tq, D = q.shape
    Tk = k.shape[1]
    sc = np.float32(scale).reshape(1, 1, 1)
    O = np.empty((H, Tq, D), np.float32)
    L = np.empty((H, Tq, 1), np.float32)
    for h in range(H):
        kf = bf16_to_f32(k[h])[None, :, :]
        vf = bf16_to_f32(v[h])[None, :, :]
        for i0 in range(0, Tq, block):
            i1 = min(Tq, i0 + block)
            qf = bf16_to_f32(q[h, i0:i1])[:, None, :]
            prod = _binary("MUL", np.broadcast_to(qf, (i1 - i0, Tk, D)).copy(),
                           np.broadcast_to(kf, (i1 - i0, Tk, D)).copy(), "f32")
            S = _reduce("SUM", prod, "f32", (2,))[:, :, 0]
            S = _binary("MUL", S, np.broadcast_to(sc[0], S.shape).copy(), "f32")
            if causal:
                qi = np.arange(i0, i1)[:, None]
                kj = np.arange(Tk)[None, :]
                S = np.where(kj <= qi, S, np.float32(-np.inf)).astype(np.float32)
            m = _reduce("MAX", S, "f32", (1,))
            e = _unary("EXP", _binary("ADD", S, np.broadcast_to(_unary("NEG", m, "f32"), S.shape).copy(), "f32"),
                       "f32")
            ssum = _reduce("SUM", e, "f32", (1,))
            P = _binary("MUL", e, np.broadcast_to(_unary("RECIP", ssum, "f32"), e.shape).copy(), "f32")
            pv = _binary("MUL", np.broadcast_to(P[:, :, None], (i1 - i0, Tk, D)).copy(),
                         np.broadcast_to(vf, (i1 - i0, Tk, D)).copy(), "f32")
            O[h, i0:i1] = _reduce("SUM", pv, "f32", (1,))[:, 0, :]
            L[h, i0:i1] = _binary("ADD", m, _unary("LOG", ssum, "f32"), "f32")
    return (O if out_dtype == "f32" else _cast(O, "f32", out_dtype)), L


# ---------------------------------------------------------------------------
# the interpreter
# ---------------------------------------------------------------------------

class Interpreter:
    """Evaluates a workload graph node by node.

    ``inputs`` maps each BUFFER slot to a numpy array in storage form
    (bfloat16 as uint16 bit patterns). ``max_elems`` is the largest node the
    interpreter materialises whole; ``slab_elems`` bounds one slab.
    """

    def __init__(self, spec, inputs: dict, max_elems: int = 1 << 28, slab_elems: int = 1 << 24):
        self.spec = spec
        self.inputs = inputs
        self.meta = infer(spec)
        self.max_elems = max_elems
        self.slab_elems = slab_elems
        self.memo: dict[int, np.ndarray] = {}
        self.memo_custom: dict = {}

    def size(self, i: int) -> int:
        return int(np.prod(self.meta[i][0], dtype=np.int64))

    def value(self, i: int) -> np.ndarray:
        """The whole value of node ``i`` (memoised)."""
        if i not in self.memo:
            self.memo[i] = self._eval(i, None, {})
        return self.memo[i]

    def _eval(self, i: int, rows, cache: dict) -> np.ndarray:
        """Node ``i``, or only rows [r0, r1) of its dim 0 when ``rows`` is set."""
        if rows is not None and i in cache:
            return cache[i]
        nd = self.spec.nodes[i]
        op = nd["op"]
        shape, dt = self.meta[i]
        src = nd.get("src", ())

        def arg(j):
            if rows is None:
                return self.value(j)
            return self._eval(j, rows, cache)

        if op == "BUFFER":
            arr = np.asarray(self.inputs[nd["slot"]])
            if tuple(arr.shape) != shape or arr.dtype != STORAGE[dt]:
                raise OracleError(f"input {nd['slot']}: {arr.shape}/{arr.dtype}, expected {shape}/{dt}")
            r = arr
            if rows is not None:
                r = arr[rows[0]:rows[1]]
        elif op == "CONST":
            sh = shape if rows is None else (rows[1] - rows[0],) + tuple(shape[1:])
            if dt == "bf16":
                r = np.full(sh, f32_to_bf16(np.float32(nd["value"]).reshape(1))[0], dtype=np.uint16)
            elif dt in INTS:
                r = np.full(sh, np.int64(int(nd["value"])).astype(STORAGE[dt]), dtype=STORAGE[dt])
            else:
                r = np.full(sh, nd["value"], dtype=STORAGE[dt])
        elif op == "VIEW":
            base = self.value(src[0])
            if nd.get("raw") is not None:
                r = _raw_view(base, nd["raw"])
            else:
                r = base
                for mv in nd["movement"]:
                    r = _apply_movement(r, mv)
            if rows is not None:
                r = r[rows[0]:rows[1]]
        elif op in ("NEG", "EXP", "LOG", "SQRT", "RECIP"):
            r = _unary(op, np.ascontiguousarray(arg(src[0])), dt)
        elif op == "CAST":
            r = _cast(np.ascontiguousarray(arg(src[0])), self.meta[src[0]][1], dt)
        elif op in ("ADD", "MUL", "CMPLT"):
            r = _binary(op, np.ascontiguousarray(arg(src[0])), np.ascontiguousarray(arg(src[1])),
                        self.meta[src[0]][1])
        elif op == "WHERE":
            c = arg(src[0])
            r = np.where(c != 0, arg(src[1]), arg(src[2])).astype(STORAGE[dt])
        elif op in ("SUM", "MAX"):
            axes = tuple(nd["axes"])
            sdt = self.meta[src[0]][1]
            if rows is None and self.size(src[0]) > self.max_elems:
                r = self._reduce_in_slabs(i, op, src[0], sdt, axes)
            else:
                if rows is not None and 0 in axes:
                    raise OracleError("a slab cannot reduce over dim 0")
                r = _reduce(op, np.ascontiguousarray(arg(src[0])), sdt, axes)
        elif op == "CONTIGUOUS":
            r = np.ascontiguousarray(arg(src[0])).copy()
        elif op == "GATHER":
            if rows is not None:
                raise OracleError("GATHER is not evaluated in slabs")
            r = gather(np.asarray(self.value(src[0])), np.asarray(self.value(src[1])), nd["axis"], dt)
        elif op == "SCATTER":
            if rows is not None:
                raise OracleError("SCATTER is not evaluated in slabs")
            r = scatter(np.asarray(self.value(src[0])), np.asarray(self.value(src[1])),
                        np.asarray(self.value(src[2])), nd["axis"], dt)
        elif op == "CUSTOM":
            if rows is not None:
                raise OracleError("a CUSTOM node is not evaluated in slabs")
            key = ("sdpa_fwd", tuple(src), nd["scale"], nd["causal"])
            if key not in self.memo_custom:
                self.memo_custom[key] = {}
            got = self.memo_custom[key]
            if nd["out"] not in got:
                o, lse = sdpa_fwd(np.asarray(self.value(src[0])), np.asarray(self.value(src[1])),
                                  np.asarray(self.value(src[2])), nd["scale"], nd["causal"],
                                  dt if nd["out"] == 0 else "f32")
                got[0] = o if nd["out"] == 0 else got.get(0)
                got[1] = lse
            r = got[nd["out"]]
            if r is None:  # O was asked in another dtype than a sibling's
                r = sdpa_fwd(np.asarray(self.value(src[0])), np.asarray(self.value(src[1])),
                             np.asarray(self.value(src[2])), nd["scale"], nd["causal"], dt)[0]
        else:
            raise OracleError(f"op {op}")
        r = np.ascontiguousarray(r) if op not in ("VIEW", "BUFFER") else r
        if rows is not None:
            cache[i] = r
        return r

    def _reduce_in_slabs(self, i, op, s, sdt, axes):
        if 0 in axes:
            raise OracleError(f"node {i}: too large to materialise and reduces dim 0")
        shape = self.meta[s][0]
        per_row = max(1, self.size(s) // max(1, shape[0]))
        step = max(1, self.slab_elems // per_row)
        parts = []
        for r0 in range(0, shape[0], step):
            r1 = min(shape[0], r0 + step)
            x = self._eval(s, (r0, r1), {})
            parts.append(_reduce(op, np.ascontiguousarray(x), sdt, axes))
        return np.concatenate(parts, axis=0)


def run(spec, inputs: dict, **kw) -> list:
    """Evaluate ``spec`` and return its outputs in storage form."""
    it = Interpreter(spec, inputs, **kw)
    return [np.array(it.value(o), copy=True) for o in spec.outputs]


def dtype_of(spec, node: int) -> str:
    return infer(spec)[node][1]
