"""Seeded synthetic inputs and declarative workload graphs.

This module is shared by the tests, the benchmark and the CPU oracle's
callers. It holds no arithmetic of the method: a graph here is only a record
of which primitive is applied to which earlier node (the limn README,
"Architecture" and "The op set"), with movement ops kept as the list the user
wrote. Shape inference, View composition and every primitive's evaluation are
implemented separately by the library (``reduce_view_amd``) and by the oracle
(``oracle/``); neither imports the other.

Random inputs: ``numpy.random.default_rng(seed)`` (PCG64), drawn in the order
each workload lists them, as float64, rounded to float32 by numpy's cast
(round-to-nearest-even) and, for bfloat16 storage, rounded again by torch's
float32 -> bfloat16 conversion (round-to-nearest-even). ``normal(mu, s)`` takes
``s`` as the standard deviation. bfloat16 arrays are carried as ``uint16``
bit patterns.
"""

from __future__ import annotations

import numpy as np

# Names of the primitive ops a graph may hold (limn README, "The op set").
OPS = (
    "BUFFER", "CONST", "VIEW", "NEG", "EXP", "LOG", "SQRT", "RECIP", "CAST",
    "ADD", "MUL", "CMPLT", "WHERE", "SUM", "MAX", "CONTIGUOUS",
    "GATHER", "SCATTER", "ASSIGN", "CUSTOM",
)
DTYPES = ("f32", "bf16", "f16", "f64", "i32", "i16", "i8")
MOVEMENT = ("reshape", "permute", "expand", "pad", "shrink")


class Spec:
    """A topologically ordered node list plus the ids of its outputs.

    Every node is a plain dict. Keys used:
      op        one of OPS
      src       tuple of earlier node ids
      slot      BUFFER: name of the input array; its shape and dtype
      shape     BUFFER, CONST: shape (tuple)
      dtype     BUFFER, CONST: storage dtype; CAST: target dtype
      value     CONST: the scalar
      axes      SUM, MAX: reduced axes (dims are kept with size 1)
      movement  VIEW: tuple of (name, arg) movement ops applied in order
      raw       VIEW: explicit descriptor dict(shape, strides, offset,
                mask_lo, mask_hi) in elements over the source's row-major
                storage, instead of ``movement``
    """

    def __init__(self, name: str = "graph"):
        self.name = name
        self.nodes: list[dict] = []
        self.outputs: list[int] = []

    # sources -----------------------------------------------------------
    def _add(self, **kw) -> int:
        kw.setdefault("src", ())
        self.nodes.append(kw)
        return len(self.nodes) - 1

    def buffer(self, slot: str, shape, dtype: str) -> int:
        return self._add(op="BUFFER", slot=slot, shape=tuple(shape), dtype=dtype)

    def const(self, value: float, shape, dtype: str) -> int:
        return self._add(op="CONST", value=float(value), shape=tuple(shape), dtype=dtype)

    # movement ----------------------------------------------------------
    def view(self, src: int, *movement) -> int:
        mv = tuple((m[0], _freeze(m[1])) for m in movement)
        for m in mv:
            if m[0] not in MOVEMENT:
                raise ValueError(f"unknown movement op {m[0]!r}")
        return self._add(op="VIEW", src=(src,), movement=mv)

    def raw_view(self, src: int, shape, strides, offset=0, mask_lo=None, mask_hi=None) -> int:
        shape = tuple(int(s) for s in shape)
        raw = dict(shape=shape, strides=tuple(int(s) for s in strides), offset=int(offset),
                   mask_lo=tuple(mask_lo) if mask_lo is not None else tuple(0 for _ in shape),
                   mask_hi=tuple(mask_hi) if mask_hi is not None else shape)
        return self._add(op="VIEW", src=(src,), raw=raw)

    # elementwise -------------------------------------------------------
    def neg(self, x): return self._add(op="NEG", src=(x,))
    def exp(self, x): return self._add(op="EXP", src=(x,))
    def log(self, x): return self._add(op="LOG", src=(x,))
    def sqrt(self, x): return self._add(op="SQRT", src=(x,))
    def recip(self, x): return self._add(op="RECIP", src=(x,))
    def cast(self, x, dtype): return self._add(op="CAST", src=(x,), dtype=dtype)
    def add(self, x, y): return self._add(op="ADD", src=(x, y))
    def mul(self, x, y): return self._add(op="MUL", src=(x, y))
    def cmplt(self, x, y): return self._add(op="CMPLT", src=(x, y))
    def where(self, c, x, y): return self._add(op="WHERE", src=(c, x, y))

    # reduce / barriers -------------------------------------------------
    def sum(self, x, axes): return self._add(op="SUM", src=(x,), axes=tuple(axes))
    def max(self, x, axes): return self._add(op="MAX", src=(x,), axes=tuple(axes))
    def contiguous(self, x): return self._add(op="CONTIGUOUS", src=(x,))

    # indexed (limn README, "The op set": GATHER, SCATTER) -------------
    def gather(self, data, index, axis: int):
        """out[p] = data[p with its ``axis`` coordinate replaced by index[p]]
        (index int32, shaped like data but along ``axis``; an index outside
        [0, data.shape[axis]) reads zero)."""
        return self._add(op="GATHER", src=(data, index), axis=int(axis))

    def scatter(self, base, index, values, axis: int, atomic: bool = False):
        """base with values[p] added at p with its ``axis`` coordinate replaced
        by index[p], for every p of index's shape in ascending row-major
        order (colliding adds in that order; an index outside the axis drops
        its value). ``atomic`` asks the device for unordered atomic adds
        (the same value up to the order of colliding float adds)."""
        return self._add(op="SCATTER", src=(base, index, values), axis=int(axis), atomic=bool(atomic))

    # the one CUSTOM kernel: fused attention forward --------------------
    def sdpa(self, q, k, v, scale: float, causal: bool = False, out_dtype: str = "f32"):
        """Fused attention forward as CUSTOM ``sdpa_fwd`` (limn README, "The op
        set", escape hatch: a kernel a device supplies whole, one node per
        output, the siblings sharing their sources). q (H, Tq, D), k and v
        (H, Tk, D), all bfloat16. Returns the ids of O = softmax(scale * q k^T,
        keys j > query i masked when ``causal``) v, shape (H, Tq, D), and of
        L, the logsumexp of each query row, shape (H, Tq, 1) float32."""
        kw = dict(kind="sdpa_fwd", src=(q, k, v), scale=float(scale), causal=bool(causal))
        o = self._add(op="CUSTOM", out=0, dtype=out_dtype, **kw)
        lse = self._add(op="CUSTOM", out=1, dtype="f32", **kw)
        return o, lse

    def output(self, *ids) -> None:
        self.outputs.extend(ids)


def _freeze(a):
    if isinstance(a, (list, tuple)):
        return tuple(_freeze(x) for x in a)
    return int(a)


# ---------------------------------------------------------------------------
# workload graphs (the composed ops spelled in primitives: x - y is
# ADD(x, NEG(y)), x / y is MUL(x, RECIP(y)), rsqrt is RECIP(SQRT(.)), a mean
# is SUM times CONST(1/N), relu(y) is WHERE(CMPLT(0, y), y, 0)).
# ---------------------------------------------------------------------------

def matmul_broadcast(m: int, n: int, k: int, dtype: str = "f32") -> Spec:
    """Y = SUM_k MUL(A viewed as (m,n,k) with n-stride 0, B viewed as (m,n,k)
    with m-stride 0): the limn README's one-nest matmul and the Luminal IR
    blog's naive matmul with a stride-0 loop."""
    g = Spec(f"matmul_broadcast_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), dtype)
    b = g.buffer("B", (k, n), dtype)
    a3 = g.view(a, ("reshape", (m, 1, k)), ("expand", (m, n, k)))
    b3 = g.view(b, ("permute", (1, 0)), ("reshape", (1, n, k)), ("expand", (m, n, k)))
    y = g.sum(g.mul(a3, b3), (2,))
    g.output(y)
    return g


def matmul_broadcast_raw(m: int, n: int, k: int) -> Spec:
    """The same contraction with the two Views written as explicit
    descriptors: A with strides (k, 0, 1), B with strides (0, 1, n)."""
    g = Spec(f"matmul_raw_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), "f32")
    b = g.buffer("B", (k, n), "f32")
    a3 = g.raw_view(a, (m, n, k), (k, 0, 1))
    b3 = g.raw_view(b, (m, n, k), (0, 1, n))
    g.output(g.sum(g.mul(a3, b3), (2,)))
    return g


def ew_chain(rows: int, cols: int, masked: bool = False, edges=(3, 5)) -> Spec:
    """out = WHERE(CMPLT(a, b), a*b, EXP(-a)) + c, with b a permuted view of
    a (cols, rows) buffer and c a row vector expanded down the rows through a
    stride-0 dim. With ``masked`` the operand a is a shrink-then-pad view of a
    larger buffer whose border of ``edges`` rows/cols reads as zero."""
    g = Spec(f"ew_chain_{rows}x{cols}{'_masked' if masked else ''}")
    if masked:
        er, ec = edges
        big = g.buffer("Abig", (rows, cols), "f32")
        a = g.view(big, ("shrink", ((er, rows - er), (ec, cols - ec))),
                   ("pad", ((er, er), (ec, ec))))
    else:
        a = g.buffer("a", (rows, cols), "f32")
    bb = g.buffer("Bb", (cols, rows), "f32")
    b = g.view(bb, ("permute", (1, 0)))
    cv = g.buffer("c", (cols,), "f32")
    c = g.view(cv, ("reshape", (1, cols)), ("expand", (rows, cols)))
    out = g.add(g.where(g.cmplt(a, b), g.mul(a, b), g.exp(g.neg(a))), c)
    g.output(out)
    return g


def transpose(rows: int, cols: int, dtype: str = "f32") -> Spec:
    """Y = CONTIGUOUS(VIEW(X, permute(1, 0))): X is (rows, cols), Y (cols, rows)."""
    g = Spec(f"transpose_{rows}x{cols}")
    x = g.buffer("X", (rows, cols), dtype)
    g.output(g.contiguous(g.view(x, ("permute", (1, 0)))))
    return g


def softmax(rows: int, n: int) -> Spec:
    """Row softmax with the max shift: m = MAX(x), e = EXP(x - m),
    y = e * RECIP(SUM(e))."""
    g = Spec(f"softmax_{rows}x{n}")
    x = g.buffer("x", (rows, n), "f32")
    m = g.max(x, (1,))
    mb = g.view(m, ("expand", (rows, n)))
    e = g.exp(g.add(x, g.neg(mb)))
    s = g.sum(e, (1,))
    rb = g.view(g.recip(s), ("expand", (rows, n)))
    g.output(g.mul(e, rb))
    return g


def softmax_noshift(rows: int, n: int) -> Spec:
    """Softmax written without the max shift (the Litmus README's
    no_max_subtract family): overflows for large-magnitude rows."""
    g = Spec(f"softmax_noshift_{rows}x{n}")
    x = g.buffer("x", (rows, n), "f32")
    e = g.exp(x)
    s = g.sum(e, (1,))
    g.output(g.mul(e, g.view(g.recip(s), ("expand", (rows, n)))))
    return g


def rmsnorm(rows: int, n: int, eps: float = 1e-6, dtype: str = "f32") -> Spec:
    """y = (x * r) * w, r = RECIP(SQRT(SUM(x*x) * (1/n) + eps)) (Tiki README,
    "Compile model code": float32 reduction, multiplication order x*inv*w).
    Every value in ``dtype`` (f16: each primitive computes in float32 and
    rounds back, the SUM keeps a float32 total; f64 throughout)."""
    g = Spec(f"rmsnorm_{rows}x{n}" + ("" if dtype == "f32" else f"_{dtype}"))
    x = g.buffer("x", (rows, n), dtype)
    w = g.buffer("w", (n,), dtype)
    ss = g.sum(g.mul(x, x), (1,))
    ms = g.mul(ss, g.const(1.0 / n, (rows, 1), dtype))
    r = g.recip(g.sqrt(g.add(ms, g.const(eps, (rows, 1), dtype))))
    rb = g.view(r, ("expand", (rows, n)))
    wb = g.view(w, ("reshape", (1, n)), ("expand", (rows, n)))
    g.output(g.mul(g.mul(x, rb), wb))
    return g


def layernorm(rows: int, n: int, eps: float = 1e-5, dtype: str = "bf16") -> Spec:
    """torch-semantics LayerNorm (biased variance) with ``dtype`` storage and
    float32 arithmetic: xf = CAST(x), mu = SUM(xf)/n, xc = xf - mu,
    v = SUM(xc*xc)/n, r = RECIP(SQRT(v + eps)), y = CAST((xc*r)*g + b)."""
    g = Spec(f"layernorm_{rows}x{n}")
    x = g.buffer("x", (rows, n), dtype)
    gm = g.buffer("gamma", (n,), dtype)
    bt = g.buffer("beta", (n,), dtype)
    xf = g.cast(x, "f32")
    inv_n = g.const(1.0 / n, (rows, 1), "f32")
    mu = g.mul(g.sum(xf, (1,)), inv_n)
    xc = g.add(xf, g.neg(g.view(mu, ("expand", (rows, n)))))
    v = g.mul(g.sum(g.mul(xc, xc), (1,)), inv_n)
    r = g.recip(g.sqrt(g.add(v, g.const(eps, (rows, 1), "f32"))))
    gf = g.view(g.cast(gm, "f32"), ("reshape", (1, n)), ("expand", (rows, n)))
    bf = g.view(g.cast(bt, "f32"), ("reshape", (1, n)), ("expand", (rows, n)))
    y = g.add(g.mul(g.mul(xc, g.view(r, ("expand", (rows, n)))), gf), bf)
    g.output(g.cast(y, dtype))
    return g


def gemm_relu2_sum(m: int, n: int, k: int, emit_y: bool = False) -> Spec:
    """S = SUM(relu(y)^2) with y = SUM_k CAST(A) * CAST(B) over bf16 A (m,k)
    and B (k,n) viewed as (m,n,k) through stride-0 dims (limn README's
    headline example ((x @ W).relu() ** 2).sum(), in primitives)."""
    g = Spec(f"gemm_relu2_sum_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), "bf16")
    b = g.buffer("B", (k, n), "bf16")
    a3 = g.cast(g.view(a, ("reshape", (m, 1, k)), ("expand", (m, n, k))), "f32")
    b3 = g.cast(g.view(b, ("permute", (1, 0)), ("reshape", (1, n, k)), ("expand", (m, n, k))), "f32")
    y = g.sum(g.mul(a3, b3), (2,))
    zero = g.const(0.0, (m, n, 1), "f32")
    r = g.where(g.cmplt(zero, y), y, zero)
    s = g.sum(g.mul(r, r), (0, 1, 2))
    g.output(s)
    if emit_y:
        g.output(y)
    return g


def gemm_bf16(m: int, n: int, k: int) -> Spec:
    """y = SUM_k CAST(A) * CAST(B), stored as float32 (m, n, 1)."""
    g = Spec(f"gemm_bf16_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), "bf16")
    b = g.buffer("B", (k, n), "bf16")
    a3 = g.cast(g.view(a, ("reshape", (m, 1, k)), ("expand", (m, n, k))), "f32")
    b3 = g.cast(g.view(b, ("permute", (1, 0)), ("reshape", (1, n, k)), ("expand", (m, n, k))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    return g


# ---------------------------------------------------------------------------
# seeded inputs
# ---------------------------------------------------------------------------

def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns by torch's conversion (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def inputs_matmul(m: int, n: int, k: int, seed: int = 0) -> dict:
    rng = np.random.default_rng(seed)
    return {"A": _f32(rng.normal(0.0, 1.0, (m, k))), "B": _f32(rng.normal(0.0, 1.0, (k, n)))}


def inputs_ew(rows: int, cols: int, seed: int = 1) -> dict:
    """Draw order: a, Bb, c, Abig, then the transpose input X."""
    rng = np.random.default_rng(seed)
    d = {}
    d["a"] = _f32(rng.uniform(-4.0, 4.0, (rows, cols)))
    d["Bb"] = _f32(rng.uniform(-4.0, 4.0, (cols, rows)))
    d["c"] = _f32(rng.uniform(-4.0, 4.0, (cols,)))
    d["Abig"] = _f32(rng.uniform(-4.0, 4.0, (rows, cols)))
    d["X"] = _f32(rng.uniform(-1.0, 1.0, (rows, cols)))
    return d


def inputs_softmax(rows: int, n: int, seed: int = 2) -> dict:
    rng = np.random.default_rng(seed)
    return {"x": _f32(rng.uniform(-1e3, 1e3, (rows, n)))}


def inputs_rmsnorm(rows: int, n: int, seed: int = 3, dtype: str = "f32") -> dict:
    """x ~ N(0, 1) then w ~ N(1, 0.1), float64 draws rounded once (RNE) to
    ``dtype`` (f32, f16 or f64)."""
    rng = np.random.default_rng(seed)
    to = {"f32": np.float32, "f16": np.float16, "f64": np.float64}[dtype]
    x = rng.normal(0.0, 1.0, (rows, n)).astype(to)
    w = rng.normal(1.0, 0.1, (n,)).astype(to)
    return {"x": x, "w": w}


def chain_int(rows: int, cols: int, dtype: str = "i8") -> Spec:
    """y = a * b + c in an int dtype (wraps modulo 2^width, limn README, "The
    op set")."""
    g = Spec(f"chain_{dtype}_{rows}x{cols}")
    a = g.buffer("a", (rows, cols), dtype)
    b = g.buffer("b", (rows, cols), dtype)
    c = g.buffer("c", (rows, cols), dtype)
    y = g.add(g.mul(a, b), c)
    g.output(y)
    return g


def inputs_chain_int(rows: int, cols: int, dtype: str = "i8", seed: int = 8) -> dict:
    """a, b, c uniform over the whole range of ``dtype``, in that order."""
    rng = np.random.default_rng(seed)
    info = np.iinfo({"i8": np.int8, "i16": np.int16, "i32": np.int32}[dtype])
    mk = lambda: rng.integers(info.min, info.max + 1, (rows, cols), dtype=np.int64).astype(info.dtype)  # noqa: E731
    return {"a": mk(), "b": mk(), "c": mk()}


def inputs_layernorm(rows: int, n: int, seed: int = 4) -> dict:
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(_f32(rng.normal(100.0, 1.0, (rows, n))))
    gm = to_bf16_bits(_f32(rng.normal(1.0, 0.1, (n,))))
    bt = to_bf16_bits(_f32(rng.normal(0.0, 0.1, (n,))))
    return {"x": x, "gamma": gm, "beta": bt}


def inputs_gemm(m: int, n: int, k: int, seed: int = 5) -> dict:
    rng = np.random.default_rng(seed)
    a = to_bf16_bits(_f32(rng.normal(0.0, 1.0 / np.sqrt(k), (m, k))))
    b = to_bf16_bits(_f32(rng.normal(0.0, 1.0, (k, n))))
    return {"A": a, "B": b}


def inputs_gemm_integer(m: int, n: int, k: int, seed: int = 7, lo: int = -2, hi: int = 2) -> dict:
    """Integer-valued bf16 operands in [lo, hi]: every partial sum is an
    integer below 2^24, so any summation order gives the same float32."""
    rng = np.random.default_rng(seed)
    a = to_bf16_bits(rng.integers(lo, hi + 1, (m, k)).astype(np.float32))
    b = to_bf16_bits(rng.integers(lo, hi + 1, (k, n)).astype(np.float32))
    return {"A": a, "B": b}


# Full-size workloads the measurements are quoted on (shape, seed).
FULL = {
    "matmul64": dict(m=64, n=64, k=64),
    "ew_chain": dict(rows=4096, cols=4096),
    "softmax": dict(rows=16384, n=4096),
    "rmsnorm": dict(rows=16384, n=4096),
    "layernorm": dict(rows=8192, n=8192),
    "gemm": dict(m=4096, n=4096, k=4096),
}


def copy(rows: int, cols: int) -> Spec:
    """out = CONTIGUOUS(x): a plain copy, the bandwidth reference."""
    g = Spec(f"copy_{rows}x{cols}")
    x = g.buffer("X", (rows, cols), "f32")
    g.output(g.contiguous(x))
    return g


def attention(h: int, tq: int, tk: int, d: int, causal: bool = True, out_dtype: str = "f32",
              outputs: str = "ol") -> Spec:
    """Fused attention forward over bfloat16 q (h, tq, d), k, v (h, tk, d),
    scale 1/sqrt(d): outputs O (and L when ``outputs`` has an 'l')."""
    g = Spec(f"attention_{h}x{tq}x{tk}x{d}{'_causal' if causal else ''}")
    q = g.buffer("Q", (h, tq, d), "bf16")
    k = g.buffer("K", (h, tk, d), "bf16")
    v = g.buffer("V", (h, tk, d), "bf16")
    o, lse = g.sdpa(q, k, v, 1.0 / float(np.sqrt(d)), causal, out_dtype)
    g.output(*([o] if "o" in outputs else []), *([lse] if "l" in outputs else []))
    return g


def inputs_attention(h: int, tq: int, tk: int, d: int, seed: int = 6) -> dict:
    """Q, K, V ~ N(0, 1) drawn in that order, rounded to bfloat16."""
    rng = np.random.default_rng(seed)
    return {"Q": to_bf16_bits(_f32(rng.standard_normal((h, tq, d)))),
            "K": to_bf16_bits(_f32(rng.standard_normal((h, tk, d)))),
            "V": to_bf16_bits(_f32(rng.standard_normal((h, tk, d))))}


def embedding_gather(vocab: int, dim: int, n: int, dtype: str = "f32") -> Spec:
    """Rows of a (vocab, dim) table picked by n int32 ids: GATHER along axis 0
    with the ids broadcast across the row (an (n, 1) id column expanded to
    (n, dim))."""
    g = Spec(f"embedding_gather_{vocab}x{dim}_{n}")
    table = g.buffer("table", (vocab, dim), dtype)
    ids = g.buffer("ids", (n, 1), "i32")
    g.output(g.gather(table, g.view(ids, ("expand", (n, dim))), 0))
    return g


def embedding_scatter(vocab: int, dim: int, n: int, dtype: str = "f32", atomic: bool = False) -> Spec:
    """The gather's transpose: n rows of values added into a zero (vocab, dim)
    table at rows given by n int32 ids (repeated ids add up, in order)."""
    g = Spec(f"embedding_scatter_{vocab}x{dim}_{n}" + ("_atomic" if atomic else ""))
    vals = g.buffer("values", (n, dim), dtype)
    ids = g.buffer("ids", (n, 1), "i32")
    zero = g.const(0.0, (vocab, dim), dtype)
    g.output(g.scatter(zero, g.view(ids, ("expand", (n, dim))), vals, 0, atomic))
    return g


def inputs_embedding(vocab: int, dim: int, n: int, seed: int = 9, dtype: str = "f32") -> dict:
    """table ~ N(0, 1) (vocab, dim), ids uniform in [0, vocab) (n, 1), values
    ~ N(0, 1) (n, dim), drawn in that order."""
    rng = np.random.default_rng(seed)
    to = {"f32": np.float32, "f16": np.float16, "f64": np.float64}[dtype]
    table = rng.standard_normal((vocab, dim)).astype(to)
    ids = rng.integers(0, vocab, (n, 1)).astype(np.int32)
    values = rng.standard_normal((n, dim)).astype(to)
    return {"table": table, "ids": ids, "values": values}


def unary_map(op: str, n: int, dtype: str = "f32") -> Spec:
    """y = OP(x) over a flat (n,) buffer (one of NEG, EXP, LOG, SQRT, RECIP)."""
    if op not in ("NEG", "EXP", "LOG", "SQRT", "RECIP"):
        raise ValueError(op)
    g = Spec(f"{op.lower()}_{n}")
    x = g.buffer("x", (n,), dtype)
    g.output(g._add(op=op, src=(x,)))
    return g


def fp32_sweep(lo_bits: int, hi_bits: int, step: int = 1) -> np.ndarray:
    """Every ``step``-th float32 whose bit pattern lies in [lo_bits, hi_bits)
    (unsigned order: 0x00000000.. are +0 upward, 0x80000000.. are -0
    downward), as a float32 array. No randomness."""
    return np.arange(lo_bits, hi_bits, step, dtype=np.uint32).view(np.float32)


def gemm_bf16_bt(m: int, n: int, k: int) -> Spec:
    """y = SUM_k CAST(A) * CAST(Bt) with the second operand stored [n][k]
    (k-contiguous), viewed as (m, n, k) with m-stride 0."""
    g = Spec(f"gemm_bf16_bt_{m}x{n}x{k}")
    a = g.buffer("A", (m, k), "bf16")
    bt = g.buffer("Bt", (n, k), "bf16")
    a3 = g.cast(g.view(a, ("reshape", (m, 1, k)), ("expand", (m, n, k))), "f32")
    b3 = g.cast(g.view(bt, ("reshape", (1, n, k)), ("expand", (m, n, k))), "f32")
    g.output(g.sum(g.mul(a3, b3), (2,)))
    return g


def cast_matrix(n: int) -> Spec:
    """Every CAST between the seven dtypes: one (n,) input ``x_<src>`` per
    dtype and 49 outputs CAST(x_src, dst), source-major in ``DTYPES`` order
    (a CAST to the source's own dtype is a copy)."""
    g = Spec(f"cast_matrix_{n}")
    xs = {dt: g.buffer(f"x_{dt}", (n,), dt) for dt in DTYPES}
    for src in DTYPES:
        for dst in DTYPES:
            g.output(g.cast(xs[src], dst))
    return g


# Values a CAST must get right at the edges: halfway cases of every float
# width, overflow to infinity, subnormals, float64 values that round twice on
# their way to a half width, truncation toward zero and wraparound of ints.
CAST_FLOAT_WITNESSES = (
    0.0, -0.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 2.9999, -2.9999, 127.9, 128.0, -128.0, -129.5, 255.5,
    300.0, -300.7, 32767.5, 32768.0, -32769.9, 40000.0, 65504.0, 65519.99, 65520.0, 1e5, 16777217.0,
    2147483520.0, -2147483648.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -11, 1 + 3 * 2 ** -11,
    1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -11 + 2 ** -40, 1 + 2 ** -24, 1 + 2 ** -24 + 2 ** -50, 2 ** -24,
    2 ** -25, 1.5 * 2 ** -25, 2 ** -14, 2 ** -126, 2 ** -133, 2 ** -149, 2 ** -150, 3.0e38, 3.389e38,
    3.4e38, 3.5e38, 1e300, -1e300, 1e-300, float("inf"), float("-inf"), float("nan"), 0.1, 1 / 3,
)
CAST_INT_WITNESSES = (
    0, 1, -1, 127, 128, -128, -129, 255, 256, 300, 2049, 2051, 32767, 32768, -32768, -32769, 40000,
    65504, 65519, 65520, 65535, 16777217, 16777219, 2 ** 24 + 2 ** 16 + 1, 2 ** 31 - 1, -2 ** 31,
    2 ** 31 - 64, 123456789, -987654321,
)
_INT_RANGE = {"i32": (-2 ** 31, 2 ** 31 - 1), "i16": (-2 ** 15, 2 ** 15 - 1), "i8": (-128, 127)}


def inputs_cast(n: int = 1024, seed: int = 10) -> dict:
    """``x_<dt>`` for every dtype: the witnesses above that the dtype holds
    (floats rounded into it by numpy's or torch's RNE cast, ints in range),
    then seeded fill: for the float widths half uniformly random bit
    patterns (every class: NaN, infinities, subnormals) and half
    N(0, 1) * 10^U(-3, 6); for the ints uniform over the whole range.
    Draw order: the dtypes in ``DTYPES`` order."""
    rng = np.random.default_rng(seed)
    out = {}
    fw = np.array(CAST_FLOAT_WITNESSES, dtype=np.float64)
    for dt in DTYPES:
        if dt in _INT_RANGE:
            lo, hi = _INT_RANGE[dt]
            w = np.array([v for v in CAST_INT_WITNESSES if lo <= v <= hi], dtype=np.int64)
            fill = rng.integers(lo, hi, size=n, endpoint=True, dtype=np.int64)
            store = {"i32": np.int32, "i16": np.int16, "i8": np.int8}[dt]
            out[f"x_{dt}"] = np.concatenate([w, fill])[:n].astype(store)
            continue
        nb = {"f64": 64, "f32": 32, "f16": 16, "bf16": 16}[dt]
        half = n // 2
        bits = rng.integers(0, 2 ** nb if nb < 64 else 2 ** 63, size=half, dtype=np.uint64)
        if nb == 64:
            bits = bits | (rng.integers(0, 2, size=half, dtype=np.uint64) << np.uint64(63))
        mags = rng.standard_normal(n - half) * 10.0 ** rng.uniform(-3.0, 6.0, n - half)
        with np.errstate(over="ignore", invalid="ignore"):
            if dt == "f64":
                vals = np.concatenate([fw, bits.view(np.float64), mags])
                out[f"x_{dt}"] = vals[:n].astype(np.float64)
            elif dt == "f32":
                vals = np.concatenate([fw.astype(np.float32), bits.astype(np.uint32).view(np.float32),
                                       mags.astype(np.float32)])
                out[f"x_{dt}"] = vals[:n]
            elif dt == "f16":
                vals = np.concatenate([fw.astype(np.float16), bits.astype(np.uint16).view(np.float16),
                                       mags.astype(np.float16)])
                out[f"x_{dt}"] = vals[:n]
            else:
                wb = to_bf16_bits(fw.astype(np.float32))
                mb = to_bf16_bits(mags.astype(np.float32))
                out[f"x_{dt}"] = np.concatenate([wb, bits.astype(np.uint16), mb])[:n]
    return out


def reduce(shape, axes, op: str = "SUM", dtype: str = "f32", permute=None, pad=None) -> Spec:
    """y = SUM or MAX of x over ``axes`` (kept with size 1). ``permute`` and
    ``pad`` (per-dim (before, after)) first view x through those movements,
    in that order."""
    g = Spec(f"{op.lower()}_{'x'.join(map(str, shape))}_{''.join(map(str, axes))}")
    x = g.buffer("x", tuple(shape), dtype)
    mv = []
    if permute is not None:
        mv.append(("permute", tuple(permute)))
    if pad is not None:
        mv.append(("pad", tuple(tuple(p) for p in pad)))
    v = g.view(x, *mv) if mv else x
    g.output(g.sum(v, axes) if op == "SUM" else g.max(v, axes))
    return g


def mean_rows(rows: int, n: int) -> Spec:
    """Row means SUM(x) * (1/n) of a (rows, n) float32 x."""
    g = Spec(f"mean_rows_{rows}x{n}")
    x = g.buffer("x", (rows, n), "f32")
    g.output(g.mul(g.sum(x, (1,)), g.const(1.0 / n, (rows, 1), "f32")))
    return g


def inputs_reduce(shape, dtype: str = "f32", seed: int = 11, dist: str = "normal") -> dict:
    """x of ``shape``: floats N(0, 1) (``dist="normal"``) or U(-1, 1)
    (``"uniform"``), drawn in float64 and rounded once into the dtype
    (bfloat16 through float32); ints uniform over the whole range."""
    rng = np.random.default_rng(seed)
    shape = tuple(shape)
    if dtype in ("i32", "i16", "i8"):
        lo, hi = _INT_RANGE[dtype]
        store = {"i32": np.int32, "i16": np.int16, "i8": np.int8}[dtype]
        return {"x": rng.integers(lo, hi, size=shape, endpoint=True, dtype=np.int64).astype(store)}
    x = rng.standard_normal(shape) if dist == "normal" else rng.uniform(-1.0, 1.0, shape)
    if dtype == "f64":
        return {"x": x}
    if dtype == "f16":
        return {"x": x.astype(np.float16)}
    x32 = _f32(x)
    return {"x": to_bf16_bits(x32) if dtype == "bf16" else x32}
