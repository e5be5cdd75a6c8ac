"""Python binding of the reduce_view C ABI (include/rv.h).

Argument marshalling only: every call goes to the compiled library
(``_lib/librv.so``), which does the graph intake, View algebra, scheduling,
lowering, code generation and launches. torch is used for device memory and
streams. The binding raises ``RVError`` (carrying the rv_status and the
library's message) on every failing call, and importing it fails loudly when
the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "librv.so")

RV_MAX_DIMS = 8
RV_SCRATCH_BYTES = 64 << 20  # the library's own workspace per GPU (rv_launch_noalloc)
STATUS = {0: "RV_OK", -1: "RV_E_INVALID", -2: "RV_E_UNSUPPORTED_OP", -3: "RV_E_UNSUPPORTED_LAYOUT",
          -4: "RV_E_DTYPE", -5: "RV_E_OUT_OF_BOUNDS", -6: "RV_E_WORKSPACE", -7: "RV_E_DEVICE",
          -8: "RV_E_COMPILE", -9: "RV_E_LAUNCH"}
DTYPE = {"f32": 0, "bf16": 1, "f16": 2, "f64": 3, "i32": 4, "i16": 5, "i8": 6}
DTYPE_NAME = {v: k for k, v in DTYPE.items()}
OP = {n: i for i, n in enumerate((
    "BUFFER", "CONST", "VIEW", "NEG", "EXP", "LOG", "SQRT", "RECIP", "CAST", "ADD", "MUL", "CMPLT",
    "WHERE", "SUM", "MAX", "CONTIGUOUS", "GATHER", "SCATTER", "ASSIGN", "CUSTOM"))}


class RVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class rv_view(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("shape", ctypes.c_int64 * RV_MAX_DIMS), ("strides", ctypes.c_int64 * RV_MAX_DIMS),
                ("offset", ctypes.c_int64), ("mask_lo", ctypes.c_int64 * RV_MAX_DIMS),
                ("mask_hi", ctypes.c_int64 * RV_MAX_DIMS)]

    def to_dict(self) -> dict:
        n = self.ndim
        return dict(shape=tuple(self.shape[:n]), strides=tuple(self.strides[:n]), offset=self.offset,
                    mask_lo=tuple(self.mask_lo[:n]), mask_hi=tuple(self.mask_hi[:n]))


class rv_node(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("dtype", ctypes.c_int32), ("src", ctypes.c_int32 * 3),
                ("buf", ctypes.c_int32), ("reduce_axes", ctypes.c_uint32), ("reserved", ctypes.c_int32),
                ("cval", ctypes.c_double), ("view", rv_view)]


class rv_buffer(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("nelems", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python reduce_view_amd/build.py)")
    # One HIP runtime per process: torch ships its own libamdhip64 (same
    # SONAME as the system one the library names), so torch goes first and
    # the library binds to the runtime torch's tensors and streams live in.
    # Loaded the other way round, the process holds two runtimes and the
    # library's sees no device.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    sig = {
        "rv_init": [ctypes.c_int],
        "rv_compile": [P(rv_node), ctypes.c_int32, P(ctypes.c_int32), ctypes.c_int32, P(vp)],
        "rv_node_shape": [P(rv_node), ctypes.c_int32, ctypes.c_int32, P(rv_view), P(ctypes.c_int32)],
        "rv_program_io": [vp, P(ctypes.c_int32), P(ctypes.c_int32)],
        "rv_output_desc": [vp, ctypes.c_int32, P(rv_view), P(ctypes.c_int32)],
        "rv_workspace_size": [vp, P(ctypes.c_size_t)],
        "rv_launch": [vp, P(rv_buffer), ctypes.c_int32, vp, ctypes.c_size_t, vp],
        "rv_launch_noalloc": [vp, P(rv_buffer), ctypes.c_int32, vp],
        "rv_describe": [vp, ctypes.c_char_p, ctypes.c_size_t, P(ctypes.c_size_t)],
        "rv_source": [vp, ctypes.c_char_p, ctypes.c_size_t, P(ctypes.c_size_t)],
        "rv_view_contiguous": [P(ctypes.c_int64), ctypes.c_int32, P(rv_view)],
        "rv_view_reshape": [P(rv_view), P(ctypes.c_int64), ctypes.c_int32, P(rv_view)],
        "rv_view_permute": [P(rv_view), P(ctypes.c_int32), P(rv_view)],
        "rv_view_expand": [P(rv_view), P(ctypes.c_int64), P(rv_view)],
        "rv_view_pad": [P(rv_view), P(ctypes.c_int64), P(ctypes.c_int64), P(rv_view)],
        "rv_view_shrink": [P(rv_view), P(ctypes.c_int64), P(ctypes.c_int64), P(rv_view)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.rv_program_free.argtypes = [vp]
    lib.rv_program_free.restype = None
    lib.rv_last_error.argtypes = []
    lib.rv_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()

# every symbol include/rv.h declares
EXPORTS = ("rv_init", "rv_compile", "rv_node_shape", "rv_program_io", "rv_output_desc",
           "rv_workspace_size", "rv_launch", "rv_launch_noalloc", "rv_describe", "rv_source", "rv_program_free",
           "rv_last_error", "rv_view_contiguous", "rv_view_reshape", "rv_view_permute",
           "rv_view_expand", "rv_view_pad", "rv_view_shrink")


def _check(status: int) -> None:
    if status != 0:
        raise RVError(status, _lib.rv_last_error().decode())


def _i64(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_int64 * max(1, len(xs)))(*xs)


# ---- the C calls, same names ----------------------------------------------

def rv_init(device: int = 0) -> None:
    _check(_lib.rv_init(device))


def rv_view_contiguous(shape) -> rv_view:
    out = rv_view()
    _check(_lib.rv_view_contiguous(_i64(shape), len(shape), ctypes.byref(out)))
    return out


def rv_view_reshape(v: rv_view, shape) -> rv_view:
    out = rv_view()
    _check(_lib.rv_view_reshape(ctypes.byref(v), _i64(shape), len(shape), ctypes.byref(out)))
    return out


def rv_view_permute(v: rv_view, perm) -> rv_view:
    out = rv_view()
    p = (ctypes.c_int32 * max(1, len(perm)))(*[int(x) for x in perm])
    _check(_lib.rv_view_permute(ctypes.byref(v), p, ctypes.byref(out)))
    return out


def rv_view_expand(v: rv_view, shape) -> rv_view:
    out = rv_view()
    _check(_lib.rv_view_expand(ctypes.byref(v), _i64(shape), ctypes.byref(out)))
    return out


def rv_view_pad(v: rv_view, before, after) -> rv_view:
    out = rv_view()
    _check(_lib.rv_view_pad(ctypes.byref(v), _i64(before), _i64(after), ctypes.byref(out)))
    return out


def rv_view_shrink(v: rv_view, lo, hi) -> rv_view:
    out = rv_view()
    _check(_lib.rv_view_shrink(ctypes.byref(v), _i64(lo), _i64(hi), ctypes.byref(out)))
    return out


def rv_node_shape(nodes, i: int):
    v = rv_view()
    dt = ctypes.c_int32()
    _check(_lib.rv_node_shape(nodes, len(nodes), i, ctypes.byref(v), ctypes.byref(dt)))
    return tuple(v.shape[:v.ndim]), DTYPE_NAME[dt.value]


def rv_compile(nodes, outputs) -> "Program":
    outs = (ctypes.c_int32 * len(outputs))(*outputs)
    h = ctypes.c_void_p()
    _check(_lib.rv_compile(nodes, len(nodes), outs, len(outputs), ctypes.byref(h)))
    return Program(h)


def rv_program_io(h):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.rv_program_io(h, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def rv_output_desc(h, i: int):
    v = rv_view()
    dt = ctypes.c_int32()
    _check(_lib.rv_output_desc(h, i, ctypes.byref(v), ctypes.byref(dt)))
    return tuple(v.shape[:v.ndim]), DTYPE_NAME[dt.value]


def rv_workspace_size(h) -> int:
    n = ctypes.c_size_t()
    _check(_lib.rv_workspace_size(h, ctypes.byref(n)))
    return n.value


def rv_launch(h, bufs, workspace_ptr: int, ws_bytes: int, stream_ptr: int) -> None:
    arr = (rv_buffer * max(1, len(bufs)))(*bufs)
    _check(_lib.rv_launch(h, arr, len(bufs), ctypes.c_void_p(workspace_ptr or None), ws_bytes,
                          ctypes.c_void_p(stream_ptr or None)))


def rv_launch_noalloc(h, bufs, stream_ptr: int) -> None:
    """rv_launch with the library's own workspace (for callers that cannot
    allocate)."""
    arr = (rv_buffer * max(1, len(bufs)))(*bufs)
    _check(_lib.rv_launch_noalloc(h, arr, len(bufs), ctypes.c_void_p(stream_ptr or None)))


def _text(fn, h) -> str:
    need = ctypes.c_size_t()
    _check(fn(h, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check(fn(h, buf, need.value, None))
    return buf.value.decode()


def rv_describe(h) -> str:
    return _text(_lib.rv_describe, h)


def rv_source(h) -> str:
    return _text(_lib.rv_source, h)


def rv_program_free(h) -> None:
    _lib.rv_program_free(h)


def rv_last_error() -> str:
    return _lib.rv_last_error().decode()


# ---- marshalling a declarative graph (reduce_view_amd.synth.Spec) ----------

def _blank_view() -> rv_view:
    return rv_view()


# CUSTOM kernel ids and flags (include/rv.h)
CUSTOM_SDPA_FWD = 1
SCATTER_ORDERED, SCATTER_ATOMIC = 0, 1
SDPA_CAUSAL = 1


def nodes_from_spec(spec):
    """rv_node array and slot names for a ``synth.Spec``. Movement ops are
    composed by the library's own rv_view_* calls; shapes of computed
    sources come from rv_node_shape."""
    n = len(spec.nodes)
    arr = (rv_node * n)()
    slots: list[str] = []
    for i, nd in enumerate(spec.nodes):
        x = arr[i]
        x.op = OP[nd["op"]]
        x.src[:] = [-1, -1, -1]
        for k, s in enumerate(nd.get("src", ())):
            x.src[k] = s
        op = nd["op"]
        if op == "BUFFER":
            if nd["slot"] not in slots:
                slots.append(nd["slot"])
            x.buf = slots.index(nd["slot"])
            x.dtype = DTYPE[nd["dtype"]]
            x.view = rv_view_contiguous(nd["shape"])
        elif op == "CONST":
            x.dtype = DTYPE[nd["dtype"]]
            x.cval = nd["value"]
            x.view = rv_view_contiguous(nd["shape"])
        elif op == "CAST":
            x.dtype = DTYPE[nd["dtype"]]
        elif op in ("SUM", "MAX"):
            mask = 0
            for a in nd["axes"]:
                mask |= 1 << a
            x.reduce_axes = mask
        elif op == "VIEW":
            src_shape, _ = rv_node_shape(arr, nd["src"][0])
            if nd.get("raw") is not None:
                r = nd["raw"]
                v = rv_view()
                v.ndim = len(r["shape"])
                for d in range(v.ndim):
                    v.shape[d] = r["shape"][d]
                    v.strides[d] = r["strides"][d]
                    v.mask_lo[d] = r["mask_lo"][d]
                    v.mask_hi[d] = r["mask_hi"][d]
                v.offset = r["offset"]
            else:
                def moved(v):
                    for name, a in nd["movement"]:
                        if name == "reshape":
                            v = rv_view_reshape(v, a)
                        elif name == "permute":
                            v = rv_view_permute(v, a)
                        elif name == "expand":
                            v = rv_view_expand(v, a)
                        elif name == "pad":
                            v = rv_view_pad(v, [w[0] for w in a], [w[1] for w in a])
                        elif name == "shrink":
                            v = rv_view_shrink(v, [w[0] for w in a], [w[1] for w in a])
                    return v
                v = None
                s0 = nd["src"][0]
                if arr[s0].op == OP["VIEW"]:
                    # a View of a View: the movements applied to the inner
                    # View give one View of the inner's source, when they
                    # compose (else the inner value stays a node of its own)
                    try:
                        v = moved(rv_view.from_buffer_copy(arr[s0].view))
                        x.src[0] = arr[s0].src[0]
                    except RVError as e:
                        if e.name != "RV_E_UNSUPPORTED_LAYOUT":
                            raise
                        v = None
                if v is None:
                    v = moved(rv_view_contiguous(src_shape))
            x.view = v
        elif op in ("GATHER", "SCATTER"):
            x.reduce_axes = 1 << int(nd["axis"])
            x.buf = SCATTER_ATOMIC if nd.get("atomic") else SCATTER_ORDERED
        elif op == "CUSTOM":
            if nd.get("kind") != "sdpa_fwd":
                raise RVError(-2, f"CUSTOM kernel {nd.get('kind')!r} is not supported")
            x.buf = CUSTOM_SDPA_FWD
            x.dtype = DTYPE[nd["dtype"]]
            x.cval = nd["scale"]
            x.reduce_axes = (SDPA_CAUSAL if nd["causal"] else 0) | (int(nd["out"]) << 16)
    return arr, slots


# ---- a compiled program with torch-managed memory --------------------------

_TORCH_DTYPE = None


def _torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64,
            "i32": torch.int32, "i16": torch.int16, "i8": torch.int8}[name]


class Program:
    """Owns an rv_program handle. ``slots`` names the input slots in order."""

    def __init__(self, handle: ctypes.c_void_p):
        self.h = handle
        self.slots: list[str] = []
        self.n_inputs, self.n_outputs = rv_program_io(handle)
        self.out_desc = [rv_output_desc(handle, i) for i in range(self.n_outputs)]
        self.ws_bytes = rv_workspace_size(handle)
        # one cached workspace per (device, stream): launches on different
        # streams may overlap, and the kernels keep scratch state there
        self._ws = {}

    def __del__(self):
        try:
            if self.h:
                rv_program_free(self.h)
                self.h = None
        except Exception:
            pass

    def describe(self) -> dict:
        import json
        return json.loads(rv_describe(self.h))

    def source(self) -> str:
        return rv_source(self.h)

    def alloc_outputs(self, device="cuda"):
        import torch
        return [torch.empty(shape, dtype=_torch_dtype(dt), device=device) for shape, dt in self.out_desc]

    def workspace(self, device="cuda", stream=None):
        """The cached workspace for launches on ``stream`` (None if the
        program needs none). Launches that may overlap must not share one:
        each stream gets its own."""
        import torch
        if not self.ws_bytes:
            return None
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        key = (str(dev), int(stream.cuda_stream) if stream is not None else 0)
        ws = self._ws.get(key)
        if ws is None:
            ws = self._ws[key] = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        return ws

    @staticmethod
    def _ws_args(ws):
        """(pointer, size in bytes) of a workspace tensor, or (0, 0)."""
        if ws is None:
            return 0, 0
        return ws.data_ptr(), ws.numel() * ws.element_size()

    def prepare(self, inputs: dict, outputs, stream, workspace=None):
        """Marshal the buffers once; the returned callable enqueues the
        program with no per-call Python work beyond the C call (for launch
        loops and graph capture)."""
        bufs = []
        for name in self.slots:
            t = inputs[name]
            if not t.is_contiguous():
                raise RVError(-1, f"input {name} must be contiguous")
            bufs.append(rv_buffer(t.data_ptr(), t.numel(), DTYPE[_dtype_name(t.dtype)], 0))
        for t in outputs:
            bufs.append(rv_buffer(t.data_ptr(), t.numel(), DTYPE[_dtype_name(t.dtype)], 0))
        arr = (rv_buffer * max(1, len(bufs)))(*bufs)
        n = len(bufs)
        ws = workspace if workspace is not None else self.workspace(outputs[0].device if outputs else "cuda", stream)
        wp, wsb = self._ws_args(ws)
        wptr = ctypes.c_void_p(wp or None)
        sptr = ctypes.c_void_p(stream.cuda_stream or None)
        h = self.h
        fn = _lib.rv_launch
        keep = (inputs, outputs, ws)

        def go():
            _check(fn(h, arr, n, wptr, wsb, sptr))
        go.keep = keep
        return go

    def launch(self, inputs: dict, outputs=None, stream=None, workspace=None):
        """Enqueue on ``stream`` (default: torch's current stream). ``inputs``
        maps slot names to device tensors (contiguous, of the declared dtype).
        Returns the output tensors."""
        import torch
        if outputs is None:
            outputs = self.alloc_outputs()
        bufs = []
        for name in self.slots:
            t = inputs[name]
            if not t.is_contiguous():
                raise RVError(-1, f"input {name} must be contiguous")
            bufs.append(rv_buffer(t.data_ptr(), t.numel(), DTYPE[_dtype_name(t.dtype)], 0))
        for t in outputs:
            bufs.append(rv_buffer(t.data_ptr(), t.numel(), DTYPE[_dtype_name(t.dtype)], 0))
        if stream is None:
            stream = torch.cuda.current_stream()
        ws = workspace if workspace is not None else self.workspace(outputs[0].device if outputs else "cuda", stream)
        wptr, wsb = self._ws_args(ws)
        rv_launch(self.h, bufs, wptr, wsb, stream.cuda_stream)
        return outputs


def _dtype_name(tdt) -> str:
    import torch
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16", torch.float64: "f64",
            torch.int32: "i32", torch.int16: "i16", torch.int8: "i8"}[tdt]


def compile_spec(spec) -> Program:
    """Compile a ``synth.Spec`` graph (host only; no device needed)."""
    nodes, slots = nodes_from_spec(spec)
    prog = rv_compile(nodes, list(spec.outputs))
    prog.slots = slots
    return prog
