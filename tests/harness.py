"""Test-side helpers: moving seeded numpy inputs to the device, running a
compiled program through the C ABI binding, and reading results back."""

from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def gamma(n: int, u: float = U) -> float:
    """gamma_n = n u / (1 - n u) (Litmus README, ToleranceBound: the
    reduction-order term)."""
    return n * u / (1.0 - n * u) if n * u < 1 else float("inf")


def to_device(arr: np.ndarray, device="cuda"):
    import torch
    if arr.dtype == np.uint16:  # bfloat16 bit patterns
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def run(prog, inputs: dict, device="cuda"):
    import torch
    dev_in = {k: to_device(v, device) for k, v in inputs.items() if k in prog.slots}
    outs = prog.launch(dev_in)
    torch.cuda.synchronize()
    return [to_host(o) for o in outs]


def ulp32(x) -> np.ndarray:
    """Spacing of float32 at |x| (2^-149 for zero/subnormals)."""
    a = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(a).astype(np.float64)


def ulp_bf16(x) -> np.ndarray:
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -133)))
    return 2.0 ** (e - 7)


def report(name: str, err: np.ndarray, bound: np.ndarray) -> dict:
    """max |err|, max bound, max err/bound for the record."""
    err = np.asarray(err, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    r = dict(name=name, max_err=float(err.max(initial=0.0)), max_bound=float(bound.max(initial=0.0)),
             max_err_over_bound=float(ratio.max(initial=0.0)))
    print("BOUND", r, flush=True)
    return r


def contraction_sum_depth(desc: dict) -> int:
    """Additions a relu^2-sum partial passes through after the contraction:
    the epilogue's partial sum in the last MFMA kernel (the slice fold when
    the contraction is split over k) plus the fold of the partials."""
    mf = [k for k in desc["kernels"] if k["class"] == "MFMA"][-1]
    fo = [k for k in desc["kernels"] if k["class"] == "FOLD"]
    return mf["plan_detail"]["partial_sum_depth"] + (fo[0]["plan_detail"]["sum_depth"] if fo else 0)
