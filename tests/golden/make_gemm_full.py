"""Writes tests/golden/gemm_relu2_sum_4096.json: the oracle's result for the
full-size bf16 contraction workload S = SUM(relu(y)^2), y = SUM_k CAST(A) *
CAST(B), A, B (4096, 4096) bf16 from seed 5, plus the fp64 ingredients of its
tolerance. Calls only oracle/ (and numpy for |A| @ |B|, a bound ingredient).
Run from the repository root: python tests/golden/make_gemm_full.py"""

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import interp  # noqa: E402
from reduce_view_amd import synth  # noqa: E402

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def main():
    m = n = k = 4096
    t = time.time()
    inp = synth.inputs_gemm(m, n, k, seed=5)
    spec = synth.gemm_relu2_sum(m, n, k, emit_y=True)
    s, y = oracle.run(spec, inp)
    y = y[:, :, 0].astype(np.float64)
    a = np.abs(interp.bf16_to_f32(inp["A"]).astype(np.float64))
    b = np.abs(interp.bf16_to_f32(inp["B"]).astype(np.float64))
    dy = 4 * gamma(k - 1) * (a @ b)
    q = np.maximum(y, 0) ** 2
    prop = float(np.sum((2 * np.abs(y) * dy + dy ** 2) * (y > -dy)))
    rows = [0, 1, 2047, 4095]
    out = {
        "workload": "gemm_relu2_sum 4096x4096x4096, inputs_gemm seed 5",
        "S": float(s.ravel()[0]),
        "S_bits": int(np.asarray(s, np.float32).view(np.uint32).ravel()[0]),
        "sum_q": float(q.sum()),
        "propagated_y_term": prop,
        "max_dy": float(dy.max()),
        "sample_rows": rows,
        "sample_y_bits": [[int(v) for v in np.asarray(y[r], np.float32).view(np.uint32)[:64]] for r in rows],
        "seconds": round(time.time() - t, 1),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_relu2_sum_4096.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path, out["S"], out["seconds"])


if __name__ == "__main__":
    main()
