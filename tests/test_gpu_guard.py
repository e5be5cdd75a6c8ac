"""Out-of-bounds writes have no numerical signature (Litmus README,
"Benchmark": of its planted bugs, an out-of-bounds write past the tensor is
among those no value check sees). Every output and the workspace of each
program is placed inside a larger allocation whose bands before and after
hold a sentinel pattern; the program is launched on the interior pointers
and the bands must come back untouched. One case per kernel class and plan,
at ragged shapes (tails that are not multiples of any vector width or tile)."""

import numpy as np
import pytest

from reduce_view_amd import rv, synth
from tests import test_gpu_parity as P
from tests.harness import to_device

pytestmark = pytest.mark.gpu

BAND = 4096  # bytes on each side (keeps the interior 256-byte aligned)
SENTINEL = 0xA5


def _guarded(nbytes, dev):
    import torch
    buf = torch.full((BAND + nbytes + BAND,), SENTINEL, dtype=torch.uint8, device=dev)
    return buf, buf[BAND:BAND + nbytes]


def _case(spec, inputs, classes):
    import torch
    prog = P._prog(spec)
    got = {(k["class"], k["plan"]) for k in prog.describe()["kernels"]}
    assert classes <= got, (classes, got)
    dev = torch.device("cuda", 0)
    dev_in = {k: to_device(v) for k, v in inputs.items() if k in prog.slots}
    outs, bufs = [], []
    for t in prog.alloc_outputs(dev):
        b, inner = _guarded(t.numel() * t.element_size(), dev)
        outs.append(inner.view(t.dtype).view(t.shape))
        bufs.append(b)
    ws = None
    if prog.ws_bytes:
        b, ws = _guarded(prog.ws_bytes, dev)
        bufs.append(b)
    stream = torch.cuda.current_stream()
    prog.launch(dev_in, outs, stream=stream, workspace=ws)
    torch.cuda.synchronize()
    for b in bufs:
        h = b.cpu().numpy()
        assert (h[:BAND] == SENTINEL).all() and (h[-BAND:] == SENTINEL).all(), spec.name


def _rng_inputs(shapes, seed):
    rng = np.random.default_rng(seed)
    return {k: (synth.to_bf16_bits(rng.standard_normal(s).astype(np.float32)) if dt == "bf16"
                else rng.standard_normal(s).astype(np.float32)) for k, (s, dt) in shapes.items()}


CASES = {
    "ew_tiled_masked": (lambda: synth.ew_chain(67, 131, masked=True), lambda: synth.inputs_ew(67, 131),
                        {("EW", "tiled2d")}),
    "ew_transpose": (lambda: synth.transpose(100, 37), lambda: {"X": synth.inputs_ew(100, 37)["X"]},
                     {("EW", "tiled2d")}),
    "ew_rowmajor_i8": (lambda: synth.chain_int(33, 77, "i8"), lambda: synth.inputs_chain_int(33, 77, "i8"),
                       {("EW", "rowmajor")}),
    "ew_cast_matrix": (lambda: synth.cast_matrix(77), lambda: synth.inputs_cast(77), {("EW", "rowmajor")}),
    "row_softmax": (lambda: synth.softmax(33, 1000), lambda: synth.inputs_softmax(33, 1000), {("ROW", "row")}),
    "row_layernorm": (lambda: synth.layernorm(9, 1000), lambda: synth.inputs_layernorm(9, 1000), {("ROW", "row")}),
    "row_stream": (lambda: synth.softmax(5, 70001), lambda: synth.inputs_softmax(5, 70001), {("ROW", "row_stream")}),
    "reduce_cells": (lambda: synth.matmul_broadcast(37, 70, 19), lambda: synth.inputs_matmul(37, 70, 19),
                     {("REDUCE", "cells")}),
    "split_row": (lambda: synth.reduce((7, 200003), (1,)), lambda: synth.inputs_reduce((7, 200003)),
                  {("SPLIT", "split_row"), ("FOLD", "fold_cells")}),
    "split_cols": (lambda: synth.reduce((40009, 77), (0,)), lambda: synth.inputs_reduce((40009, 77)),
                   {("SPLIT", "split_cols"), ("FOLD", "fold_cells")}),
    "mfma_fold_ragged": (lambda: synth.gemm_relu2_sum(257, 129, 65), lambda: synth.inputs_gemm(257, 129, 65),
                         {("EW", "rowmajor"), ("MFMA", "gemm_w6"), ("FOLD", "fold")}),
    "mfma_store_ragged": (lambda: synth.gemm_bf16(300, 257, 64), lambda: synth.inputs_gemm(300, 257, 64),
                          {("MFMA", "gemm_w6")}),
    "mfma_store_shifted": (lambda: synth.gemm_bf16(520, 264, 96), lambda: synth.inputs_gemm(520, 264, 96),
                           {("MFMA", "gemm_w6")}),
    "mfma_split_fold": (lambda: synth.gemm_relu2_sum(300, 520, 2048), lambda: synth.inputs_gemm(300, 520, 2048),
                        {("MFMA", "gemm_w6"), ("MFMA", "gemm_slices"), ("FOLD", "fold")}),
    "mfma_split_store": (lambda: synth.gemm_bf16(40, 24, 1024), lambda: synth.inputs_gemm(40, 24, 1024),
                         {("EW", "rowmajor"), ("MFMA", "gemm_w6"), ("MFMA", "gemm_slices")}),
    "attn": (lambda: synth.attention(2, 300, 333, 64, True),
             lambda: synth.inputs_attention(2, 300, 333, 64), {("ATTN", "attn_fwd")}),
    "attn_chunked": (lambda: synth.attention(1, 4100, 4100, 32, True),
                     lambda: synth.inputs_attention(1, 4100, 4100, 32), {("ATTN", "attn_fwd"), ("ATTN", "attn_merge")}),
    "gather": (lambda: synth.embedding_gather(50, 6, 30), lambda: synth.inputs_embedding(50, 6, 30),
               {("EW", "rowmajor")}),
    "scatter_ordered": (lambda: synth.embedding_scatter(20, 6, 100), lambda: synth.inputs_embedding(20, 6, 100),
                        {("SCATTER", "scatter_fold")}),
    "scatter_atomic": (lambda: synth.embedding_scatter(20, 6, 100, atomic=True),
                       lambda: synth.inputs_embedding(20, 6, 100), {("SCATTER", "scatter_atomic")}),
}


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rv.rv_init(0)


@pytest.mark.parametrize("name", list(CASES))
def test_writes_stay_inside_outputs_and_workspace(name):
    mk_spec, mk_in, classes = CASES[name]
    P._case(f"guard bands {name}")
    _case(mk_spec(), mk_in(), classes)
