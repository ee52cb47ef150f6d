"""The synthetic workloads use the pages' shapes (CPU only)."""
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "microbench_shapes.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            rows.append((line[0], int(line[1]), int(line[2]), int(line[3])))
    return rows


def test_single_gemm_cases_use_the_printed_microbench_shapes():
    rows = _golden_rows()
    cases = list(synth.CASES.values())
    assert len(rows) == len(cases) == 4
    for (layer, M, K, N), c in zip(rows, cases):
        assert (c.M, c.K, c.N) == (M, K, N), layer


def test_stack_is_the_3b_scale_config():
    assert synth.N_LAYERS == 36
    shapes = {name: (K, N) for name, K, N in synth.STACK_PROJS}
    rows = _golden_rows()
    for layer, M, K, N in rows:
        assert shapes[layer.split(".")[1]] == (K, N)
    assert synth.STACK_M == tuple(r[1] for r in rows)


def test_inputs_are_seeded_and_shaped():
    c = synth.CASES["int8_w8a16_1x2048x2048"]
    a, b = synth.case_inputs(c), synth.case_inputs(c)
    assert np.array_equal(a.w, b.w) and np.array_equal(a.x, b.x)
    assert a.w.shape == (2048, 2048) and a.w.dtype == np.float32
    assert a.x.shape == (1, 2048) and a.x.dtype == np.uint16
    assert a.calib.shape == (64, 2048)
    assert abs(float(a.w.std()) - 0.02) < 1e-3
    w0 = synth.stack_weight(0, 3, 1, "cpu")
    assert w0.shape == (11008, 2048) and w0.dtype == torch.float32
    assert torch.equal(w0, synth.stack_weight(0, 3, 1, "cpu"))
    assert not torch.equal(w0[:2048, :], synth.stack_weight(0, 3, 0, "cpu"))
    assert abs(float(w0.std()) - 0.02) < 1e-3
    calib, x = synth.stack_inputs(0, 16)
    assert calib.shape == (64, 2048) and x.shape == (16, 2048)
