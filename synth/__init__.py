"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and describes workload shapes.  It holds
none of the quantized-linear arithmetic (no scales, no codes, no products), so
both sides of a parity check can take their inputs from here without sharing
any of the method.

Recipe (the pages benchmark a 3B-scale configuration with hidden size 2048,
intermediate size 11008 and 36 layers, and microbenchmark q_proj, up_proj and
down_proj of that model at four token counts -- "Nano-vLLM-MoE" README, section
"FP8 W8A8 static quantization", Setup list and "Linear-backend microbench
(3B-scale)" table):

* generator: ``numpy.random.default_rng(seed)`` (PCG64),
  ``standard_normal(dtype=float32)``;
* weights W[N, K] (out x in) are ``0.02 * N(0, 1)`` in fp32;
* activations and calibration batches are ``N(0, 1)`` fp32 draws cast to
  bf16 with round-to-nearest-even (torch's CPU cast, an independent library);
* draw order inside one single-GEMM case: W, then the 64-row calibration
  batch, then x;
* the 36-layer stack (1.76 G weights) draws each (layer, projection) weight on
  the device with torch's Philox generator seeded with
  ``seed * 1000003 + 3 * layer + proj + 1`` (``torch.randn`` in fp32, times
  0.02), so any layer can be produced without drawing the ones before it and
  without minutes of host RNG; its calibration batch and input come from
  ``default_rng((seed, 1000))`` in that order.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

HIDDEN = 2048
INTERMEDIATE = 11008
N_LAYERS = 36
CALIB_ROWS = 64
WEIGHT_STD = 0.02

# (name, K_in, N_out) of one decoder layer's three projections, in chain order.
STACK_PROJS = (("q_proj", HIDDEN, HIDDEN),
               ("up_proj", HIDDEN, INTERMEDIATE),
               ("down_proj", INTERMEDIATE, HIDDEN))
STACK_M = (1, 16, 256, 1024)


@dataclasses.dataclass(frozen=True)
class GemmCase:
    """One quantized-linear call: shapes, scheme and weight codec."""
    name: str
    scheme: str          # "w8a16" or "w8a8_static"
    qtype: str           # "int8" or "fp8_e4m3fn"
    granularity: str     # "per_channel" or "per_tensor"
    M: int
    K: int
    N: int
    seed: int = 0


# The four single-GEMM workloads: the pages' q_proj / up_proj / down_proj /
# up_proj microbench shapes, each with the scheme it is exercised with here.
CASES = {
    "int8_w8a16_1x2048x2048": GemmCase("int8_w8a16_1x2048x2048", "w8a16", "int8",
                                       "per_channel", 1, 2048, 2048),
    "fp8_w8a16_16x2048x11008": GemmCase("fp8_w8a16_16x2048x11008", "w8a16", "fp8_e4m3fn",
                                        "per_channel", 16, 2048, 11008),
    "int8_w8a8_256x11008x2048": GemmCase("int8_w8a8_256x11008x2048", "w8a8_static", "int8",
                                         "per_channel", 256, 11008, 2048),
    "fp8_w8a8_1024x2048x11008": GemmCase("fp8_w8a8_1024x2048x11008", "w8a8_static", "fp8_e4m3fn",
                                         "per_tensor", 1024, 2048, 11008),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even cast of an fp32 array to bf16, returned as uint16 bits.

    Uses torch's CPU cast so that neither side of a parity check supplies it.
    """
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """W[N, K] fp32 ~ 0.02 * N(0, 1)."""
    return (np.float32(WEIGHT_STD) * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float32)


def act_bf16(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """x[M, K] ~ N(0, 1), cast to bf16 (uint16 bits)."""
    return f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


@dataclasses.dataclass
class CaseInputs:
    w: np.ndarray        # fp32 [N, K]
    calib: np.ndarray    # bf16 bits [64, K] (drawn for every case, used by W8A8)
    x: np.ndarray        # bf16 bits [M, K]


def case_inputs(case: GemmCase, M: int | None = None) -> CaseInputs:
    """Inputs of a single-GEMM case.  ``M`` overrides the row count of x only."""
    rng = np.random.default_rng(case.seed)
    w = weight(rng, case.N, case.K)
    calib = act_bf16(rng, CALIB_ROWS, case.K)
    x = act_bf16(rng, case.M if M is None else M, case.K)
    return CaseInputs(w, calib, x)


def small_inputs(seed: int, M: int, K: int, N: int, w_std: float = WEIGHT_STD):
    """(W fp32 [N,K], calib bf16 bits [64,K], x bf16 bits [M,K]) for arbitrary sizes."""
    rng = np.random.default_rng(seed)
    w = (np.float32(w_std) * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float32)
    calib = act_bf16(rng, CALIB_ROWS, K)
    x = act_bf16(rng, M, K)
    return w, calib, x


def stack_weight(seed: int, layer: int, proj: int, device) -> torch.Tensor:
    """fp32 weight of projection ``proj`` (0 q, 1 up, 2 down) of decoder layer ``layer``.

    Drawn on ``device`` (the recipe is defined for a GPU device; a CPU device
    gives a different, equally seeded stream).
    """
    _, K, N = STACK_PROJS[proj]
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 3 * layer + proj + 1)
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32).mul_(WEIGHT_STD)


def stack_inputs(seed: int, M: int):
    """(calib bf16 bits [64, 2048], x bf16 bits [M, 2048]) of the layer stack."""
    rng = np.random.default_rng((seed, 1000))
    calib = act_bf16(rng, CALIB_ROWS, HIDDEN)
    x = act_bf16(rng, M, HIDDEN)
    return calib, x
