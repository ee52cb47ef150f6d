"""Helpers for the GPU parity tests: moving seeded inputs to the device and the
tolerance on bf16/fp32 results (relL2 <= 4e-3 and |err| <= 8e-3 (|ref| + rms(ref)))."""
import numpy as np
import torch

REL_L2_TOL = 4e-3
ELEM_TOL = 8e-3


def dev():
    return torch.device("cuda:0")


def bf16_to_gpu(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def f32_to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.uint8).numpy()


def check_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """relL2 <= 4e-3 and |err| <= 8e-3 (|ref| + rms(ref)) elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    nrm = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / nrm if nrm > 0 else err
    rms = np.sqrt(np.mean(ref ** 2))
    elem = np.max(np.abs(got - ref) / (np.abs(ref) + rms)) if rms > 0 else np.max(np.abs(got - ref))
    assert rel <= REL_L2_TOL, f"{what}: relL2 {rel:.3e}"
    assert elem <= ELEM_TOL, f"{what}: elementwise {elem:.3e}"
    return rel, elem
