"""ctypes binding of libqlq.so: argument marshalling only.

Every function here checks shapes and dtypes, allocates outputs with PyTorch on
the tensors' device, and forwards plain pointers, sizes and the current HIP
stream to the C ABI declared in include/qlq.h.  All arithmetic runs in the HIP
kernels; there is no fallback path: if the library is not built, or the tensors
are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlq.so")

QTYPES = {"int8": 0, "fp8_e4m3fn": 1}
GRANULARITIES = {"per_channel": 0, "per_tensor": 1}
OUTS = {"bf16": 0, "acc": 1}
SCHEMES = {"w8a16": 0, "w8a8_static": 1, "w8a8_static_fused": 2, "w8a8_dynamic": 3}
STATUS = {0: "QLQ_OK", 1: "QLQ_ERR_INVALID_ARG", 2: "QLQ_ERR_UNSUPPORTED", 3: "QLQ_ERR_HIP"}

# name -> (restype, argtypes), mirroring include/qlq.h
_c = ctypes
_SIGNATURES = {
    "qlq_packed_weight_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64]),
    "qlq_workspace_bytes": (_c.c_size_t, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "qlq_quantize_weight": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                       _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "qlq_unpack_weight": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p]),
    "qlq_calibrate_input_scale": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p]),
    "qlq_quantize_act_static": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_float, _c.c_int,
                                           _c.c_void_p, _c.c_void_p]),
    "qlq_qlinear_w8a16": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                                     _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "qlq_qlinear_w8a16_noalloc": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p,
                                             _c.c_void_p, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p]),
    "qlq_qlinear_w8a8_static": (_c.c_int, [_c.c_void_p, _c.c_float, _c.c_int64, _c.c_int64, _c.c_int64,
                                           _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int, _c.c_int,
                                           _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "qlq_qlinear_w8a8_static_requant": (_c.c_int, [_c.c_void_p, _c.c_float, _c.c_int64, _c.c_int64, _c.c_int64,
                                                   _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int, _c.c_float,
                                                   _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                                   _c.c_void_p]),
    "qlq_quantize_act_dynamic": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p,
                                            _c.c_void_p, _c.c_void_p]),
    "qlq_qlinear_w8a8_static_fused": (_c.c_int, [_c.c_void_p, _c.c_float, _c.c_int64, _c.c_int64, _c.c_int64,
                                                 _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int, _c.c_int,
                                                 _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "qlq_qlinear_w8a8_dynamic": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                            _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int, _c.c_int,
                                            _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "qlq_kv_quantize": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p,
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "qlq_kv_dequantize": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                                     _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "qlq_linear": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                              _c.c_int64, _c.c_int, _c.c_float, _c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p,
                              _c.c_size_t, _c.c_void_p]),
    "qlq_linear_workspace_bytes": (_c.c_size_t, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "qlq_gemm_plan": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p]),
    "qlq_scale_is_calibrated": (_c.c_int, [_c.c_float]),
    "qlq_status_string": (_c.c_char_p, [_c.c_int]),
    "qlq_last_error": (_c.c_char_p, []),
    "qlq_version": (_c.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


class QlqError(RuntimeError):
    """A non-OK status from libqlq (validation or launch failure)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libqlq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                                      "`python -m weight_quantized_linear_qlinear_amd.build`")
                h = ctypes.CDLL(_LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    f = getattr(h, name)
                    f.restype = res
                    f.argtypes = args
                _lib = h
    return _lib


def _check(status: int):
    if status != 0:
        raise QlqError(status, lib().qlq_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _require_gpu(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("qlq operates on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("qlq needs contiguous (row-major) tensors")


def _qtype(q: str) -> int:
    if q not in QTYPES:
        raise ValueError(f"qtype must be one of {sorted(QTYPES)}")
    return QTYPES[q]


def code_dtype(qtype: str) -> torch.dtype:
    """torch dtype used for 1-byte codes: int8 for INT8, uint8 (raw bits) for e4m3fn."""
    return torch.int8 if qtype == "int8" else torch.uint8


# ---------------------------------------------------------------------- sizing
def packed_weight_bytes(N: int, K: int) -> int:
    return int(lib().qlq_packed_weight_bytes(N, K))


def workspace_bytes(scheme: str, M: int, K: int, N: int, qtype: str) -> int:
    return int(lib().qlq_workspace_bytes(SCHEMES[scheme], M, K, N, _qtype(qtype)))


class _PlanInfo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("cfg", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]


def gemm_plan(scheme: str, M: int, K: int, N: int, qtype: str) -> dict:
    """The launch plan a GEMM call takes for these sizes (test hook; host only)."""
    info = _PlanInfo()
    _check(lib().qlq_gemm_plan(SCHEMES[scheme], M, K, N, _qtype(qtype), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in _PlanInfo._fields_}


def scale_is_calibrated(s: float) -> bool:
    """Whether the quantizers take the refined-reciprocal division for scale s (test hook)."""
    return bool(lib().qlq_scale_is_calibrated(float(s)))


_workspaces: dict = {}


def _workspace(dev: torch.device, nbytes: int) -> torch.Tensor | None:
    """A zero-filled per-device workspace, grown on demand (the kernels leave it zeroed)."""
    if nbytes == 0:
        return None
    key = (dev.type, dev.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


# ---------------------------------------------------------------------- weights
@dataclasses.dataclass
class QuantizedWeight:
    """A packed quantized weight of logical shape [N, K] and its fp32 scales."""
    packed: torch.Tensor      # uint8, packed_weight_bytes(N, K)
    scale: torch.Tensor       # fp32 [N] (per channel) or [1] (per tensor)
    N: int
    K: int
    qtype: str
    granularity: str


def quantize_weight(w: torch.Tensor, qtype: str, granularity: str = "per_channel",
                    packed: torch.Tensor | None = None, scale: torch.Tensor | None = None) -> QuantizedWeight:
    """Quantize and pack W[N, K] (fp32 or bf16, on the GPU)."""
    _require_gpu(w)
    if w.dim() != 2 or w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be a 2-D fp32 or bf16 tensor")
    N, K = w.shape
    if granularity not in GRANULARITIES:
        raise ValueError(f"granularity must be one of {sorted(GRANULARITIES)}")
    if packed is None:
        packed = torch.empty(packed_weight_bytes(N, K), dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(N if granularity == "per_channel" else 1, dtype=torch.float32, device=w.device)
    _check(lib().qlq_quantize_weight(_ptr(w), int(w.dtype == torch.bfloat16), N, K, _qtype(qtype),
                                     GRANULARITIES[granularity], _ptr(packed), _ptr(scale), _stream(w.device)))
    return QuantizedWeight(packed, scale, N, K, qtype, granularity)


def unpack_weight(qw: QuantizedWeight) -> torch.Tensor:
    """Row-major [N, K] codes of a packed weight (test hook)."""
    out = torch.empty((qw.N, qw.K), dtype=code_dtype(qw.qtype), device=qw.packed.device)
    _check(lib().qlq_unpack_weight(_ptr(qw.packed), qw.N, qw.K, _ptr(out), _stream(out.device)))
    return out


# ---------------------------------------------------------------------- activations
def calibrate_input_scale(x_calib: torch.Tensor, qtype: str, out: torch.Tensor | None = None) -> torch.Tensor:
    """Static input scale absmax(x_calib) / qmax as a one-element fp32 device tensor."""
    _require_gpu(x_calib)
    if x_calib.dtype != torch.bfloat16:
        raise ValueError("x_calib must be bf16")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x_calib.device)
    _check(lib().qlq_calibrate_input_scale(_ptr(x_calib), x_calib.numel(), _qtype(qtype), _ptr(out),
                                           _stream(x_calib.device)))
    return out


def quantize_act_static(x: torch.Tensor, input_scale: float, qtype: str,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Codes of x [M, K] bf16 with the fixed scalar input_scale."""
    _require_gpu(x)
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bf16 tensor")
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K), dtype=code_dtype(qtype), device=x.device)
    _check(lib().qlq_quantize_act_static(_ptr(x), M, K, float(input_scale), _qtype(qtype), _ptr(out),
                                         _stream(x.device)))
    return out


def quantize_act_dynamic(x: torch.Tensor, qtype: str, out: torch.Tensor | None = None,
                         x_scale: torch.Tensor | None = None):
    """Per-token codes of x [M, K] bf16 and their row scales: (xq [M, K], x_scale fp32 [M])."""
    _require_gpu(x)
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bf16 tensor")
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K), dtype=code_dtype(qtype), device=x.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().qlq_quantize_act_dynamic(_ptr(x), M, K, _qtype(qtype), _ptr(out), _ptr(x_scale),
                                          _stream(x.device)))
    return out, x_scale


# ---------------------------------------------------------------------- GEMMs
def qlinear_w8a16(x: torch.Tensor, qw: QuantizedWeight, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = x W^T with W dequantized to bf16 in the kernel; x bf16 [M, K] -> y bf16 [M, N]."""
    _require_gpu(x)
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.shape[1] != qw.K:
        raise ValueError(f"x must be bf16 [M, {qw.K}]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, qw.N), dtype=torch.bfloat16, device=x.device)
    nbytes = workspace_bytes("w8a16", M, qw.K, qw.N, qw.qtype)
    ws = workspace if workspace is not None else _workspace(x.device, nbytes)
    _check(lib().qlq_qlinear_w8a16(_ptr(x), M, qw.K, qw.N, _ptr(qw.packed), _ptr(qw.scale), qw.scale.numel(),
                                   _qtype(qw.qtype), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(x.device)))
    return out


def qlinear_w8a16_noalloc(x: torch.Tensor, qw: QuantizedWeight, out: torch.Tensor) -> torch.Tensor:
    """qlinear_w8a16 without a workspace (split-K scratch inside the library); out is required."""
    _require_gpu(x, out)
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.shape[1] != qw.K:
        raise ValueError(f"x must be bf16 [M, {qw.K}]")
    M = x.shape[0]
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, qw.N):
        raise ValueError(f"out must be bf16 [{M}, {qw.N}]")
    _check(lib().qlq_qlinear_w8a16_noalloc(_ptr(x), M, qw.K, qw.N, _ptr(qw.packed), _ptr(qw.scale),
                                           qw.scale.numel(), _qtype(qw.qtype), _ptr(out), _stream(x.device)))
    return out


def qlinear_w8a8_static(xq: torch.Tensor, input_scale: float, qw: QuantizedWeight, out_mode: str = "bf16",
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W8A8 static GEMM on codes xq [M, K]: bf16 y [M, N], or raw accumulators (out_mode="acc")."""
    _require_gpu(xq)
    if xq.dim() != 2 or xq.element_size() != 1 or xq.shape[1] != qw.K:
        raise ValueError(f"xq must be 1-byte codes [M, {qw.K}]")
    M = xq.shape[0]
    if out is None:
        if out_mode == "acc":
            dt = torch.int32 if qw.qtype == "int8" else torch.float32
        else:
            dt = torch.bfloat16
        out = torch.empty((M, qw.N), dtype=dt, device=xq.device)
    nbytes = workspace_bytes("w8a8_static", M, qw.K, qw.N, qw.qtype)
    ws = workspace if workspace is not None else _workspace(xq.device, nbytes)
    _check(lib().qlq_qlinear_w8a8_static(_ptr(xq), float(input_scale), M, qw.K, qw.N, _ptr(qw.packed),
                                         _ptr(qw.scale), qw.scale.numel(), _qtype(qw.qtype), OUTS[out_mode],
                                         _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                                         _stream(xq.device)))
    return out


def qlinear_w8a8_static_requant(xq: torch.Tensor, input_scale: float, qw: QuantizedWeight, next_scale: float,
                                out: torch.Tensor | None = None, out_codes: torch.Tensor | None = None,
                                workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """W8A8 static GEMM on codes xq [M, K] that also quantizes its bf16 output for the next static layer:
    returns (y bf16 [M, N], codes [M, N] of y at next_scale, same qtype)."""
    _require_gpu(xq)
    if xq.dim() != 2 or xq.element_size() != 1 or xq.shape[1] != qw.K:
        raise ValueError(f"xq must be 1-byte codes [M, {qw.K}]")
    M = xq.shape[0]
    if out is None:
        out = torch.empty((M, qw.N), dtype=torch.bfloat16, device=xq.device)
    if out_codes is None:
        out_codes = torch.empty((M, qw.N), dtype=code_dtype(qw.qtype), device=xq.device)
    if out_codes.shape != (M, qw.N) or out_codes.element_size() != 1:
        raise ValueError(f"out_codes must be 1-byte codes [{M}, {qw.N}]")
    nbytes = workspace_bytes("w8a8_static", M, qw.K, qw.N, qw.qtype)
    ws = workspace if workspace is not None else _workspace(xq.device, nbytes)
    _check(lib().qlq_qlinear_w8a8_static_requant(_ptr(xq), float(input_scale), M, qw.K, qw.N, _ptr(qw.packed),
                                                 _ptr(qw.scale), qw.scale.numel(), _qtype(qw.qtype),
                                                 float(next_scale), _ptr(out), _ptr(out_codes), _ptr(ws),
                                                 0 if ws is None else ws.numel(), _stream(xq.device)))
    return out, out_codes


def _w8a8_out(M: int, qw: QuantizedWeight, out_mode: str, dev: torch.device) -> torch.Tensor:
    if out_mode == "acc":
        dt = torch.int32 if qw.qtype == "int8" else torch.float32
    else:
        dt = torch.bfloat16
    return torch.empty((M, qw.N), dtype=dt, device=dev)


def qlinear_w8a8_static_fused(x: torch.Tensor, input_scale: float, qw: QuantizedWeight, out_mode: str = "bf16",
                              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """quantize_act_static + qlinear_w8a8_static in one call, from bf16 x [M, K]."""
    _require_gpu(x)
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.shape[1] != qw.K:
        raise ValueError(f"x must be bf16 [M, {qw.K}]")
    M = x.shape[0]
    if out is None:
        out = _w8a8_out(M, qw, out_mode, x.device)
    nbytes = workspace_bytes("w8a8_static_fused", M, qw.K, qw.N, qw.qtype)
    ws = workspace if workspace is not None else _workspace(x.device, nbytes)
    _check(lib().qlq_qlinear_w8a8_static_fused(_ptr(x), float(input_scale), M, qw.K, qw.N, _ptr(qw.packed),
                                               _ptr(qw.scale), qw.scale.numel(), _qtype(qw.qtype), OUTS[out_mode],
                                               _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                                               _stream(x.device)))
    return out


def qlinear_w8a8_dynamic(xq: torch.Tensor, x_scale: torch.Tensor, qw: QuantizedWeight, out_mode: str = "bf16",
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W8A8 GEMM on per-token codes xq [M, K] with row scales x_scale fp32 [M]."""
    _require_gpu(xq, x_scale)
    if xq.dim() != 2 or xq.element_size() != 1 or xq.shape[1] != qw.K:
        raise ValueError(f"xq must be 1-byte codes [M, {qw.K}]")
    M = xq.shape[0]
    if x_scale.dtype != torch.float32 or x_scale.numel() != M:
        raise ValueError(f"x_scale must be fp32 [{M}]")
    if out is None:
        out = _w8a8_out(M, qw, out_mode, xq.device)
    nbytes = workspace_bytes("w8a8_dynamic", M, qw.K, qw.N, qw.qtype)
    ws = workspace if workspace is not None else _workspace(xq.device, nbytes)
    _check(lib().qlq_qlinear_w8a8_dynamic(_ptr(xq), _ptr(x_scale), M, qw.K, qw.N, _ptr(qw.packed),
                                          _ptr(qw.scale), qw.scale.numel(), _qtype(qw.qtype), OUTS[out_mode],
                                          _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                                          _stream(xq.device)))
    return out


# ---------------------------------------------------------------------- routed Linear
LINEAR_SCHEMES = {"w8a16": 0, "w8a8_static": 1, "w8a8_dynamic": 3}


def linear_workspace_bytes(scheme: str, M: int, K: int, N: int, qtype: str) -> int:
    return int(lib().qlq_linear_workspace_bytes(LINEAR_SCHEMES[scheme], M, K, N, _qtype(qtype)))


def linear(scheme: str, x: torch.Tensor, qw: QuantizedWeight, input_scale: float = 1.0,
           bias: torch.Tensor | None = None, bf16_fallback_max_m: int = 0, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Routed quantized Linear: bf16 x [M, K] -> bf16 y [M, N] (+ bf16 bias [N])."""
    _require_gpu(x)
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.shape[1] != qw.K:
        raise ValueError(f"x must be bf16 [M, {qw.K}]")
    if bias is not None:
        _require_gpu(bias)
        if bias.dtype != torch.bfloat16 or bias.numel() != qw.N:
            raise ValueError(f"bias must be bf16 [{qw.N}]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, qw.N), dtype=torch.bfloat16, device=x.device)
    nbytes = linear_workspace_bytes(scheme, M, qw.K, qw.N, qw.qtype)
    ws = workspace if workspace is not None else _workspace(x.device, nbytes)
    _check(lib().qlq_linear(LINEAR_SCHEMES[scheme], _ptr(x), M, qw.K, qw.N, _ptr(qw.packed), _ptr(qw.scale),
                            qw.scale.numel(), _qtype(qw.qtype), float(input_scale), _ptr(bias),
                            int(bf16_fallback_max_m), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                            _stream(x.device)))
    return out


# ---------------------------------------------------------------------- KV cache
@dataclasses.dataclass
class QuantizedKV:
    """Mixed K-int8 / V-FP8 cache entries for [T, H, D] keys and values."""
    k_codes: torch.Tensor     # int8 [T, H, D]
    k_scales: torch.Tensor    # float16 [T, H, D / 32]
    v_codes: torch.Tensor     # uint8 e4m3fn bits [T, H, D]
    v_scales: torch.Tensor    # float16 [T, H]


def kv_quantize(k: torch.Tensor, v: torch.Tensor, out: QuantizedKV | None = None) -> QuantizedKV:
    """Quantize bf16 K and V [T, H, D] (D % 32 == 0) into cache entries."""
    _require_gpu(k, v)
    if k.dim() != 3 or k.shape != v.shape or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("k and v must be bf16 [T, H, D] of the same shape")
    T, H, D = k.shape
    if out is None:
        out = QuantizedKV(torch.empty((T, H, D), dtype=torch.int8, device=k.device),
                          torch.empty((T, H, max(D // 32, 1)), dtype=torch.float16, device=k.device),
                          torch.empty((T, H, D), dtype=torch.uint8, device=k.device),
                          torch.empty((T, H), dtype=torch.float16, device=k.device))
    _check(lib().qlq_kv_quantize(_ptr(k), _ptr(v), T, H, D, _ptr(out.k_codes), _ptr(out.k_scales),
                                 _ptr(out.v_codes), _ptr(out.v_scales), _stream(k.device)))
    return out


def kv_dequantize(q: QuantizedKV, k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None):
    """Cache entries -> bf16 (K, V) [T, H, D]."""
    _require_gpu(q.k_codes, q.k_scales, q.v_codes, q.v_scales)
    T, H, D = q.k_codes.shape
    if k_out is None:
        k_out = torch.empty((T, H, D), dtype=torch.bfloat16, device=q.k_codes.device)
    if v_out is None:
        v_out = torch.empty((T, H, D), dtype=torch.bfloat16, device=q.k_codes.device)
    _check(lib().qlq_kv_dequantize(_ptr(q.k_codes), _ptr(q.k_scales), _ptr(q.v_codes), _ptr(q.v_scales), T, H, D,
                                   _ptr(k_out), _ptr(v_out), _stream(q.k_codes.device)))
    return k_out, v_out
