"""Block-scaled (NVFP4 / MXFP8) MoE layer forward for MI355X: Python binding.

Argument marshalling only: tensors are checked (dtype, contiguity, shape,
device) and their device pointers handed to the C ABI in include/moe_fp4.h;
every step of the layer runs in the HIP library libmoe_fp4.so. There is no
fallback: if the library is missing, importing the binding fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmoe_fp4.so")

MODES = {"w4a4_tensor": 0, "w4a4_token": 1, "w4a16": 2, "mxfp8": 3, "w4a4_token_4o6": 4,
         "w4a4_token_mxfp4": 5}
ACTS = {"swiglu": 0, "relu2": 1}
WFMTS = {"nvfp4": 0, "mxfp8": 1, "mxfp4": 2}
VIEWS = {"topk_ids": 0, "topk_w": 1, "counts": 2, "offsets": 3, "row_to_route": 4,
         "route_to_row": 5, "x_codes": 6, "x_scales": 7, "x_g": 8, "a2_pre": 9,
         "a2_codes": 10, "a2_scales": 11, "a2_g": 12, "o": 13, "x_mx_codes": 14,
         "x_mx_scales": 15, "a2_mx_codes": 16, "a2_mx_scales": 17}
STAGES = ["route", "permute", "quantize_x", "fc1", "quantize_fc2_input", "fc2", "finalize"]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe_fp4 error {code}: {msg}")
        self.code = code


class _Dims(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("act", ctypes.c_int32), ("wfmt", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(_Dims)
    sig = {
        "moe_prepared_bytes": (sz, [D]),
        "moe_prepare_weights": (ctypes.c_int, [D, P, P, P, sz, P]),
        "moe_check_prepared": (ctypes.c_int, [D, P, P]),
        "moe_workspace_bytes": (sz, [D, i32, i32, i32]),
        "moe_forward": (ctypes.c_int, [D, P, sz, P, P, i32, i32, i32, i32, i32, i32, P, sz, P, P]),
        "moe_forward_status": (ctypes.c_int, [P, ctypes.POINTER(i32), P]),
        "moe_forward_noalloc": (ctypes.c_int, [D, P, sz, P, P, i32, i32, i32, i32, i32, i32, P, P]),
        "moe_finalize": (ctypes.c_int, [P, i32, P, P, i32, i32, i32, P, P]),
        "moe_quantize": (ctypes.c_int, [P, i32, i32, i32, P, P, P, P, P]),
        "moe_workspace_view": (ctypes.c_int, [D, i32, i32, i32, i32, ctypes.POINTER(sz),
                                              ctypes.POINTER(sz)]),
        "moe_stage_timing": (ctypes.c_int, [i32]),
        "moe_stage_times": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), i32,
                                           ctypes.POINTER(i32)]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


_lib = _load()
EXPORTS = ["moe_prepared_bytes", "moe_prepare_weights", "moe_check_prepared",
           "moe_workspace_bytes", "moe_forward", "moe_forward_noalloc", "moe_forward_status",
           "moe_finalize", "moe_quantize",
           "moe_workspace_view", "moe_stage_timing", "moe_stage_times", "moe_last_error"]


def lib_path() -> str:
    return _LIB_PATH


def _check(rc: int):
    if rc != 0:
        raise MoeError(rc, _lib.moe_last_error().decode())


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtype, shape=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclass(frozen=True)
class Dims:
    E: int
    H: int
    I: int
    act: str = "swiglu"
    wfmt: str = "nvfp4"

    @property
    def N1(self) -> int:
        return 2 * self.I if self.act == "swiglu" else self.I

    def c(self) -> _Dims:
        return _Dims(self.E, self.H, self.I, ACTS[self.act], WFMTS[self.wfmt])


def prepared_bytes(d: Dims) -> int:
    n = _lib.moe_prepared_bytes(ctypes.byref(d.c()))
    if n == 0:
        raise MoeError(1, _lib.moe_last_error().decode())
    return n


def prepare_weights(d: Dims, w1: torch.Tensor, w2: torch.Tensor, out=None, stream=None):
    """Quantize and reorder checkpoint-layout weights W1 [E, N1, H], W2 [E, H, I]
    (fp32, on the GPU) into a prepared blob (uint8 tensor on the same GPU)."""
    _need(w1, "w1", torch.float32, (d.E, d.N1, d.H))
    _need(w2, "w2", torch.float32, (d.E, d.H, d.I), w1.device)
    n = prepared_bytes(d)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w1.device)
    _need(out, "out", torch.uint8, device=w1.device)
    _check(_lib.moe_prepare_weights(ctypes.byref(d.c()), _ptr(w1), _ptr(w2), _ptr(out),
                                    out.numel(), ctypes.c_void_p(_stream(stream))))
    return out


def check_prepared(d: Dims, blob: torch.Tensor, stream=None):
    _check(_lib.moe_check_prepared(ctypes.byref(d.c()), _ptr(blob),
                                   ctypes.c_void_p(_stream(stream))))


def workspace_bytes(d: Dims, T: int, K: int, mode: str) -> int:
    n = _lib.moe_workspace_bytes(ctypes.byref(d.c()), T, K, MODES[mode])
    if n == 0:
        raise MoeError(1, _lib.moe_last_error().decode())
    return n


def forward(d: Dims, blob: torch.Tensor, x: torch.Tensor, logits: torch.Tensor, K: int,
            mode: str, router_weight_on_input: bool = False, deterministic: bool = True,
            workspace=None, out=None, stream=None) -> torch.Tensor:
    """One MoE layer forward. x [T, H] bf16, logits [T, E] fp32; returns y [T, H]
    bf16. The workspace (uint8, see workspace_bytes) may be passed in to be
    reused and inspected with workspace_view."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != d.H:
        raise ValueError(f"x must be [T, {d.H}], got {tuple(x.shape)}")
    T = x.shape[0]
    _need(logits, "router_logits", torch.float32, (T, d.E), x.device)
    _need(blob, "prepared", torch.uint8, device=x.device)
    if blob.numel() < prepared_bytes(d):
        raise MoeError(3, f"prepared blob has {blob.numel()} bytes, {prepared_bytes(d)} needed "
                          "for these dimensions")
    if workspace is None:
        workspace = torch.empty(workspace_bytes(d, T, K, mode), dtype=torch.uint8,
                                device=x.device)
    _need(workspace, "workspace", torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, d.H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (T, d.H), x.device)
    _check(_lib.moe_forward(ctypes.byref(d.c()), _ptr(blob), blob.numel(), _ptr(x), _ptr(logits), T, K,
                            MODES[mode], ACTS[d.act], int(bool(router_weight_on_input)),
                            int(bool(deterministic)), _ptr(workspace), workspace.numel(),
                            _ptr(out), ctypes.c_void_p(_stream(stream))))
    return out


def forward_noalloc(d: Dims, blob: torch.Tensor, x: torch.Tensor, logits: torch.Tensor, K: int,
                    mode: str, router_weight_on_input: bool = False, deterministic: bool = True,
                    out=None, stream=None) -> torch.Tensor:
    """forward() on the library's built-in workspace (moe_forward_noalloc): no
    workspace argument and no device allocation by the library. Forwards that
    overlap in time on one GPU share that workspace and must not be run
    concurrently. `out` (y, [T, H] bf16) is allocated here when not given."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != d.H:
        raise ValueError(f"x must be [T, {d.H}], got {tuple(x.shape)}")
    T = x.shape[0]
    _need(logits, "router_logits", torch.float32, (T, d.E), x.device)
    _need(blob, "prepared", torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, d.H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (T, d.H), x.device)
    _check(_lib.moe_forward_noalloc(ctypes.byref(d.c()), _ptr(blob), blob.numel(), _ptr(x),
                                    _ptr(logits), T, K, MODES[mode], ACTS[d.act],
                                    int(bool(router_weight_on_input)), int(bool(deterministic)),
                                    _ptr(out), ctypes.c_void_p(_stream(stream))))
    return out


def forward_status(workspace: torch.Tensor, stream=None) -> int:
    """Status word of the last forward on `workspace` (synchronises): 0, or
    MOE_ERR_INVALID (1) when the blob's header did not match the call."""
    _need(workspace, "workspace", torch.uint8)
    st = ctypes.c_int32(-1)
    _check(_lib.moe_forward_status(_ptr(workspace), ctypes.byref(st),
                                   ctypes.c_void_p(_stream(stream))))
    return st.value


def finalize(permuted_out: torch.Tensor, route_to_row: torch.Tensor, weights, T: int, K: int,
             out=None, stream=None) -> torch.Tensor:
    """Unfused finalize: y[t] = sum_k w[t, k] * permuted_out[route_to_row[t*K + k]]."""
    if permuted_out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("permuted_out must be float32 or bfloat16")
    _need(permuted_out, "permuted_out", permuted_out.dtype)
    R, H = permuted_out.shape
    if R != T * K:
        raise ValueError(f"permuted_out has {R} rows, expected T*K = {T * K}")
    _need(route_to_row, "route_to_row", torch.int32, (T * K,), permuted_out.device)
    if weights is not None:
        _need(weights, "weights", torch.float32, (T, K), permuted_out.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=permuted_out.device)
    _need(out, "out", torch.bfloat16, (T, H), permuted_out.device)
    _check(_lib.moe_finalize(_ptr(permuted_out), int(permuted_out.dtype == torch.bfloat16),
                             _ptr(route_to_row), _ptr(weights), T, K, H, _ptr(out),
                             ctypes.c_void_p(_stream(stream))))
    return out


def quantize(v: torch.Tensor, kind: str, stream=None):
    """Block-quantize an fp32 [rows, cols] matrix. kind: "nvfp4_tensor",
    "nvfp4_row", "mxfp8" or "nvfp4_row_4o6". Returns (codes, scales, g) as uint8/uint8/fp32
    tensors (g is None for MXFP8)."""
    _need(v, "v", torch.float32)
    rows, cols = v.shape
    k = {"nvfp4_tensor": 0, "nvfp4_row": 1, "mxfp8": 2, "nvfp4_row_4o6": 3}[kind]
    dev = v.device
    if k == 2:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        g = None
    else:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        g = torch.empty((1 if k == 0 else rows,), dtype=torch.float32, device=dev)
    scratch = torch.empty(256, dtype=torch.uint8, device=dev)
    _check(_lib.moe_quantize(_ptr(v), rows, cols, k, _ptr(codes), _ptr(scales), _ptr(g),
                             _ptr(scratch), ctypes.c_void_p(_stream(stream))))
    return codes, scales, g


_VIEW_DTYPES = {0: torch.int32, 1: torch.float32, 2: torch.int32, 3: torch.int32,
                4: torch.int32, 5: torch.int32, 6: torch.uint8, 7: torch.uint8,
                8: torch.float32, 10: torch.uint8, 11: torch.uint8, 12: torch.float32,
                13: torch.float32, 14: torch.uint8, 15: torch.uint8, 16: torch.uint8, 17: torch.uint8}


def workspace_view(d: Dims, workspace: torch.Tensor, T: int, K: int, mode: str, view: str):
    """A typed, flat view into the workspace after a forward (no copy)."""
    vid = VIEWS[view]
    off, nbytes = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.moe_workspace_view(ctypes.byref(d.c()), T, K, MODES[mode], vid,
                                   ctypes.byref(off), ctypes.byref(nbytes)))
    raw = workspace[off.value: off.value + nbytes.value]
    if vid == 9:
        dt = torch.bfloat16 if mode == "w4a16" else torch.float32
    else:
        dt = _VIEW_DTYPES[vid]
    return raw.view(dt)


def stage_timing(enable: bool):
    _check(_lib.moe_stage_timing(int(enable)))


def stage_times():
    """(dict stage -> summed ms, number of forwards) since the last call."""
    ms = (ctypes.c_float * len(STAGES))()
    n = ctypes.c_int32(0)
    _check(_lib.moe_stage_times(ms, len(STAGES), ctypes.byref(n)))
    return {s: ms[i] for i, s in enumerate(STAGES)}, n.value
