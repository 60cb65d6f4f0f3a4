"""Python binding of libforge, the gfx950 fused weight-gradient + optimizer step.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/forge.h``.  PyTorch is used for
device memory and streams; tensors are passed by their device pointers.

The library must have been built (``python backward_weight_gradient_amd/build.py``
or ``__graft_entry__.build()``); importing this package without it raises
``ImportError`` -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

# torch is imported before libforge is loaded so that the library's
# libamdhip64.so.7 dependency resolves to the HIP runtime torch has already
# loaded: one runtime per process, which owns the device pointers and stream
# handles passed in.  Loaded first, libforge would bring up a second runtime
# from the system ROCm install, and that one need not see the device.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libforge.so")

FORGE_OK = 0
STATUS_NAMES = ["FORGE_OK", "FORGE_E_NULL", "FORGE_E_SHAPE", "FORGE_E_DTYPE", "FORGE_E_ALIGN",
                "FORGE_E_STEP", "FORGE_E_HYPER", "FORGE_E_ALIAS", "FORGE_E_UNSUPPORTED", "FORGE_E_HIP",
                "FORGE_E_SCRATCH"]
(FORGE_E_NULL, FORGE_E_SHAPE, FORGE_E_DTYPE, FORGE_E_ALIGN, FORGE_E_STEP, FORGE_E_HYPER,
 FORGE_E_ALIAS, FORGE_E_UNSUPPORTED, FORGE_E_HIP, FORGE_E_SCRATCH) = range(1, 11)
FORGE_DGRAD_SCRATCH_BYTES = 64 << 20   # the static scratch of forge_dgrad_split_noalloc
FORGE_QUOTIENT_COUNTS = 2048 * 8       # counters written by forge_debug_quotients

FORGE_F32, FORGE_BF16, FORGE_S8, FORGE_U8, FORGE_E4M3 = 0, 1, 2, 3, 4
FORGE_ADAMW, FORGE_LION, FORGE_SGDM, FORGE_NADAM, FORGE_RADAM, FORGE_RMSPROP, FORGE_ADAGRAD, FORGE_SGD = range(8)
FORGE_ROUND_RNE, FORGE_ROUND_SR = 0, 1
OPTIMIZERS = {"adamw": FORGE_ADAMW, "lion": FORGE_LION, "sgdm": FORGE_SGDM, "nadam": FORGE_NADAM,
              "radam": FORGE_RADAM, "rmsprop": FORGE_RMSPROP, "adagrad": FORGE_ADAGRAD, "sgd": FORGE_SGD}
# which states each optimizer keeps (m: first moment / momentum, v: second moment)
KEEPS_M = {"adamw", "lion", "sgdm", "nadam", "radam"}
KEEPS_V = {"adamw", "nadam", "radam", "rmsprop", "adagrad"}
ROUNDING = {"rne": FORGE_ROUND_RNE, "sr": FORGE_ROUND_SR}


class ForgeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = f" [{forge_last_error()}]" if code == FORGE_E_HIP else ""
        super().__init__(f"{where}: {forge_status_str(code)} (code {code}){detail}")


class forge_mat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64)]


class forge_state(ctypes.Structure):
    _fields_ = [("q", forge_mat), ("scale", ctypes.c_void_p), ("block", ctypes.c_int32)]


class forge_hyper(ctypes.Structure):
    _fields_ = [("opt", ctypes.c_int32), ("round", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


FORGE_GROUP_MAX = 8


class forge_layer(ctypes.Structure):
    _fields_ = [("X", ctypes.POINTER(forge_mat)), ("dY", ctypes.POINTER(forge_mat)), ("W", ctypes.POINTER(forge_mat)),
                ("m", ctypes.POINTER(forge_state)), ("v", ctypes.POINTER(forge_state)), ("seed", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libforge.so is not built ({LIB_PATH}); run "
                          "`python backward_weight_gradient_amd/build.py` first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    st = ctypes.c_int
    lib.forge_wgrad_step.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), P(forge_state), P(forge_state),
                                     P(forge_hyper), ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p]
    lib.forge_wgrad_step.restype = st
    lib.forge_wgrad_check.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), P(forge_state), P(forge_state),
                                      P(forge_hyper), ctypes.c_int64]
    lib.forge_wgrad_check.restype = st
    lib.forge_wgrad_unfused.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), P(forge_state), P(forge_state),
                                        P(forge_hyper), ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p]
    lib.forge_wgrad_unfused.restype = st
    lib.forge_debug_sr_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    lib.forge_debug_sr_bf16.restype = st
    lib.forge_wgrad_step_group.argtypes = [P(forge_layer), ctypes.c_int32, P(forge_hyper), ctypes.c_int64,
                                           ctypes.c_void_p]
    lib.forge_wgrad_step_group.restype = st
    lib.forge_wgrad_accumulate.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), ctypes.c_int32, ctypes.c_void_p]
    lib.forge_wgrad_accumulate.restype = st
    lib.forge_wgrad_step_accumulated.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), P(forge_mat),
                                                 P(forge_state), P(forge_state), P(forge_hyper), ctypes.c_int64,
                                                 ctypes.c_uint64, ctypes.c_void_p]
    lib.forge_wgrad_step_accumulated.restype = st
    lib.forge_dgrad.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), ctypes.c_void_p]
    lib.forge_dgrad.restype = st
    lib.forge_dgrad_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.forge_dgrad_workspace_bytes.restype = ctypes.c_int64
    lib.forge_dgrad_split.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    lib.forge_dgrad_split.restype = st
    lib.forge_wgrad_step_fp8w.argtypes = [P(forge_mat), P(forge_mat), P(forge_state), P(forge_state),
                                          P(forge_state), P(forge_hyper), ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_void_p]
    lib.forge_wgrad_step_fp8w.restype = st
    lib.forge_wgrad_check_fp8w.argtypes = [P(forge_mat), P(forge_mat), P(forge_state), P(forge_state),
                                           P(forge_state), P(forge_hyper), ctypes.c_int64]
    lib.forge_wgrad_check_fp8w.restype = st
    lib.forge_dgrad_fp8w.argtypes = [P(forge_mat), P(forge_state), P(forge_mat), ctypes.c_void_p]
    lib.forge_dgrad_fp8w.restype = st
    lib.forge_dgrad_split_noalloc.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), ctypes.c_void_p]
    lib.forge_dgrad_split_noalloc.restype = st
    lib.forge_backward_step.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), P(forge_state), P(forge_state),
                                        P(forge_hyper), ctypes.c_int64, ctypes.c_uint64, P(forge_mat),
                                        ctypes.c_void_p]
    lib.forge_backward_step.restype = st
    lib.forge_backward_step_split.argtypes = [P(forge_mat), P(forge_mat), P(forge_mat), P(forge_state),
                                              P(forge_state), P(forge_hyper), ctypes.c_int64, ctypes.c_uint64,
                                              P(forge_mat), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.forge_backward_step_split.restype = st
    lib.forge_debug_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.forge_debug_e4m3.restype = st
    lib.forge_debug_e4m3_sr.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_int64, ctypes.c_void_p]
    lib.forge_debug_e4m3_sr.restype = st
    lib.forge_debug_quotients.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.forge_debug_quotients.restype = st
    lib.forge_debug_quant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.forge_debug_quant.restype = st
    lib.forge_debug_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.forge_debug_copy.restype = st
    lib.forge_debug_state_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_void_p]
    lib.forge_debug_state_stream.restype = st
    lib.forge_debug_mfma_peak.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.forge_debug_mfma_peak.restype = st
    lib.forge_status_str.argtypes = [ctypes.c_int]
    lib.forge_status_str.restype = ctypes.c_char_p
    lib.forge_version.argtypes = []
    lib.forge_version.restype = ctypes.c_char_p
    lib.forge_last_error.argtypes = []
    lib.forge_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


# ---------------------------------------------------------------------------
# Struct builders
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FORGE_F32, torch.bfloat16: FORGE_BF16, torch.int8: FORGE_S8, torch.uint8: FORGE_U8,
             torch.float8_e4m3fn: FORGE_E4M3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def mat_raw(ptr: int, dtype: int, rows: int, cols: int, ld: Optional[int] = None) -> forge_mat:
    """A forge_mat from a raw device address (no tensor)."""
    return forge_mat(ptr or None, dtype, rows, cols, cols if ld is None else ld)


def mat(t) -> forge_mat:
    """A forge_mat describing a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    ld = t.stride(0) if t.shape[0] > 1 else max(1, t.shape[1])
    return forge_mat(t.data_ptr() or None, _dtype_code(t), t.shape[0], t.shape[1], ld)


def state(t, scale=None, block: int = 0) -> forge_state:
    """A forge_state: values (f32 / bf16), or 8-bit codes (int8 / uint8 / E4M3)
    plus fp32 block scales.  The scale tensor must be float32, contiguous, on
    t's device, with rows * cols / block elements, block in {32, 64, 128}:
    the kernels read and write exactly that many scales through its pointer."""
    if scale is None:
        return forge_state(mat(t), None, 0)
    if block not in (32, 64, 128):
        raise ValueError(f"state: block must be 32, 64 or 128, got {block}")
    if t.dim() != 2 or t.shape[1] % block:
        raise ValueError("state: the code tensor must be 2-D with cols a multiple of the block")
    if scale.dtype != torch.float32 or not scale.is_contiguous() or scale.device != t.device:
        raise ValueError("state: the scale tensor must be contiguous float32 on the codes' device")
    if scale.numel() != t.shape[0] * (t.shape[1] // block):
        raise ValueError(f"state: {scale.numel()} scales given, {t.shape[0] * (t.shape[1] // block)} needed")
    return forge_state(mat(t), scale.data_ptr() or None, block)


def hyper(opt: str = "adamw", lr: float = 1e-3, beta1: float = 0.9, beta2: Optional[float] = None,
          eps: Optional[float] = None, weight_decay: float = 0.01, round: str = "sr") -> forge_hyper:
    """Hyper-parameters; beta2 defaults to 0.99 for RMSprop (its smoothing constant) and 0.999
    otherwise, eps to 1e-10 for AdaGrad and 1e-8 otherwise."""
    if beta2 is None:
        beta2 = 0.99 if opt == "rmsprop" else 0.999
    if eps is None:
        eps = 1e-10 if opt == "adagrad" else 1e-8
    return forge_hyper(OPTIMIZERS[opt], ROUNDING[round], lr, beta1, beta2, eps, weight_decay)


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _stream(stream):
    return current_stream() if stream is None else stream


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def forge_status_str(code: int) -> str:
    return lib.forge_status_str(code).decode()


def forge_version() -> str:
    return lib.forge_version().decode()


def forge_last_error() -> str:
    """HIP's description of the error behind the last FORGE_E_HIP on this thread."""
    return lib.forge_last_error().decode()


def forge_wgrad_check(X: forge_mat, dY: forge_mat, W: forge_mat, m: Optional[forge_state],
                      v: Optional[forge_state], h: forge_hyper, step: int) -> int:
    return lib.forge_wgrad_check(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step)


def forge_wgrad_step(X, dY, W, m, v, h: forge_hyper, step: int, seed: int, stream=None, check: bool = True) -> int:
    """Fused dW = dY^T X + optimizer step, in place on W / m / v.

    X, dY, W: tensors or forge_mat; m, v: forge_state (or None for v).
    """
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    rc = lib.forge_wgrad_step(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step, seed, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_wgrad_step")
    return rc


def forge_wgrad_step_group(layers, h: forge_hyper, step: int, stream=None, check: bool = True) -> int:
    """forge_wgrad_step on several independent layers in as few launches as possible.

    layers: sequence of (X, dY, W, m, v, seed) with X, dY, W tensors or forge_mat,
    m, v forge_state or None (m for AdamW, NAdam, RAdam, Lion, SGD-m; v for AdamW,
    NAdam, RAdam, RMSprop, AdaGrad).
    """
    keep = []
    arr = (forge_layer * max(1, len(layers)))()
    for i, (X, dY, W, m, v, seed) in enumerate(layers):
        X = mat(X) if not isinstance(X, forge_mat) else X
        dY = mat(dY) if not isinstance(dY, forge_mat) else dY
        W = mat(W) if not isinstance(W, forge_mat) else W
        keep.append((X, dY, W, m, v))
        arr[i].X = ctypes.pointer(X)
        arr[i].dY = ctypes.pointer(dY)
        arr[i].W = ctypes.pointer(W)
        arr[i].m = ctypes.pointer(m) if m is not None else None
        arr[i].v = ctypes.pointer(v) if v is not None else None
        arr[i].seed = seed
    rc = lib.forge_wgrad_step_group(arr, len(layers), _ref(h), step, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_wgrad_step_group")
    return rc


def forge_wgrad_accumulate(X, dY, acc, first: bool, stream=None, check: bool = True) -> int:
    """One micro-step of exact gradient accumulation: acc = dY^T X (first) or acc += dY^T X (fp32)."""
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    acc = mat(acc) if not isinstance(acc, forge_mat) else acc
    rc = lib.forge_wgrad_accumulate(_ref(X), _ref(dY), _ref(acc), 1 if first else 0, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_wgrad_accumulate")
    return rc


def forge_wgrad_step_accumulated(X, dY, acc, W, m, v, h: forge_hyper, step: int, seed: int, stream=None,
                                 check: bool = True) -> int:
    """Final micro-step: the fused step on G = acc + dY^T X (acc is consumed)."""
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    acc = mat(acc) if not isinstance(acc, forge_mat) else acc
    W = mat(W) if not isinstance(W, forge_mat) else W
    rc = lib.forge_wgrad_step_accumulated(_ref(X), _ref(dY), _ref(acc), _ref(W), _ref(m), _ref(v), _ref(h), step,
                                          seed, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_wgrad_step_accumulated")
    return rc


def forge_dgrad(dY, W, dX, stream=None, check: bool = True) -> int:
    """dX = dY W (the input gradient), fp32 accumulation; dX bf16 (RNE) or f32."""
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    dX = mat(dX) if not isinstance(dX, forge_mat) else dX
    rc = lib.forge_dgrad(_ref(dY), _ref(W), _ref(dX), _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_dgrad")
    return rc


def forge_dgrad_workspace_bytes(BT: int, N: int, K: int) -> int:
    """Bytes of workspace forge_dgrad_split uses for these shapes (0: none)."""
    return int(lib.forge_dgrad_workspace_bytes(BT, N, K))


def forge_dgrad_split(dY, W, dX, workspace=None, stream=None, check: bool = True) -> int:
    """forge_dgrad with the reduction split across workgroups into `workspace`
    (a device tensor of at least forge_dgrad_workspace_bytes bytes, or None)."""
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    dX = mat(dX) if not isinstance(dX, forge_mat) else dX
    if workspace is None:
        ptr, nbytes = None, 0
    else:
        ptr, nbytes = workspace.data_ptr() or None, workspace.numel() * workspace.element_size()
    rc = lib.forge_dgrad_split(_ref(dY), _ref(W), _ref(dX), ptr, nbytes, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_dgrad_split")
    return rc


def forge_wgrad_step_fp8w(X, dY, W: forge_state, m, v, h: forge_hyper, step: int, seed: int, stream=None,
                          check: bool = True) -> int:
    """forge_wgrad_step with an E4M3 weight (W: forge_state of E4M3 codes and
    block scales, updated in place)."""
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    rc = lib.forge_wgrad_step_fp8w(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step, seed,
                                   _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_wgrad_step_fp8w")
    return rc


def forge_wgrad_check_fp8w(X: forge_mat, dY: forge_mat, W: forge_state, m, v, h: forge_hyper, step: int) -> int:
    return lib.forge_wgrad_check_fp8w(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step)


def forge_dgrad_fp8w(dY, W: forge_state, dX, stream=None, check: bool = True) -> int:
    """dX = dY W from an E4M3 weight with block scales (decoded exactly)."""
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    dX = mat(dX) if not isinstance(dX, forge_mat) else dX
    rc = lib.forge_dgrad_fp8w(_ref(dY), _ref(W), _ref(dX), _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_dgrad_fp8w")
    return rc


def forge_dgrad_split_noalloc(dY, W, dX, stream=None, check: bool = True) -> int:
    """forge_dgrad_split with its partial sums in the library's static per-device
    scratch array (no workspace, no allocation; overlapping calls on one GPU race)."""
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    dX = mat(dX) if not isinstance(dX, forge_mat) else dX
    rc = lib.forge_dgrad_split_noalloc(_ref(dY), _ref(W), _ref(dX), _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_dgrad_split_noalloc")
    return rc


def forge_backward_step(X, dY, W, m, v, h: forge_hyper, step: int, seed: int, dX, stream=None,
                        check: bool = True) -> int:
    """dX = dY W from the current W, then the fused weight-gradient step, in that order."""
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    dX = mat(dX) if not isinstance(dX, forge_mat) else dX
    rc = lib.forge_backward_step(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step, seed, _ref(dX),
                                 _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_backward_step")
    return rc


def forge_backward_step_split(X, dY, W, m, v, h: forge_hyper, step: int, seed: int, dX, workspace=None,
                              stream=None, check: bool = True) -> int:
    """forge_backward_step with dX from the split kernel (workspace: a device tensor
    of at least forge_dgrad_workspace_bytes bytes, or None)."""
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    dX = mat(dX) if not isinstance(dX, forge_mat) else dX
    if workspace is None:
        ptr, nbytes = None, 0
    else:
        ptr, nbytes = workspace.data_ptr() or None, workspace.numel() * workspace.element_size()
    rc = lib.forge_backward_step_split(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step, seed, _ref(dX),
                                       ptr, nbytes, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_backward_step_split")
    return rc


def forge_wgrad_unfused(X, dY, W, m, v, h: forge_hyper, step: int, seed: int, dW, stream=None,
                        check: bool = True) -> int:
    """Unfused baseline: G -> dW (the tensor's dtype, f32 or bf16), then the step."""
    X = mat(X) if not isinstance(X, forge_mat) else X
    dY = mat(dY) if not isinstance(dY, forge_mat) else dY
    W = mat(W) if not isinstance(W, forge_mat) else W
    rc = lib.forge_wgrad_unfused(_ref(X), _ref(dY), _ref(W), _ref(m), _ref(v), _ref(h), step, seed,
                                 dW.data_ptr(), _dtype_code(dW), _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_wgrad_unfused")
    return rc


def forge_debug_e4m3(inp, out, stream=None, check: bool = True) -> int:
    """E4M3 rounding of a float32 tensor into a uint8 code tensor (test hook)."""
    rc = lib.forge_debug_e4m3(inp.data_ptr(), out.data_ptr(), inp.numel(), _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_e4m3")
    return rc


def forge_debug_e4m3_sr(inp, out, seed: int, step: int, stream=None, check: bool = True) -> int:
    """The FP8 weight store's stochastic rounding of a float32 tensor into a
    uint8 code tensor, element i with the SR bits of flat index i (test hook)."""
    if out.numel() != inp.numel() or out.element_size() != 1:
        raise ValueError("forge_debug_e4m3_sr: out must be a 1-byte tensor with inp's element count")
    rc = lib.forge_debug_e4m3_sr(inp.data_ptr(), out.data_ptr(), inp.numel(), seed & (2**64 - 1), step,
                                 _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_e4m3_sr")
    return rc


def forge_debug_quotients(counts, stream=None, check: bool = True) -> int:
    """Exhaustive check of the quantiser's fast scale / reciprocal quotients
    against IEEE division (test hook); counts: int64 device tensor of
    FORGE_QUOTIENT_COUNTS elements (see forge.h for the layout)."""
    if counts.numel() != FORGE_QUOTIENT_COUNTS or counts.element_size() != 8 or not counts.is_contiguous():
        raise ValueError("forge_debug_quotients: counts must be a contiguous 8-byte tensor of "
                         "FORGE_QUOTIENT_COUNTS elements")
    rc = lib.forge_debug_quotients(counts.data_ptr(), _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_quotients")
    return rc


def forge_debug_quant(inp, codes, scales, dtype: int, second_moment: bool, block: int, stream=None,
                      check: bool = True) -> int:
    """The epilogue's 8-bit block quantiser on a 2-D float32 tensor (test hook):
    codes (int8 / uint8 / float8_e4m3fn, same shape) and fp32 scales
    [rows, cols / block] are written; dtype FORGE_S8, FORGE_U8 or FORGE_E4M3."""
    if inp.dim() != 2 or not inp.is_contiguous() or inp.dtype != torch.float32:
        raise ValueError("forge_debug_quant: inp must be a contiguous 2-D float32 tensor")
    rows, cols = inp.shape
    if codes.shape != inp.shape or not codes.is_contiguous() or codes.element_size() != 1:
        raise ValueError("forge_debug_quant: codes must be a contiguous 1-byte tensor of inp's shape")
    if scales.dtype != torch.float32 or not scales.is_contiguous() or \
            (block > 0 and scales.numel() != rows * (cols // block)):
        raise ValueError("forge_debug_quant: scales must be contiguous float32 with rows * cols / block elements")
    rc = lib.forge_debug_quant(inp.data_ptr() or None, codes.data_ptr() or None, scales.data_ptr() or None,
                               rows, cols, dtype, 1 if second_moment else 0, block, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_quant")
    return rc


def forge_debug_copy(src, dst, stream=None, check: bool = True) -> int:
    """dst = src through the streaming-ceiling copy kernel (measurement hook)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("forge_debug_copy: src and dst sizes differ")
    rc = lib.forge_debug_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_copy")
    return rc


def forge_debug_state_stream(W, m, v, stream=None, check: bool = True) -> int:
    """The epilogue-shaped W (bf16) / m / v (fp32) read-and-write stream (measurement hook)."""
    N, K = W.shape
    if W.dtype != torch.bfloat16 or m.dtype != torch.float32 or v.dtype != torch.float32 or \
            m.shape != W.shape or v.shape != W.shape or not (W.is_contiguous() and m.is_contiguous()
                                                              and v.is_contiguous()):
        raise ValueError("forge_debug_state_stream: W bf16, m and v float32, contiguous, of one shape")
    rc = lib.forge_debug_state_stream(W.data_ptr(), m.data_ptr(), v.data_ptr(), N, K, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_state_stream")
    return rc


def forge_debug_mfma_peak(out, blocks: int, iters: int, stream=None, check: bool = True) -> int:
    """The matrix-core ceiling loop; `out` holds at least 256 * blocks floats (measurement hook)."""
    if out.numel() < 256 * blocks or out.dtype != torch.float32:
        raise ValueError("forge_debug_mfma_peak: out must be float32 with 256 * blocks elements")
    rc = lib.forge_debug_mfma_peak(out.data_ptr(), blocks, iters, _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_mfma_peak")
    return rc


def forge_debug_sr_bf16(inp, out, seed: int, step: int, tensor_id: int, stream=None, check: bool = True) -> int:
    """Stochastic rounding of a float32 tensor into a bf16 tensor (test hook)."""
    rc = lib.forge_debug_sr_bf16(inp.data_ptr(), out.data_ptr(), inp.numel(), seed, step, tensor_id,
                                 _stream(stream))
    if check and rc != FORGE_OK:
        raise ForgeError(rc, "forge_debug_sr_bf16")
    return rc
