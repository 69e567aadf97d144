"""learnable_butterfly_rotation_amd -- MI355X (gfx950) learnable butterfly
rotation fused with round-to-nearest group quantization.

Thin ctypes binding over the C ABI of ``libbfly.so`` (include/bfly.h).  The
functions carry the C names; they only marshal torch tensors into pointers,
sizes and the current HIP stream -- every step of the computation runs in the
library's HIP kernels.  There is no CPU fallback: if the library is missing
or no GPU is present the calls raise.

Build the library with ``python -m learnable_butterfly_rotation_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "BflyError", "lib", "library_path", "BFLY_F32", "BFLY_BF16", "BFLY_SYM_ABSMAX",
    "BFLY_ASYM_MINMAX", "bfly_coeff_bytes", "bfly_forward_workspace_bytes", "bfly_prepare",
    "bfly_prepare_hadamard",
    "bfly_forward", "bfly_forward_quant", "bfly_kron_forward", "bfly_kron_forward_wide",
    "bfly_kron_forward_wide_workspace_bytes", "bfly_quant_matmul",
    "bfly_backward", "bfly_backward_workspace_bytes", "bfly_kron_backward",
    "bfly_kron_backward_workspace_bytes", "bfly_calib_config", "bfly_calib_step",
    "bfly_calib_workspace_bytes", "bfly_calib_weight_config", "bfly_calib_step_weight",
    "bfly_calib_step_weight_workspace_bytes", "bfly_status_string",
    "bfly_last_hip_error", "bfly_time_next_forward", "bfly_forward_quant_noalloc",
]

BFLY_F32 = 0
BFLY_BF16 = 1
BFLY_SYM_ABSMAX = 0
BFLY_ASYM_MINMAX = 1

STATUS_NAMES = {0: "BFLY_OK", 1: "BFLY_ERR_NULL", 2: "BFLY_ERR_SIZE", 3: "BFLY_ERR_DTYPE",
                4: "BFLY_ERR_ALIGN", 5: "BFLY_ERR_QUANT", 6: "BFLY_ERR_WORKSPACE",
                7: "BFLY_ERR_UNSUPPORTED", 8: "BFLY_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libbfly.so")
_lib = None


class BflyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s: %s (%s)" % (where, STATUS_NAMES.get(status, status), bfly_status_string(status))
        if status == 8:
            msg += ", hipError %d" % bfly_last_hip_error()
        super().__init__(msg)


def lib():
    """The loaded libbfly.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError("libbfly.so is not built: run "
                               "`python -m learnable_butterfly_rotation_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.bfly_coeff_bytes.argtypes = [i32]
        L.bfly_coeff_bytes.restype = sz
        L.bfly_forward_workspace_bytes.argtypes = [i64, i32]
        L.bfly_forward_workspace_bytes.restype = sz
        L.bfly_prepare.argtypes = [vp, i32, vp, sz, vp]
        L.bfly_prepare_hadamard.argtypes = [i32, vp, sz, vp]
        L.bfly_forward.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i32, vp, vp, vp, sz,
                                   vp]
        L.bfly_forward_quant.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, i64, i32,
                                         vp, vp, i32, i32, ctypes.c_int, vp, sz, vp]
        L.bfly_forward_quant_noalloc.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp,
                                                 i64, i32, vp, i32, i32, ctypes.c_int, vp]
        L.bfly_kron_forward.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, i64, i32,
                                        i32, vp, vp, vp, i32, i32, ctypes.c_int, vp, sz, vp]
        L.bfly_kron_forward_wide.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, i64,
                                             i32, i32, vp, vp, vp, i32, i32, ctypes.c_int, vp, sz,
                                             vp]
        L.bfly_kron_forward_wide_workspace_bytes.argtypes = [i64, i32, i32]
        L.bfly_kron_forward_wide_workspace_bytes.restype = sz
        L.bfly_quant_matmul.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, i64, i32,
                                        i32, i32, i32, ctypes.c_int, vp]
        L.bfly_backward.argtypes = [vp, vp, vp, vp, vp, i64, i32, vp, vp, vp, sz, vp]
        L.bfly_backward_workspace_bytes.argtypes = [i64, i32]
        L.bfly_backward_workspace_bytes.restype = sz
        L.bfly_calib_step.argtypes = [vp, i64, i32, vp, vp, vp, i32,
                                      ctypes.POINTER(bfly_calib_config), vp, vp, sz, vp]
        L.bfly_calib_workspace_bytes.argtypes = [i64, i32]
        L.bfly_calib_workspace_bytes.restype = sz
        L.bfly_calib_step_weight.argtypes = [vp, i64, vp, ctypes.c_int, i32, i32, vp, vp, vp, i32,
                                             ctypes.POINTER(bfly_calib_weight_config), vp, vp, sz,
                                             vp]
        L.bfly_calib_step_weight_workspace_bytes.argtypes = [i64, i32, i32]
        L.bfly_calib_step_weight_workspace_bytes.restype = sz
        L.bfly_kron_backward.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp, vp, vp, vp, sz, vp]
        L.bfly_kron_backward_workspace_bytes.argtypes = [i64, i32, i32]
        L.bfly_kron_backward_workspace_bytes.restype = sz
        L.bfly_status_string.argtypes = [ctypes.c_int]
        L.bfly_status_string.restype = ctypes.c_char_p
        L.bfly_last_hip_error.restype = i32
        L.bfly_time_next_forward.argtypes = [vp, vp]
        for f in (L.bfly_prepare, L.bfly_prepare_hadamard, L.bfly_forward, L.bfly_forward_quant,
                  L.bfly_forward_quant_noalloc,
                  L.bfly_kron_forward, L.bfly_kron_forward_wide, L.bfly_quant_matmul,
                  L.bfly_backward,
                  L.bfly_kron_backward, L.bfly_calib_step, L.bfly_calib_step_weight,
                  L.bfly_time_next_forward):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

class bfly_calib_config(ctypes.Structure):
    """Settings of bfly_calib_step (include/bfly.h)."""
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("bins", ctypes.c_int32),
                ("lambda_kl", ctypes.c_float), ("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float)]


class bfly_calib_weight_config(ctypes.Structure):
    """Settings of bfly_calib_step_weight (include/bfly.h)."""
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("bins", ctypes.c_int32), ("lambda_kl", ctypes.c_float), ("lr", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float)]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return BFLY_F32
    if t.dtype == torch.bfloat16:
        return BFLY_BF16
    raise TypeError("libbfly takes float32 or bfloat16 rows, got %s" % t.dtype)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status, where):
    if status != 0:
        raise BflyError(status, where)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _table_ws(n, theta, coeffs, workspace, like):
    """The workspace of a forward call: the caller's, or -- when the call
    needs one (angles without a table; n = 8192 always) and none is given --
    a fresh uint8 tensor of bfly_forward_workspace_bytes(rows, n) from
    torch's allocator on the device of `like` (torch supplies the device
    memory; the library allocates none)."""
    if workspace is not None or (n != 8192 and (coeffs is not None or theta is None)):
        return workspace
    import torch
    nbytes = bfly_forward_workspace_bytes(like.shape[0], n)
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=like.device)


# ---------------------------------------------------------------------------
# the C ABI, one function per entry point
# ---------------------------------------------------------------------------

def bfly_coeff_bytes(n: int) -> int:
    return lib().bfly_coeff_bytes(n)


def bfly_forward_workspace_bytes(rows: int, n: int) -> int:
    return lib().bfly_forward_workspace_bytes(rows, n)


def bfly_prepare(theta, n: int, coeffs, stream=None) -> None:
    """coeffs (uint8 tensor of >= bfly_coeff_bytes(n) bytes) <- table of theta."""
    _check(lib().bfly_prepare(_ptr(theta), n, _ptr(coeffs), coeffs.numel() * coeffs.element_size(),
                              _stream(stream)), "bfly_prepare")


def bfly_prepare_hadamard(n: int, coeffs, stream=None) -> None:
    """coeffs <- table of H_n = Q(pi/4) D, the orthonormal Walsh-Hadamard matrix."""
    _check(lib().bfly_prepare_hadamard(n, _ptr(coeffs), coeffs.numel() * coeffs.element_size(),
                                       _stream(stream)), "bfly_prepare_hadamard")


def bfly_forward(x, y, theta=None, coeffs=None, workspace=None, stream=None) -> None:
    """y[r] = Q(theta) x[r]; x, y: [rows, n] float32/bfloat16 on the GPU."""
    rows, n = x.shape
    ws = _table_ws(n, theta, coeffs, workspace, x)
    _check(lib().bfly_forward(_ptr(x), _dt(x), _ptr(y), _dt(y), rows, n, _ptr(theta),
                              _ptr(coeffs), _ptr(ws), _nbytes(ws), _stream(stream)),
           "bfly_forward")


def bfly_forward_quant(x, y, codes, scales, zeros=None, theta=None, coeffs=None, bits=4,
                       group=128, mode=BFLY_SYM_ABSMAX, workspace=None, stream=None) -> None:
    """Forward fused with per-group RTN quantization (y may be None)."""
    rows, n = x.shape
    ws = _table_ws(n, theta, coeffs, workspace, x)
    _check(lib().bfly_forward_quant(_ptr(x), _dt(x), _ptr(y), _dt(y) if y is not None else 0,
                                    _ptr(codes), _ptr(scales), _ptr(zeros), rows, n, _ptr(theta),
                                    _ptr(coeffs), bits, group, mode, _ptr(ws), _nbytes(ws),
                                    _stream(stream)),
           "bfly_forward_quant")


def bfly_forward_quant_noalloc(x, y, codes, scales, zeros=None, theta=None, bits=4, group=128,
                               mode=BFLY_SYM_ABSMAX, stream=None) -> None:
    """bfly_forward_quant from angles, its table in the library's fixed
    per-device scratch (no allocation; overlapping calls on one device race)."""
    rows, n = x.shape
    _check(lib().bfly_forward_quant_noalloc(_ptr(x), _dt(x), _ptr(y),
                                            _dt(y) if y is not None else 0, _ptr(codes),
                                            _ptr(scales), _ptr(zeros), rows, n, _ptr(theta), bits,
                                            group, mode, _stream(stream)),
           "bfly_forward_quant_noalloc")


def bfly_kron_forward(x, y, mix, codes=None, scales=None, zeros=None, theta_b=None, coeffs_b=None,
                      bits=4, group=128, mode=BFLY_SYM_ABSMAX, workspace=None, stream=None) -> None:
    """(O kron B) on rows of n = m * nb; mix: [m, m] float32 on the GPU."""
    rows, n = x.shape
    m = mix.shape[0]
    ws = _table_ws(n // m, theta_b, coeffs_b, workspace, x)
    _check(lib().bfly_kron_forward(_ptr(x), _dt(x), _ptr(y), _dt(y) if y is not None else 0,
                                   _ptr(codes), _ptr(scales), _ptr(zeros), rows, m, n // m,
                                   _ptr(theta_b), _ptr(coeffs_b), _ptr(mix), bits, group, mode,
                                   _ptr(ws), _nbytes(ws), _stream(stream)), "bfly_kron_forward")


def bfly_kron_forward_wide_workspace_bytes(rows: int, m: int, nb: int) -> int:
    return lib().bfly_kron_forward_wide_workspace_bytes(rows, m, nb)


def bfly_kron_forward_wide(x, y, mix, workspace, codes=None, scales=None, zeros=None,
                           theta_b=None, coeffs_b=None, bits=4, group=128,
                           mode=BFLY_SYM_ABSMAX, stream=None) -> None:
    """(O kron B) on rows of n = m * nb for m up to 64 (`workspace`: a uint8
    tensor of bfly_kron_forward_wide_workspace_bytes; bf16 rows with nb = 256
    run in one pass, others in two through the workspace)."""
    rows, n = x.shape
    m = mix.shape[0]
    _check(lib().bfly_kron_forward_wide(
        _ptr(x), _dt(x), _ptr(y), _dt(y) if y is not None else 0, _ptr(codes), _ptr(scales),
        _ptr(zeros), rows, m, n // m, _ptr(theta_b), _ptr(coeffs_b), _ptr(mix), bits, group, mode,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
        "bfly_kron_forward_wide")


def bfly_quant_matmul(a, codes, scales, zeros, y, bits=2, group=128, mode=BFLY_ASYM_MINMAX,
                      stream=None) -> None:
    """y = a w^T with w's rows as group codes; a: [rows, k] bfloat16, codes:
    uint8 [n_out, k*bits/8], scales/zeros: float16 [n_out, k/group]."""
    rows, k = a.shape
    n_out = codes.shape[0]
    _check(lib().bfly_quant_matmul(_ptr(a), _dt(a), _ptr(codes), _ptr(scales), _ptr(zeros),
                                   _ptr(y), _dt(y), rows, n_out, k, bits, group, mode,
                                   _stream(stream)), "bfly_quant_matmul")


def bfly_backward_workspace_bytes(rows: int, n: int) -> int:
    return lib().bfly_backward_workspace_bytes(rows, n)


def bfly_backward(x, g, y, dx, dtheta, workspace, theta=None, coeffs=None, stream=None) -> None:
    """y = Q x (optional), dx = Q^T g, dtheta = sum over rows of dL/dtheta."""
    rows, n = x.shape
    _check(lib().bfly_backward(_ptr(x), _ptr(g), _ptr(y), _ptr(dx), _ptr(dtheta), rows, n,
                               _ptr(theta), _ptr(coeffs), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "bfly_backward")


def bfly_status_string(status: int) -> str:
    return lib().bfly_status_string(status).decode()


def bfly_last_hip_error() -> int:
    return lib().bfly_last_hip_error()


def bfly_time_next_forward(start_event: int, stop_event: int) -> None:
    """Attach two caller-owned hipEvent_t handles (timing enabled) to the
    next fused forward-kernel dispatch, for kernel-only timing."""
    _check(lib().bfly_time_next_forward(start_event, stop_event), "bfly_time_next_forward")


def bfly_kron_backward_workspace_bytes(rows: int, m: int, nb: int) -> int:
    return lib().bfly_kron_backward_workspace_bytes(rows, m, nb)


def bfly_kron_backward(x, g, dx, dtheta_b, mix, workspace, theta_b=None, coeffs_b=None,
                       stream=None) -> None:
    """dx = (O kron B)^T g and dtheta_b (summed over rows and segments);
    x, g, dx: [rows, m*nb] float32; mix: [m, m] float32 on the GPU."""
    rows, n = x.shape
    m = mix.shape[0]
    _check(lib().bfly_kron_backward(_ptr(x), _ptr(g), _ptr(dx), _ptr(dtheta_b), rows, m, n // m,
                                    _ptr(theta_b), _ptr(coeffs_b), _ptr(mix), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "bfly_kron_backward")


def bfly_calib_workspace_bytes(rows: int, n: int) -> int:
    return lib().bfly_calib_workspace_bytes(rows, n)


def bfly_calib_step(x, theta, adam_m, adam_v, step: int, cfg: bfly_calib_config, loss, workspace,
                    stream=None) -> None:
    """One calibration step on rows x ([rows, n] float32): theta, adam_m,
    adam_v ([log2 n, n/2] float32) updated in place; loss [3] float32."""
    rows, n = x.shape
    _check(lib().bfly_calib_step(_ptr(x), rows, n, _ptr(theta), _ptr(adam_m), _ptr(adam_v), step,
                                 ctypes.byref(cfg), _ptr(loss), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "bfly_calib_step")


def bfly_calib_step_weight_workspace_bytes(rows: int, out: int, n: int) -> int:
    return lib().bfly_calib_step_weight_workspace_bytes(rows, out, n)


def bfly_calib_step_weight(x, w, theta, adam_m, adam_v, step: int, cfg: bfly_calib_weight_config,
                           loss, workspace, stream=None) -> None:
    """One calibration step with the layer-output loss: x [rows, n] float32,
    w [out, n] float32/bfloat16; theta, adam_m, adam_v updated in place."""
    rows, n = x.shape
    out = w.shape[0]
    _check(lib().bfly_calib_step_weight(_ptr(x), rows, _ptr(w), _dt(w), out, n, _ptr(theta),
                                        _ptr(adam_m), _ptr(adam_v), step, ctypes.byref(cfg),
                                        _ptr(loss), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "bfly_calib_step_weight")
