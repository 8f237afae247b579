"""Python binding of libssm.so, the gfx950 selective-scan (S6) library.

Argument marshalling only: every step of the scan and of the decode step runs
in the HIP kernels behind the C ABI declared in ``include/ssm.h``. PyTorch
supplies device memory and the current HIP stream. There is no fallback: if
the library is not built, or a tensor is not on the GPU, the call raises.

Functions (same names as the C ABI):
  ssm_scan_fwd(x, delta, A, Bt, Ct, Dskip=None, z=None, state_in=None,
               state_out=None, y=None, workspace=None) -> y
  ssm_step(x, delta, A, Bt, Ct, state, Dskip=None, z=None, y=None) -> y
  ssm_scan_fwd_noalloc(x, delta, A, Bt, Ct, y, ...) -> y: ssm_scan_fwd with the
      library's static workspace, for callers that cannot allocate
  ssm_scan_fwd_dt / ssm_step_dt: the same with delta_raw and dt_bias in place
      of delta; the kernels use softplus(delta_raw + dt_bias) as the step size
  ssm_scan_fwd_conv(x_raw, conv_w, delta_raw, dt_bias, A, Bt, Ct, conv_b=None,
                    conv_state=None, ...) -> y: ssm_scan_fwd_dt behind the x
      branch of the Mamba block (SiLU of a causal width-4 convolution of x_raw);
      ssm_step_conv, its decode step, shifts conv_state in place
  ssm_scan_fwd_trap / ssm_step_trap: the exponential-trapezoidal rule, with a
      per-token weight lam and the token before the first (x_prev, B_prev)
  ssm_ssd_fwd(x, delta, A, Bt, Ct, Dskip=None, state_in=None, state_out=None,
              y=None) -> y: the Mamba-2 SSD layer (x (batch, L, H, P), Bt/Ct
      (batch, L, G, N), bfloat16)
  ssm_scan_bwd(x, delta, A, Bt, Ct, dy, Dskip=None, z=None, state_in=None,
               dstate=None) -> dict: the gradient of ssm_scan_fwd (dx, ddelta,
      dA, dBt, dCt, dDskip, dz, dstate_in)
  ssm_scan_bwd_dt(x, delta_raw, dt_bias, A, Bt, Ct, dy, ...) -> dict: the same for
      ssm_scan_fwd_dt, with ddelta_raw and ddt_bias in place of ddelta
  ssm_scan_bwd_conv(x_raw, conv_w, delta_raw, dt_bias, A, Bt, Ct, dy, ...) -> dict:
      the same for ssm_scan_fwd_conv, with dx_raw, dconv_w, dconv_b, dconv_state
  ssm_scan_bwd_trap(x, delta, lam, A, Bt, Ct, dy, ...) -> dict: the same for
      ssm_scan_fwd_trap, with dlam, and dx_prev, dB_prev for the earlier token
  ssm_ssd_step(x, delta, A, Bt, Ct, state, Dskip=None, y=None) -> y: one SSD
      decode token (x (batch, H, P), Bt/Ct (batch, G, N), state in place)
  ssm_scan_workspace_bytes(batch, L, D, N, dtype) -> int
  ssm_scan_workspace_status(workspace, stream=None) -> int: SSM_OK, or
      SSM_ERR_TIMEOUT when a wait of the last scan on that workspace gave up
      (waits for the stream)
  ssm_scan_bwd_workspace_bytes(batch, L, D, N, dtype) -> int
  ssm_status_string(status) -> str, ssm_version() -> str
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "SSM_F32", "SSM_BF16", "SSMError", "lib", "lib_path", "ssm_scan_fwd", "ssm_step", "ssm_scan_fwd_dt", "ssm_step_dt",
    "ssm_scan_fwd_conv", "ssm_step_conv", "ssm_scan_bwd_conv",
    "ssm_scan_fwd_trap", "ssm_step_trap", "ssm_ssd_fwd", "ssm_ssd_step", "ssm_scan_bwd", "ssm_scan_bwd_dt", "ssm_scan_bwd_trap", "ssm_scan_workspace_bytes",
    "ssm_scan_bwd_workspace_bytes", "ssm_status_string", "ssm_version", "EXPORTS", "new_workspace",
    "workspace_error", "ssm_scan_workspace_status", "SSM_ERR_TIMEOUT", "ssm_scan_fwd_noalloc",
]

SSM_F32 = 0
SSM_BF16 = 1
STATUS = {0: "SSM_OK", -1: "SSM_ERR_NULL", -2: "SSM_ERR_SHAPE", -3: "SSM_ERR_DTYPE",
          -4: "SSM_ERR_UNSUPPORTED", -5: "SSM_ERR_ALIGN", -6: "SSM_ERR_WORKSPACE", -7: "SSM_ERR_HIP",
          -8: "SSM_ERR_TIMEOUT"}
SSM_ERR_TIMEOUT = -8

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; SSM_LIBRARY names another build of the same ABI (the host
# tests use it to run against a sanitizer build of the argument checks).
lib_path = os.environ.get("SSM_LIBRARY") or os.path.join(_HERE, "libssm.so")

# The functions include/ssm.h declares.
EXPORTS = ("ssm_status_string", "ssm_version", "ssm_scan_workspace_bytes", "ssm_scan_fwd", "ssm_step",
           "ssm_scan_fwd_dt", "ssm_step_dt", "ssm_scan_fwd_trap", "ssm_step_trap", "ssm_ssd_fwd",
           "ssm_scan_bwd_workspace_bytes", "ssm_scan_bwd", "ssm_scan_bwd_dt", "ssm_scan_bwd_trap", "ssm_ssd_step",
           "ssm_scan_workspace_status", "ssm_scan_fwd_noalloc", "ssm_scan_fwd_conv", "ssm_step_conv",
           "ssm_scan_bwd_conv_workspace_bytes", "ssm_scan_bwd_conv")

_lib: Optional[ctypes.CDLL] = None


class SSMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({ssm_status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    L = ctypes.CDLL(lib_path)
    i64, vp, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.ssm_status_string.argtypes = [ci]
    L.ssm_status_string.restype = ctypes.c_char_p
    L.ssm_version.argtypes = []
    L.ssm_version.restype = ctypes.c_char_p
    L.ssm_scan_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    L.ssm_scan_workspace_bytes.restype = sz
    L.ssm_scan_workspace_status.argtypes = [vp, sz, vp]
    L.ssm_scan_workspace_status.restype = ci
    L.ssm_scan_fwd.argtypes = [i64, i64, i64, i64, ci] + [vp] * 10 + [vp, sz, vp]
    L.ssm_scan_fwd.restype = ci
    L.ssm_scan_fwd_noalloc.argtypes = [i64, i64, i64, i64, ci] + [vp] * 10 + [vp]
    L.ssm_scan_fwd_noalloc.restype = ci
    L.ssm_step.argtypes = [i64, i64, i64, ci] + [vp] * 9 + [vp]
    L.ssm_step.restype = ci
    L.ssm_scan_fwd_dt.argtypes = [i64, i64, i64, i64, ci] + [vp] * 11 + [vp, sz, vp]
    L.ssm_scan_fwd_dt.restype = ci
    L.ssm_step_dt.argtypes = [i64, i64, i64, ci] + [vp] * 10 + [vp]
    L.ssm_step_dt.restype = ci
    L.ssm_scan_fwd_conv.argtypes = [i64, i64, i64, i64, ci] + [vp] * 14 + [vp, sz, vp]
    L.ssm_scan_fwd_conv.restype = ci
    L.ssm_scan_fwd_trap.argtypes = [i64, i64, i64, i64, ci] + [vp] * 13 + [vp, sz, vp]
    L.ssm_scan_fwd_trap.restype = ci
    L.ssm_step_conv.argtypes = [i64, i64, i64, ci] + [vp] * 13 + [vp]
    L.ssm_step_conv.restype = ci
    L.ssm_step_trap.argtypes = [i64, i64, i64, ci] + [vp] * 12 + [vp]
    L.ssm_step_trap.restype = ci
    L.ssm_ssd_fwd.argtypes = [i64] * 6 + [ci] + [vp] * 9 + [vp]
    L.ssm_ssd_fwd.restype = ci
    L.ssm_ssd_step.argtypes = [i64] * 5 + [ci] + [vp] * 8 + [vp]
    L.ssm_ssd_step.restype = ci
    L.ssm_scan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    L.ssm_scan_bwd_workspace_bytes.restype = sz
    L.ssm_scan_bwd.argtypes = [i64, i64, i64, i64, ci] + [vp] * 18 + [vp, sz, vp]
    L.ssm_scan_bwd.restype = ci
    L.ssm_scan_bwd_dt.argtypes = [i64, i64, i64, i64, ci] + [vp] * 20 + [vp, sz, vp]
    L.ssm_scan_bwd_dt.restype = ci
    L.ssm_scan_bwd_conv_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    L.ssm_scan_bwd_conv_workspace_bytes.restype = sz
    L.ssm_scan_bwd_conv.argtypes = [i64, i64, i64, i64, ci] + [vp] * 26 + [vp, sz, vp]
    L.ssm_scan_bwd_conv.restype = ci
    L.ssm_scan_bwd_trap.argtypes = [i64, i64, i64, i64, ci] + [vp] * 24 + [vp, sz, vp]
    L.ssm_scan_bwd_trap.restype = ci
    _lib = L
    return L


def ssm_status_string(status: int) -> str:
    return lib().ssm_status_string(int(status)).decode()


def ssm_version() -> str:
    return lib().ssm_version().decode()


def ssm_scan_workspace_bytes(batch: int, L: int, D: int, N: int, dtype: int) -> int:
    return int(lib().ssm_scan_workspace_bytes(batch, L, D, N, dtype))


def ssm_scan_bwd_workspace_bytes(batch: int, L: int, D: int, N: int, dtype: int) -> int:
    return int(lib().ssm_scan_bwd_workspace_bytes(batch, L, D, N, dtype))


def new_workspace(nbytes: int, device="cuda"):
    """A scan workspace: zero-filled before first use, reusable across calls."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def ssm_scan_workspace_status(workspace, stream=None) -> int:
    """Status of the last scan that used `workspace`: SSM_OK (0) or
    SSM_ERR_TIMEOUT. Waits for `stream` (default: the current stream)."""
    if workspace is None:
        return 0
    nbytes = workspace.numel() * workspace.element_size()
    return int(lib().ssm_scan_workspace_status(_ptr(workspace, "workspace"), nbytes, _stream(stream)))


def workspace_error(workspace, stream=None) -> int:
    """Nonzero (the status code) when a wait of the last scan that used this
    workspace gave up; waits for the stream."""
    return ssm_scan_workspace_status(workspace, stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _ptr(t, name, dtype=None, shape=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _order_after_alloc(stream, allocated):
    """Tensors the binding allocates come from torch's caching allocator on the
    current stream (torch.zeros also clears them there). A launch on another
    stream first waits for the current one, and the tensors are recorded as in
    use on the launch stream, so that their memory is not handed out again
    while the kernel may still use it."""
    import torch
    allocated = [t for t in allocated if t is not None]
    if stream is None or not allocated:
        return
    cur = torch.cuda.current_stream()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream))
    if s.cuda_stream == cur.cuda_stream:
        return
    s.wait_stream(cur)
    for t in allocated:
        t.record_stream(s)


def _scan(name, x, delta, dt_bias, A, Bt, Ct, Dskip, z, state_in, state_out, y, workspace, stream,
          lam=None, x_prev=None, B_prev=None, conv_w=None, conv_b=None, conv_state=None):
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, D) and A (D, N)")
    batch, L, D = x.shape
    N = A.shape[1]
    act = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    allocated = []
    if y is None:
        y = torch.empty_like(x)
        allocated.append(y)
    ws_bytes = ssm_scan_workspace_bytes(batch, L, D, N, code)
    own_ws = workspace is None and ws_bytes > 0
    if own_ws:
        workspace = new_workspace(ws_bytes, x.device)
        allocated.append(workspace)
    raw = name in ("ssm_scan_fwd_dt", "ssm_scan_fwd_conv")
    dname = "delta_raw" if raw else "delta"
    if name == "ssm_scan_fwd_conv":
        args = [_ptr(x, "x_raw", act), _ptr(conv_w, "conv_w", f32, (D, 4)), _ptr(conv_b, "conv_b", f32, (D,)),
                _ptr(conv_state, "conv_state", act, (batch, D, 3))]
    else:
        args = [_ptr(x, "x", act)]
    args.append(_ptr(delta, dname, act, (batch, L, D)))
    if raw:
        args.append(_ptr(dt_bias, "dt_bias", f32, (D,)))
    trap = name == "ssm_scan_fwd_trap"
    if trap:
        args.append(_ptr(lam, "lam", act, (batch, L, D)))
    args += [
        _ptr(A, "A", f32, (D, N)),
        _ptr(Bt, "Bt", act, (batch, L, N)), _ptr(Ct, "Ct", act, (batch, L, N)),
        _ptr(Dskip, "Dskip", f32, (D,)), _ptr(z, "z", act, (batch, L, D)),
    ]
    if trap:
        args += [_ptr(x_prev, "x_prev", act, (batch, D)), _ptr(B_prev, "B_prev", act, (batch, N))]
    args += [
        _ptr(state_in, "state_in", f32, (batch, D, N)), _ptr(state_out, "state_out", f32, (batch, D, N)),
        _ptr(y, "y", act, (batch, L, D)),
    ]
    ws_ptr = _ptr(workspace, "workspace")
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _order_after_alloc(stream, allocated)
    st = getattr(lib(), name)(batch, L, D, N, code, *args, ws_ptr, ws_len, _stream(stream))
    if st != 0:
        raise SSMError(st, name)
    if own_ws:
        # The workspace is this call's alone, so its outcome can be read here;
        # that waits for the stream. A caller that passes its own workspace
        # reads it with ssm_scan_workspace_status when it chooses.
        st = ssm_scan_workspace_status(workspace, stream)
        if st != 0:
            raise SSMError(st, name)
    return y


def ssm_scan_fwd(x, delta, A, Bt, Ct, Dskip=None, z=None, state_in=None, state_out=None,
                 y=None, workspace=None, stream=None):
    """Selective scan forward. Shapes: x, delta, z, y (batch, L, D); A (D, N);
    Bt, Ct (batch, L, N); Dskip (D,); state_in, state_out (batch, D, N) float32.
    Allocates y and the workspace with torch when they are not given; with a
    workspace of its own the call waits for the stream and raises SSMError
    (SSM_ERR_TIMEOUT) if a wait for another workgroup's results gave up."""
    return _scan("ssm_scan_fwd", x, delta, None, A, Bt, Ct, Dskip, z, state_in, state_out, y, workspace, stream)


def ssm_scan_fwd_noalloc(x, delta, A, Bt, Ct, y, Dskip=None, z=None, state_in=None, state_out=None, stream=None):
    """ssm_scan_fwd with the library's own static workspace (for callers that
    cannot allocate): the same arguments, y required, nothing allocated."""
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, D) and A (D, N)")
    batch, L, D = x.shape
    N = A.shape[1]
    act, f32 = x.dtype, torch.float32
    code = _dtype_code(x)
    args = [_ptr(x, "x", act), _ptr(delta, "delta", act, (batch, L, D)), _ptr(A, "A", f32, (D, N)),
            _ptr(Bt, "Bt", act, (batch, L, N)), _ptr(Ct, "Ct", act, (batch, L, N)),
            _ptr(Dskip, "Dskip", f32, (D,)), _ptr(z, "z", act, (batch, L, D)),
            _ptr(state_in, "state_in", f32, (batch, D, N)), _ptr(state_out, "state_out", f32, (batch, D, N)),
            _ptr(y, "y", act, (batch, L, D))]
    st = lib().ssm_scan_fwd_noalloc(batch, L, D, N, code, *args, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_scan_fwd_noalloc")
    return y


def ssm_scan_fwd_dt(x, delta_raw, dt_bias, A, Bt, Ct, Dskip=None, z=None, state_in=None, state_out=None,
                    y=None, workspace=None, stream=None):
    """ssm_scan_fwd with the step size before its activation: the kernel uses
    softplus(delta_raw + dt_bias). delta_raw (batch, L, D); dt_bias (D,) float32
    or None (zero)."""
    return _scan("ssm_scan_fwd_dt", x, delta_raw, dt_bias, A, Bt, Ct, Dskip, z, state_in, state_out, y,
                 workspace, stream)


def ssm_scan_fwd_conv(x_raw, conv_w, delta_raw, dt_bias, A, Bt, Ct, conv_b=None, conv_state=None, Dskip=None, z=None,
                      state_in=None, state_out=None, y=None, workspace=None, stream=None):
    """ssm_scan_fwd_dt behind the x branch of the Mamba block: the kernel's x is
    SiLU of the causal width-4 convolution of x_raw (batch, L, D) along the
    tokens, with taps conv_w (D, 4) float32 (tap 3 on the token itself), bias
    conv_b (D,) float32 or None, and conv_state (batch, D, 3) in the activation
    dtype, the raw x of the three tokens before token 0 (oldest first), or None
    (zeros)."""
    return _scan("ssm_scan_fwd_conv", x_raw, delta_raw, dt_bias, A, Bt, Ct, Dskip, z, state_in, state_out, y,
                 workspace, stream, conv_w=conv_w, conv_b=conv_b, conv_state=conv_state)


def ssm_scan_fwd_trap(x, delta, lam, A, Bt, Ct, Dskip=None, z=None, x_prev=None, B_prev=None, state_in=None,
                      state_out=None, y=None, workspace=None, stream=None):
    """ssm_scan_fwd with the exponential-trapezoidal rule: lam (batch, L, D) in
    the activation dtype; x_prev (batch, D) and B_prev (batch, N), the token
    before the first, both or neither."""
    return _scan("ssm_scan_fwd_trap", x, delta, None, A, Bt, Ct, Dskip, z, state_in, state_out, y, workspace,
                 stream, lam=lam, x_prev=x_prev, B_prev=B_prev)


def _step(name, x, delta, dt_bias, A, Bt, Ct, state, Dskip, z, y, stream, lam=None, x_prev=None, B_prev=None,
          conv_w=None, conv_b=None, conv_state=None):
    import torch
    if x.dim() != 2 or A.dim() != 2:
        raise ValueError("x must be (batch, D) and A (D, N)")
    batch, D = x.shape
    N = A.shape[1]
    act = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    allocated = []
    if y is None:
        y = torch.empty_like(x)
        allocated.append(y)
    raw = name in ("ssm_step_dt", "ssm_step_conv")
    dname = "delta_raw" if raw else "delta"
    if name == "ssm_step_conv":
        args = [_ptr(x, "x_raw", act), _ptr(conv_w, "conv_w", f32, (D, 4)), _ptr(conv_b, "conv_b", f32, (D,)),
                _ptr(conv_state, "conv_state", act, (batch, D, 3))]
    else:
        args = [_ptr(x, "x", act)]
    args.append(_ptr(delta, dname, act, (batch, D)))
    if raw:
        args.append(_ptr(dt_bias, "dt_bias", f32, (D,)))
    trap = name == "ssm_step_trap"
    if trap:
        args.append(_ptr(lam, "lam", act, (batch, D)))
    args += [
        _ptr(A, "A", f32, (D, N)),
        _ptr(Bt, "Bt", act, (batch, N)), _ptr(Ct, "Ct", act, (batch, N)),
        _ptr(Dskip, "Dskip", f32, (D,)), _ptr(z, "z", act, (batch, D)),
    ]
    if trap:
        args += [_ptr(x_prev, "x_prev", act, (batch, D)), _ptr(B_prev, "B_prev", act, (batch, N))]
    args += [_ptr(state, "state", f32, (batch, D, N)), _ptr(y, "y", act, (batch, D))]
    _order_after_alloc(stream, allocated)
    st = getattr(lib(), name)(batch, D, N, code, *args, _stream(stream))
    if st != 0:
        raise SSMError(st, name)
    return y


def ssm_step(x, delta, A, Bt, Ct, state, Dskip=None, z=None, y=None, stream=None):
    """One decode step. Shapes: x, delta, z, y (batch, D); A (D, N); Bt, Ct
    (batch, N); Dskip (D,); state (batch, D, N) float32, updated in place."""
    return _step("ssm_step", x, delta, None, A, Bt, Ct, state, Dskip, z, y, stream)


def ssm_step_dt(x, delta_raw, dt_bias, A, Bt, Ct, state, Dskip=None, z=None, y=None, stream=None):
    """ssm_step with the step size before its activation (see ssm_scan_fwd_dt)."""
    return _step("ssm_step_dt", x, delta_raw, dt_bias, A, Bt, Ct, state, Dskip, z, y, stream)


def ssm_step_conv(x_raw, conv_w, conv_state, delta_raw, dt_bias, A, Bt, Ct, state, conv_b=None, Dskip=None, z=None,
                  y=None, stream=None):
    """ssm_step_dt behind the Mamba block's x branch (see ssm_scan_fwd_conv):
    x_raw (batch, D), conv_w (D, 4), conv_b (D,) or None, and conv_state
    (batch, D, 3) in the activation dtype, the raw x of the three tokens
    before, shifted in place to end with this token's."""
    return _step("ssm_step_conv", x_raw, delta_raw, dt_bias, A, Bt, Ct, state, Dskip, z, y, stream, conv_w=conv_w,
                 conv_b=conv_b, conv_state=conv_state)


def ssm_step_trap(x, delta, lam, A, Bt, Ct, state, Dskip=None, z=None, x_prev=None, B_prev=None, y=None,
                  stream=None):
    """One decode step with the exponential-trapezoidal rule: lam (batch, D);
    x_prev (batch, D) and B_prev (batch, N) are the previous token's x and Bt
    (both None at a sequence's first token)."""
    return _step("ssm_step_trap", x, delta, None, A, Bt, Ct, state, Dskip, z, y, stream, lam=lam, x_prev=x_prev,
                 B_prev=B_prev)


def ssm_ssd_fwd(x, delta, A, Bt, Ct, Dskip=None, state_in=None, state_out=None, y=None, stream=None):
    """Mamba-2 SSD layer. Shapes: x, y (batch, L, H, P) and delta (batch, L, H)
    bfloat16; A, Dskip (H,) float32; Bt, Ct (batch, L, G, N) bfloat16;
    state_in, state_out (batch, H, P, N) float32."""
    import torch
    if x.dim() != 4 or Bt.dim() != 4:
        raise ValueError("x must be (batch, L, H, P) and Bt (batch, L, G, N)")
    batch, L, H, P = x.shape
    G, N = Bt.shape[2], Bt.shape[3]
    act, f32 = x.dtype, torch.float32
    code = _dtype_code(x)
    allocated = []
    if y is None:
        y = torch.empty_like(x)
        allocated.append(y)
    args = [_ptr(x, "x", act), _ptr(delta, "delta", act, (batch, L, H)), _ptr(A, "A", f32, (H,)),
            _ptr(Bt, "Bt", act, (batch, L, G, N)), _ptr(Ct, "Ct", act, (batch, L, G, N)),
            _ptr(Dskip, "Dskip", f32, (H,)), _ptr(state_in, "state_in", f32, (batch, H, P, N)),
            _ptr(state_out, "state_out", f32, (batch, H, P, N)), _ptr(y, "y", act, (batch, L, H, P))]
    _order_after_alloc(stream, allocated)
    st = lib().ssm_ssd_fwd(batch, L, H, P, G, N, code, *args, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_ssd_fwd")
    return y


def _scan_bwd(name, x, delta, dt_bias, A, Bt, Ct, dy, Dskip, z, state_in, dstate, out, workspace, stream):
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, D) and A (D, N)")
    batch, L, D = x.shape
    N = A.shape[1]
    act, f32 = x.dtype, torch.float32
    code = _dtype_code(x)
    sp = name == "ssm_scan_bwd_dt"
    dn = "ddelta_raw" if sp else "ddelta"
    o = dict(out or {})
    given = set(o)
    new = lambda shape, dt: torch.empty(shape, dtype=dt, device=x.device)
    o.setdefault("dx", torch.empty_like(x))
    o.setdefault(dn, torch.empty_like(x))
    o.setdefault("dz", None if z is None else torch.empty_like(x))
    o.setdefault("dA", new((D, N), f32))
    o.setdefault("dBt", new((batch, L, N), f32))
    o.setdefault("dCt", new((batch, L, N), f32))
    o.setdefault("dDskip", None if Dskip is None else new((D,), f32))
    o.setdefault("dstate_in", new((batch, D, N), f32))
    if sp:
        o.setdefault("ddt_bias", new((D,), f32))
    ws_bytes = ssm_scan_bwd_workspace_bytes(batch, L, D, N, code)
    allocated = [v for k, v in o.items() if k not in given]
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
        allocated.append(workspace)
    args = [_ptr(x, "x", act), _ptr(delta, "delta_raw" if sp else "delta", act, (batch, L, D))]
    if sp:
        args.append(_ptr(dt_bias, "dt_bias", f32, (D,)))
    args += [_ptr(A, "A", f32, (D, N)),
             _ptr(Bt, "Bt", act, (batch, L, N)), _ptr(Ct, "Ct", act, (batch, L, N)),
             _ptr(Dskip, "Dskip", f32, (D,)), _ptr(z, "z", act, (batch, L, D)),
             _ptr(state_in, "state_in", f32, (batch, D, N)), _ptr(dy, "dy", act, (batch, L, D)),
             _ptr(dstate, "dstate", f32, (batch, D, N)),
             _ptr(o["dx"], "dx", act, (batch, L, D)), _ptr(o[dn], dn, act, (batch, L, D))]
    if sp:
        args.append(_ptr(o["ddt_bias"], "ddt_bias", f32, (D,)))
    args += [_ptr(o["dA"], "dA", f32, (D, N)), _ptr(o["dBt"], "dBt", f32, (batch, L, N)),
             _ptr(o["dCt"], "dCt", f32, (batch, L, N)), _ptr(o["dDskip"], "dDskip", f32, (D,)),
             _ptr(o["dz"], "dz", act, (batch, L, D)), _ptr(o["dstate_in"], "dstate_in", f32, (batch, D, N))]
    ws_ptr = _ptr(workspace, "workspace")
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _order_after_alloc(stream, allocated)
    st = getattr(lib(), name)(batch, L, D, N, code, *args, ws_ptr, ws_len, _stream(stream))
    if st != 0:
        raise SSMError(st, name)
    return o


def ssm_scan_bwd(x, delta, A, Bt, Ct, dy, Dskip=None, z=None, state_in=None, dstate=None, out=None,
                 workspace=None, stream=None):
    """Gradient of ssm_scan_fwd for the loss sum(dy * y) + sum(dstate * state_out).
    Inputs as for ssm_scan_fwd; dy like x; dstate (batch, D, N) float32 or None.
    Returns a dict: dx, ddelta, dz (like x; dz None without a gate), dA (D, N),
    dBt, dCt (batch, L, N), dDskip (D,) or None, dstate_in (batch, D, N), all
    float32 but the first three. `out` may hold preallocated outputs by those names."""
    return _scan_bwd("ssm_scan_bwd", x, delta, None, A, Bt, Ct, dy, Dskip, z, state_in, dstate, out, workspace,
                     stream)


def ssm_scan_bwd_dt(x, delta_raw, dt_bias, A, Bt, Ct, dy, Dskip=None, z=None, state_in=None, dstate=None,
                    out=None, workspace=None, stream=None):
    """Gradient of ssm_scan_fwd_dt (step size softplus(delta_raw + dt_bias)).
    As ssm_scan_bwd, with ddelta_raw (like x) in place of ddelta and ddt_bias
    (D,) float32 (set out["ddt_bias"] = None to leave it out)."""
    return _scan_bwd("ssm_scan_bwd_dt", x, delta_raw, dt_bias, A, Bt, Ct, dy, Dskip, z, state_in, dstate, out,
                     workspace, stream)


def ssm_scan_bwd_conv(x_raw, conv_w, delta_raw, dt_bias, A, Bt, Ct, dy, conv_b=None, conv_state=None, Dskip=None,
                      z=None, state_in=None, dstate=None, out=None, workspace=None, stream=None):
    """Gradient of ssm_scan_fwd_conv. As ssm_scan_bwd_dt, with dx_raw (like x_raw)
    in place of dx, and dconv_w (D, 4), dconv_b (D,) (None without conv_b) float32
    and dconv_state (batch, D, 3) in x_raw's dtype (None without conv_state;
    set out["dconv_state"] to ask for it anyway)."""
    import torch
    if x_raw.dim() != 3 or A.dim() != 2:
        raise ValueError("x_raw must be (batch, L, D) and A (D, N)")
    batch, L, D = x_raw.shape
    N = A.shape[1]
    act, f32 = x_raw.dtype, torch.float32
    code = _dtype_code(x_raw)
    o = dict(out or {})
    given = set(o)
    new = lambda shape, dt: torch.empty(shape, dtype=dt, device=x_raw.device)
    o.setdefault("dx_raw", torch.empty_like(x_raw))
    o.setdefault("dconv_w", new((D, 4), f32))
    o.setdefault("dconv_b", None if conv_b is None else new((D,), f32))
    o.setdefault("dconv_state", None if conv_state is None else new((batch, D, 3), act))
    o.setdefault("ddelta_raw", torch.empty_like(x_raw))
    o.setdefault("ddt_bias", new((D,), f32))
    o.setdefault("dA", new((D, N), f32))
    o.setdefault("dBt", new((batch, L, N), f32))
    o.setdefault("dCt", new((batch, L, N), f32))
    o.setdefault("dDskip", None if Dskip is None else new((D,), f32))
    o.setdefault("dz", None if z is None else torch.empty_like(x_raw))
    o.setdefault("dstate_in", new((batch, D, N), f32))
    ws_bytes = lib().ssm_scan_bwd_conv_workspace_bytes(batch, L, D, N, code)
    allocated = [v for k, v in o.items() if k not in given and v is not None]
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x_raw.device)
        allocated.append(workspace)
    args = [_ptr(x_raw, "x_raw", act), _ptr(conv_w, "conv_w", f32, (D, 4)), _ptr(conv_b, "conv_b", f32, (D,)),
            _ptr(conv_state, "conv_state", act, (batch, D, 3)), _ptr(delta_raw, "delta_raw", act, (batch, L, D)),
            _ptr(dt_bias, "dt_bias", f32, (D,)), _ptr(A, "A", f32, (D, N)),
            _ptr(Bt, "Bt", act, (batch, L, N)), _ptr(Ct, "Ct", act, (batch, L, N)),
            _ptr(Dskip, "Dskip", f32, (D,)), _ptr(z, "z", act, (batch, L, D)),
            _ptr(state_in, "state_in", f32, (batch, D, N)), _ptr(dy, "dy", act, (batch, L, D)),
            _ptr(dstate, "dstate", f32, (batch, D, N)),
            _ptr(o["dx_raw"], "dx_raw", act, (batch, L, D)), _ptr(o["dconv_w"], "dconv_w", f32, (D, 4)),
            _ptr(o["dconv_b"], "dconv_b", f32, (D,)), _ptr(o["dconv_state"], "dconv_state", act, (batch, D, 3)),
            _ptr(o["ddelta_raw"], "ddelta_raw", act, (batch, L, D)), _ptr(o["ddt_bias"], "ddt_bias", f32, (D,)),
            _ptr(o["dA"], "dA", f32, (D, N)), _ptr(o["dBt"], "dBt", f32, (batch, L, N)),
            _ptr(o["dCt"], "dCt", f32, (batch, L, N)), _ptr(o["dDskip"], "dDskip", f32, (D,)),
            _ptr(o["dz"], "dz", act, (batch, L, D)), _ptr(o["dstate_in"], "dstate_in", f32, (batch, D, N))]
    ws_ptr = _ptr(workspace, "workspace")
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _order_after_alloc(stream, allocated)
    st = lib().ssm_scan_bwd_conv(batch, L, D, N, code, *args, ws_ptr, ws_len, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_scan_bwd_conv")
    return o


def ssm_scan_bwd_trap(x, delta, lam, A, Bt, Ct, dy, Dskip=None, z=None, x_prev=None, B_prev=None, state_in=None,
                      dstate=None, out=None, workspace=None, stream=None):
    """Gradient of ssm_scan_fwd_trap. As ssm_scan_bwd, plus dlam (like x) and,
    when x_prev and B_prev are given, dx_prev (batch, D) in x's dtype and
    dB_prev (batch, N) float32."""
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, D) and A (D, N)")
    batch, L, D = x.shape
    N = A.shape[1]
    act, f32 = x.dtype, torch.float32
    code = _dtype_code(x)
    o = dict(out or {})
    given = set(o)
    new = lambda shape, dt: torch.empty(shape, dtype=dt, device=x.device)
    for k in ("dx", "ddelta", "dlam"):
        o.setdefault(k, torch.empty_like(x))
    o.setdefault("dz", None if z is None else torch.empty_like(x))
    o.setdefault("dA", new((D, N), f32))
    o.setdefault("dBt", new((batch, L, N), f32))
    o.setdefault("dCt", new((batch, L, N), f32))
    o.setdefault("dDskip", None if Dskip is None else new((D,), f32))
    o.setdefault("dx_prev", None if x_prev is None else new((batch, D), act))
    o.setdefault("dB_prev", None if x_prev is None else new((batch, N), f32))
    o.setdefault("dstate_in", new((batch, D, N), f32))
    ws_bytes = ssm_scan_bwd_workspace_bytes(batch, L, D, N, code)
    allocated = [v for k, v in o.items() if k not in given]
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
        allocated.append(workspace)
    args = [_ptr(x, "x", act), _ptr(delta, "delta", act, (batch, L, D)), _ptr(lam, "lam", act, (batch, L, D)),
            _ptr(A, "A", f32, (D, N)), _ptr(Bt, "Bt", act, (batch, L, N)), _ptr(Ct, "Ct", act, (batch, L, N)),
            _ptr(Dskip, "Dskip", f32, (D,)), _ptr(z, "z", act, (batch, L, D)),
            _ptr(x_prev, "x_prev", act, (batch, D)), _ptr(B_prev, "B_prev", act, (batch, N)),
            _ptr(state_in, "state_in", f32, (batch, D, N)), _ptr(dy, "dy", act, (batch, L, D)),
            _ptr(dstate, "dstate", f32, (batch, D, N)),
            _ptr(o["dx"], "dx", act, (batch, L, D)), _ptr(o["ddelta"], "ddelta", act, (batch, L, D)),
            _ptr(o["dlam"], "dlam", act, (batch, L, D)), _ptr(o["dA"], "dA", f32, (D, N)),
            _ptr(o["dBt"], "dBt", f32, (batch, L, N)), _ptr(o["dCt"], "dCt", f32, (batch, L, N)),
            _ptr(o["dDskip"], "dDskip", f32, (D,)), _ptr(o["dz"], "dz", act, (batch, L, D)),
            _ptr(o["dx_prev"], "dx_prev", act, (batch, D)), _ptr(o["dB_prev"], "dB_prev", f32, (batch, N)),
            _ptr(o["dstate_in"], "dstate_in", f32, (batch, D, N))]
    ws_ptr = _ptr(workspace, "workspace")
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _order_after_alloc(stream, allocated)
    st = lib().ssm_scan_bwd_trap(batch, L, D, N, code, *args, ws_ptr, ws_len, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_scan_bwd_trap")
    return o


def ssm_ssd_step(x, delta, A, Bt, Ct, state, Dskip=None, y=None, stream=None):
    """One Mamba-2 SSD decode token. Shapes: x, y (batch, H, P) and delta
    (batch, H) in the activation dtype; A, Dskip (H,) float32; Bt, Ct (batch,
    G, N); state (batch, H, P, N) float32, updated in place."""
    import torch
    if x.dim() != 3 or Bt.dim() != 3:
        raise ValueError("x must be (batch, H, P) and Bt (batch, G, N)")
    batch, H, P = x.shape
    G, N = Bt.shape[1], Bt.shape[2]
    act, f32 = x.dtype, torch.float32
    code = _dtype_code(x)
    allocated = []
    if y is None:
        y = torch.empty_like(x)
        allocated.append(y)
    args = [_ptr(x, "x", act), _ptr(delta, "delta", act, (batch, H)), _ptr(A, "A", f32, (H,)),
            _ptr(Bt, "Bt", act, (batch, G, N)), _ptr(Ct, "Ct", act, (batch, G, N)), _ptr(Dskip, "Dskip", f32, (H,)),
            _ptr(state, "state", f32, (batch, H, P, N)), _ptr(y, "y", act, (batch, H, P))]
    _order_after_alloc(stream, allocated)
    st = lib().ssm_ssd_step(batch, H, P, G, N, code, *args, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_ssd_step")
    return y
