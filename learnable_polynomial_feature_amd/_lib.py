"""ctypes binding of libllops.so (C ABI in include/llops.h).

Argument marshalling only: tensors are checked for device, dtype and shape,
made contiguous, and their data pointers are handed to the C entry points
together with torch's current HIP stream. Every step of the computation runs
in the library's HIP kernels; if the library is missing the calls raise.
PyTorch provides device memory and streams and nothing else here.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LLOPS_LIBRARY: another build of the same library (e.g. the host-sanitized
# one, `python -m learnable_polynomial_feature_amd.build --host-sanitize`)
LIB_PATH = os.environ.get("LLOPS_LIBRARY") or os.path.join(_HERE, "libllops.so")

F32, BF16 = 0, 1
(ENTRY_FEATMAP, ENTRY_LINATTN, ENTRY_CAUSAL, ENTRY_DECODE, ENTRY_FEATMAP_BWD, ENTRY_CAUSAL_BWD,
 ENTRY_LINATTN_BWD, ENTRY_GATED_CAUSAL, ENTRY_GATED_DECODE,
 ENTRY_GATED_CAUSAL_BWD) = 0, 1, 2, 3, 4, 5, 6, 7, 8, 9
STATUS = {0: "LLOPS_OK", 1: "LLOPS_ERR_INVALID_ARG", 2: "LLOPS_ERR_UNSUPPORTED",
          3: "LLOPS_ERR_WORKSPACE", 4: "LLOPS_ERR_HIP"}
EXPORTS = ("llops_workspace_bytes", "llops_featmap", "llops_featmap_bwd", "llops_linattn_fwd",
           "llops_linattn_causal_fwd", "llops_linattn_causal_bwd", "llops_linattn_bwd",
           "llops_decode_step", "llops_linattn_gated_causal_fwd", "llops_gated_decode_step",
           "llops_linattn_gated_causal_bwd", "llops_linattn_causal_bwd_state",
           "llops_linattn_gated_causal_bwd_state", "llops_decode_step_noalloc",
           "llops_status_str",
           "llops_last_error", "llops_profile_arm", "llops_profile_disarm")


class LlopsError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Shape(ctypes.Structure):
    """Mirror of llops_shape_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("n", ctypes.c_int64),
        ("d", ctypes.c_int32), ("dv", ctypes.c_int32), ("m", ctypes.c_int32),
        ("p", ctypes.c_int32), ("t", ctypes.c_int32),
        ("square", ctypes.c_int32), ("normalize", ctypes.c_int32), ("delta", ctypes.c_float),
        ("chunk", ctypes.c_int32), ("theta_per_head", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
    ]


_LIB = None
_P = ctypes.c_void_p


def library(path: str | None = None) -> ctypes.CDLL:
    """Load libllops.so once (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise LlopsError(-1, f"{path} not found; run learnable_polynomial_feature_amd.build")
    lib = ctypes.CDLL(path)
    SP = ctypes.POINTER(Shape)
    lib.llops_workspace_bytes.argtypes = [SP, ctypes.c_int32]
    lib.llops_workspace_bytes.restype = ctypes.c_size_t
    lib.llops_featmap.argtypes = [SP, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.llops_featmap.restype = ctypes.c_int
    lib.llops_featmap_bwd.argtypes = [SP, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.llops_featmap_bwd.restype = ctypes.c_int
    lib.llops_linattn_fwd.argtypes = [SP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.llops_linattn_fwd.restype = ctypes.c_int
    lib.llops_linattn_causal_fwd.argtypes = [SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]
    lib.llops_linattn_causal_fwd.restype = ctypes.c_int
    lib.llops_linattn_causal_bwd.argtypes = [SP] + [_P] * 12 + [ctypes.c_size_t, _P]
    lib.llops_linattn_causal_bwd.restype = ctypes.c_int
    lib.llops_linattn_causal_bwd_state.argtypes = [SP] + [_P] * 16 + [ctypes.c_size_t, _P]
    lib.llops_linattn_causal_bwd_state.restype = ctypes.c_int
    lib.llops_linattn_bwd.argtypes = [SP] + [_P] * 12 + [ctypes.c_size_t, _P]
    lib.llops_linattn_bwd.restype = ctypes.c_int
    lib.llops_decode_step.argtypes = [SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.llops_decode_step.restype = ctypes.c_int
    lib.llops_linattn_gated_causal_fwd.argtypes = [SP] + [_P] * 12 + [ctypes.c_size_t, _P]
    lib.llops_linattn_gated_causal_fwd.restype = ctypes.c_int
    lib.llops_gated_decode_step.argtypes = [SP] + [_P] * 10 + [ctypes.c_size_t, _P]
    lib.llops_gated_decode_step.restype = ctypes.c_int
    lib.llops_linattn_gated_causal_bwd.argtypes = [SP] + [_P] * 14 + [ctypes.c_size_t, _P]
    lib.llops_linattn_gated_causal_bwd.restype = ctypes.c_int
    lib.llops_linattn_gated_causal_bwd_state.argtypes = [SP] + [_P] * 18 + [ctypes.c_size_t, _P]
    lib.llops_linattn_gated_causal_bwd_state.restype = ctypes.c_int
    lib.llops_decode_step_noalloc.argtypes = [SP] + [_P] * 8 + [_P]
    lib.llops_decode_step_noalloc.restype = ctypes.c_int
    lib.llops_status_str.argtypes = [ctypes.c_int]
    lib.llops_status_str.restype = ctypes.c_char_p
    lib.llops_last_error.argtypes = []
    lib.llops_last_error.restype = ctypes.c_char_p
    lib.llops_profile_arm.argtypes = [_P, _P, ctypes.c_int32]
    lib.llops_profile_arm.restype = ctypes.c_int
    lib.llops_profile_disarm.argtypes = []
    lib.llops_profile_disarm.restype = ctypes.c_int32
    _LIB = lib
    return lib


# ---------------------------------------------------------------------------
def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Argument checks run in two passes. The first looks only at metadata
# (types, shapes, dtypes, contiguity of buffers written in place, agreement
# between tensors); the second (_on_device) then requires every tensor on one
# GPU. Nothing reaches the library before both pass, so a mismatched buffer
# can never become an out-of-bounds access on the device.
def _t(t, name: str) -> torch.Tensor:
    """An input tensor (made contiguous; inputs may be copied)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    return t.contiguous()


def _opt_t(t, name: str):
    return None if t is None else _t(t, name)


def _want(t, name: str, shape, dtype=None):
    """An input's shape (and dtype) as the call requires."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _out(t, name: str, shape, dtype) -> torch.Tensor:
    """A caller-supplied buffer the library writes in place: it must already
    have the shape and dtype and be contiguous (a copy cannot stand in)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    _want(t, name, shape, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} is written in place and must be contiguous")
    return t


def _ws_arg(ws):
    """A caller-supplied workspace: any dtype, contiguous (its byte size is
    checked by the library against llops_workspace_bytes)."""
    if ws is None:
        return None
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws


def _on_device(**tensors):
    """Every tensor handed to the library lives on one and the same GPU."""
    first = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if first is None:
            first = t.device
        elif t.device != first:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {first}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status: int):
    if status != 0:
        raise LlopsError(status, library().llops_last_error().decode())


def _theta_dims(theta: torch.Tensor, heads: int):
    if theta.dim() == 5:
        if theta.shape[0] != heads:
            raise ValueError(f"theta has {theta.shape[0]} heads, inputs have {heads}")
        return (*theta.shape[1:],), 1
    if theta.dim() == 4:
        return tuple(theta.shape), 0
    raise ValueError("theta must be [heads, p, t, d, m] or [p, t, d, m]")


def _two_thetas(theta_q, theta_k, heads: int, d: int):
    """(p, t, m, theta_per_head) of a Theta_q / Theta_k pair of one shape and
    head layout whose d matches the inputs'."""
    dq, ph = _theta_dims(theta_q, heads)
    dk, phk = _theta_dims(theta_k, heads)
    if dq != dk or ph != phk:
        raise ValueError("theta_q and theta_k must have the same shape")
    p, t, td, m = dq
    if td != d:
        raise ValueError(f"theta's d ({td}) must match the inputs' d ({d})")
    return p, t, m, ph


def make_shape(*, batch, heads, n, d, dv, m, p, t, square=False, normalize=False, delta=0.0,
               chunk=0, theta_per_head=1, in_dtype=BF16, out_dtype=F32) -> Shape:
    return Shape(batch, heads, n, d, dv, m, p, t, int(square), int(normalize),
                 float(delta), int(chunk), int(theta_per_head), int(in_dtype), int(out_dtype))


def llops_workspace_bytes(shape: Shape, entry: int) -> int:
    return int(library().llops_workspace_bytes(ctypes.byref(shape), int(entry)))


def _workspace(shape: Shape, entry: int, device, ws):
    need = llops_workspace_bytes(shape, entry)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
def llops_featmap(X, theta, *, square=False, out=None, out_dtype=torch.float32, workspace=None):
    """phi = sum_r prod_j X Theta_{j,r} [squared]; X [B, H, n, d] -> phi [B, H, n, m]."""
    X, theta = _t(X, "X"), _t(theta, "theta")
    if X.dim() != 4:
        raise ValueError("X must be [batch, heads, n, d]")
    B, H, n, d = X.shape
    (p, t, td, m), per_head = _theta_dims(theta, H)
    if td != d or theta.dtype != X.dtype:
        raise ValueError("theta's d and dtype must match X")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    idt = _dt(X)
    if out is not None:
        _out(out, "out", (B, H, n, m), out_dtype)
    workspace = _ws_arg(workspace)
    _on_device(X=X, theta=theta, out=out, workspace=workspace)
    odt = BF16 if out_dtype == torch.bfloat16 else F32
    if out is None:
        out = torch.empty((B, H, n, m), dtype=out_dtype, device=X.device)
    shape = make_shape(batch=B, heads=H, n=n, d=d, dv=1, m=m, p=p, t=t, square=square,
                       theta_per_head=per_head, in_dtype=idt, out_dtype=odt)
    lib = library()
    ws, wsb = _workspace(shape, ENTRY_FEATMAP, X.device, workspace)
    _check(lib.llops_featmap(ctypes.byref(shape), _ptr(X), _ptr(theta), _ptr(out), _ptr(ws), wsb,
                             _stream(X)))
    return out


def llops_featmap_bwd(X, theta, dphi, *, square=False, dX=None, dtheta=None, workspace=None):
    """Gradients (dX, dtheta) of sum(dphi * phi) for phi = llops_featmap(X, theta, square).

    X [B, H, n, d] and theta bf16; dphi [B, H, n, m] fp32 or bf16; dX fp32 like
    X, dtheta fp32 like theta (summed over heads when theta is shared).
    """
    X, theta, dphi = _t(X, "X"), _t(theta, "theta"), _t(dphi, "dphi")
    if X.dim() != 4:
        raise ValueError("X must be [batch, heads, n, d]")
    B, H, n, d = X.shape
    (p, t, td, m), per_head = _theta_dims(theta, H)
    if td != d or theta.dtype != X.dtype:
        raise ValueError("theta's d and dtype must match X")
    _want(dphi, "dphi", (B, H, n, m))
    idt, gdt = _dt(X), _dt(dphi)
    if dX is not None:
        _out(dX, "dX", (B, H, n, d), torch.float32)
    if dtheta is not None:
        _out(dtheta, "dtheta", tuple(theta.shape), torch.float32)
    workspace = _ws_arg(workspace)
    _on_device(X=X, theta=theta, dphi=dphi, dX=dX, dtheta=dtheta, workspace=workspace)
    if dX is None:
        dX = torch.empty((B, H, n, d), dtype=torch.float32, device=X.device)
    if dtheta is None:
        dtheta = torch.empty(theta.shape, dtype=torch.float32, device=X.device)
    shape = make_shape(batch=B, heads=H, n=n, d=d, dv=1, m=m, p=p, t=t, square=square,
                       theta_per_head=per_head, in_dtype=idt, out_dtype=gdt)
    lib = library()
    ws, wsb = _workspace(shape, ENTRY_FEATMAP_BWD, X.device, workspace)
    _check(lib.llops_featmap_bwd(ctypes.byref(shape), _ptr(X), _ptr(theta), _ptr(dphi), _ptr(dX),
                                 _ptr(dtheta), _ptr(ws), wsb, _stream(X)))
    return dX, dtheta


def _attn_shape(Q, K, V, theta_q, theta_k, square, normalize, delta, chunk):
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B, H, n, d] and V [B, H, n, dv]")
    B, H, n, d = Q.shape
    p, t, m, ph = _two_thetas(theta_q, theta_k, H, d)
    dts = {x.dtype for x in (Q, K, V, theta_q, theta_k)}
    if len(dts) != 1:
        raise ValueError("Q, K, V and theta must share one dtype")
    return make_shape(batch=B, heads=H, n=n, d=d, dv=V.shape[3], m=m, p=p, t=t, square=square,
                      normalize=normalize, delta=delta, chunk=chunk, theta_per_head=ph,
                      in_dtype=_dt(Q), out_dtype=F32)


def _attn_inputs(Q, K, V, theta_q, theta_k):
    return (_t(Q, "Q"), _t(K, "K"), _t(V, "V"), _t(theta_q, "theta_q"), _t(theta_k, "theta_k"))


def _state_inputs(S0, z0, B, H, m, dv):
    S0, z0 = _opt_t(S0, "S0"), _opt_t(z0, "z0")
    if S0 is not None:
        _want(S0, "S0", (B, H, m, dv), torch.float32)
    if z0 is not None:
        _want(z0, "z0", (B, H, m), torch.float32)
    return S0, z0


def llops_linattn_fwd(Q, K, V, theta_q, theta_k, *, square=False, normalize=False, delta=0.0,
                      out=None, workspace=None):
    """Non-causal: out = phi_Q (phi_K^T V) [/ (phi_Q (phi_K^T 1) + delta)] (fp32)."""
    Q, K, V, theta_q, theta_k = _attn_inputs(Q, K, V, theta_q, theta_k)
    shape = _attn_shape(Q, K, V, theta_q, theta_k, square, normalize, delta, 0)
    if out is not None:
        _out(out, "out", tuple(V.shape), torch.float32)
    workspace = _ws_arg(workspace)
    _on_device(Q=Q, K=K, V=V, theta_q=theta_q, theta_k=theta_k, out=out, workspace=workspace)
    if out is None:
        out = torch.empty(V.shape, dtype=torch.float32, device=Q.device)
    ws, wsb = _workspace(shape, ENTRY_LINATTN, Q.device, workspace)
    _check(library().llops_linattn_fwd(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V),
                                       _ptr(theta_q), _ptr(theta_k), _ptr(out), _ptr(ws), wsb,
                                       _stream(Q)))
    return out


def llops_linattn_causal_fwd(Q, K, V, theta_q, theta_k, *, square=False, normalize=False,
                             delta=0.0, chunk=0, S0=None, z0=None, out=None, S_final=None,
                             z_final=None, return_state=False, workspace=None):
    """Causal linear attention with optional initial/final recurrent state.

    Returns out [B, H, n, dv] fp32, or (out, S_final, z_final) when return_state.
    """
    return _causal(None, Q, K, V, theta_q, theta_k, square, normalize, delta, chunk, S0, z0, out,
                   S_final, z_final, return_state, workspace)


def llops_linattn_gated_causal_fwd(Q, K, V, theta_q, theta_k, log_gate, *, square=False,
                                   normalize=False, delta=0.0, chunk=0, S0=None, z0=None, out=None,
                                   S_final=None, z_final=None, return_state=False, workspace=None):
    """Causal linear attention whose state decays by exp(log_gate[b, h, i]) before token i.

    log_gate: fp32 [B, H, n]. Returns as llops_linattn_causal_fwd.
    """
    if log_gate is None:
        raise ValueError("log_gate is required")
    return _causal(log_gate, Q, K, V, theta_q, theta_k, square, normalize, delta, chunk, S0, z0,
                   out, S_final, z_final, return_state, workspace)


def _causal(log_gate, Q, K, V, theta_q, theta_k, square, normalize, delta, chunk, S0, z0, out,
            S_final, z_final, return_state, workspace):
    Q, K, V, theta_q, theta_k = _attn_inputs(Q, K, V, theta_q, theta_k)
    shape = _attn_shape(Q, K, V, theta_q, theta_k, square, normalize, delta, chunk)
    B, H = Q.shape[:2]
    m, dv = shape.m, shape.dv
    S0, z0 = _state_inputs(S0, z0, B, H, m, dv)
    if S_final is not None:
        _out(S_final, "S_final", (B, H, m, dv), torch.float32)
    if z_final is not None:
        _out(z_final, "z_final", (B, H, m), torch.float32)
    if out is not None:
        _out(out, "out", tuple(V.shape), torch.float32)
    if log_gate is not None:
        log_gate = _t(log_gate, "log_gate")
        _want(log_gate, "log_gate", tuple(Q.shape[:3]), torch.float32)
    workspace = _ws_arg(workspace)
    _on_device(Q=Q, K=K, V=V, theta_q=theta_q, theta_k=theta_k, S0=S0, z0=z0, S_final=S_final,
               z_final=z_final, out=out, log_gate=log_gate, workspace=workspace)
    if return_state:
        if S_final is None:
            S_final = torch.empty((B, H, m, dv), dtype=torch.float32, device=Q.device)
        if z_final is None:
            z_final = torch.empty((B, H, m), dtype=torch.float32, device=Q.device)
    if out is None:
        out = torch.empty(V.shape, dtype=torch.float32, device=Q.device)
    if log_gate is None:
        ws, wsb = _workspace(shape, ENTRY_CAUSAL, Q.device, workspace)
        _check(library().llops_linattn_causal_fwd(
            ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta_q), _ptr(theta_k),
            _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_final), _ptr(z_final), _ptr(ws), wsb,
            _stream(Q)))
    else:
        ws, wsb = _workspace(shape, ENTRY_GATED_CAUSAL, Q.device, workspace)
        _check(library().llops_linattn_gated_causal_fwd(
            ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta_q), _ptr(theta_k),
            _ptr(log_gate), _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_final), _ptr(z_final),
            _ptr(ws), wsb, _stream(Q)))
    if return_state:
        return out, S_final, z_final
    return out


def _grad_inputs(Q, K, V, theta_q, theta_k, dO, square, normalize, delta):
    Q, K, V, theta_q, theta_k = _attn_inputs(Q, K, V, theta_q, theta_k)
    shape = _attn_shape(Q, K, V, theta_q, theta_k, square, normalize, delta, 0)
    dO = _t(dO, "dO")
    _want(dO, "dO", tuple(V.shape), torch.float32)
    return Q, K, V, theta_q, theta_k, dO, shape


def _grads(Q, K, V, theta_q, theta_k):
    f32 = dict(dtype=torch.float32, device=Q.device)
    return (torch.empty(Q.shape, **f32), torch.empty(K.shape, **f32), torch.empty(V.shape, **f32),
            torch.empty(theta_q.shape, **f32), torch.empty(theta_k.shape, **f32))


def llops_linattn_causal_bwd(Q, K, V, theta_q, theta_k, dO, *, square=False, normalize=False,
                             delta=0.0, workspace=None):
    """Gradients (dQ, dK, dV, dtheta_q, dtheta_k) of sum(dO * out) for
    out = llops_linattn_causal_fwd(Q, K, V, theta_q, theta_k, ...) from a zero
    state. Q, K, V and thetas bf16; dO fp32 [B, H, n, dv]; all results fp32."""
    return _attn_bwd(True, Q, K, V, theta_q, theta_k, dO, square, normalize, delta, workspace)


def llops_linattn_causal_bwd_state(Q, K, V, theta_q, theta_k, dO, *, S0=None, z0=None,
                                   square=False, normalize=False, delta=0.0, workspace=None):
    """Gradients (dQ, dK, dV, dtheta_q, dtheta_k, dS0, dz0) of sum(dO * out) for
    out = llops_linattn_causal_fwd(..., S0=S0, z0=z0); S0 fp32 [B, H, m, dv] and
    z0 fp32 [B, H, m] (None = zeros)."""
    Q, K, V, theta_q, theta_k, dO, shape = _grad_inputs(Q, K, V, theta_q, theta_k, dO, square,
                                                        normalize, delta)
    B, H = Q.shape[:2]
    m, dv = shape.m, shape.dv
    S0, z0 = _state_inputs(S0, z0, B, H, m, dv)
    workspace = _ws_arg(workspace)
    _on_device(Q=Q, K=K, V=V, theta_q=theta_q, theta_k=theta_k, dO=dO, S0=S0, z0=z0,
               workspace=workspace)
    dQ, dK, dV, dtq, dtk = _grads(Q, K, V, theta_q, theta_k)
    f32 = dict(dtype=torch.float32, device=Q.device)
    dS0, dz0 = torch.empty((B, H, m, dv), **f32), torch.empty((B, H, m), **f32)
    ws, wsb = _workspace(shape, ENTRY_CAUSAL_BWD, Q.device, workspace)
    _check(library().llops_linattn_causal_bwd_state(
        ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta_q), _ptr(theta_k), _ptr(S0),
        _ptr(z0), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dtq), _ptr(dtk), _ptr(dS0),
        _ptr(dz0), _ptr(ws), wsb, _stream(Q)))
    return dQ, dK, dV, dtq, dtk, dS0, dz0


def llops_linattn_bwd(Q, K, V, theta_q, theta_k, dO, *, square=False, normalize=False, delta=0.0,
                      workspace=None):
    """The same gradients for the non-causal llops_linattn_fwd."""
    return _attn_bwd(False, Q, K, V, theta_q, theta_k, dO, square, normalize, delta, workspace)


def _attn_bwd(causal, Q, K, V, theta_q, theta_k, dO, square, normalize, delta, workspace):
    Q, K, V, theta_q, theta_k, dO, shape = _grad_inputs(Q, K, V, theta_q, theta_k, dO, square,
                                                        normalize, delta)
    workspace = _ws_arg(workspace)
    _on_device(Q=Q, K=K, V=V, theta_q=theta_q, theta_k=theta_k, dO=dO, workspace=workspace)
    dQ, dK, dV, dtq, dtk = _grads(Q, K, V, theta_q, theta_k)
    lib = library()
    ws, wsb = _workspace(shape, ENTRY_CAUSAL_BWD if causal else ENTRY_LINATTN_BWD, Q.device,
                         workspace)
    fn = lib.llops_linattn_causal_bwd if causal else lib.llops_linattn_bwd
    _check(fn(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta_q), _ptr(theta_k),
              _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dtq), _ptr(dtk), _ptr(ws), wsb,
              _stream(Q)))
    return dQ, dK, dV, dtq, dtk


def llops_linattn_gated_causal_bwd(Q, K, V, theta_q, theta_k, log_gate, dO, *, square=False,
                                   normalize=False, delta=0.0, workspace=None):
    """Gradients (dQ, dK, dV, dtheta_q, dtheta_k, dlog_gate) of sum(dO * out) for
    out = llops_linattn_gated_causal_fwd(Q, K, V, theta_q, theta_k, log_gate, ...)
    from a zero state. Q, K, V and thetas bf16; log_gate fp32 [B, H, n]; dO fp32
    [B, H, n, dv]; all results fp32."""
    return _gated_bwd(Q, K, V, theta_q, theta_k, log_gate, dO, None, None, False, square,
                      normalize, delta, workspace)


def llops_linattn_gated_causal_bwd_state(Q, K, V, theta_q, theta_k, log_gate, dO, *, S0=None,
                                         z0=None, square=False, normalize=False, delta=0.0,
                                         workspace=None):
    """The gated backward for the forward continued from (S0, z0) (None = zeros):
    (dQ, dK, dV, dtheta_q, dtheta_k, dlog_gate, dS0, dz0)."""
    return _gated_bwd(Q, K, V, theta_q, theta_k, log_gate, dO, S0, z0, True, square, normalize,
                      delta, workspace)


def _gated_bwd(Q, K, V, theta_q, theta_k, log_gate, dO, S0, z0, state, square, normalize, delta,
               workspace):
    Q, K, V, theta_q, theta_k, dO, shape = _grad_inputs(Q, K, V, theta_q, theta_k, dO, square,
                                                        normalize, delta)
    log_gate = _t(log_gate, "log_gate")
    _want(log_gate, "log_gate", tuple(Q.shape[:3]), torch.float32)
    B, H = Q.shape[:2]
    m, dv = shape.m, shape.dv
    S0, z0 = _state_inputs(S0, z0, B, H, m, dv)
    workspace = _ws_arg(workspace)
    _on_device(Q=Q, K=K, V=V, theta_q=theta_q, theta_k=theta_k, dO=dO, log_gate=log_gate, S0=S0,
               z0=z0, workspace=workspace)
    dQ, dK, dV, dtq, dtk = _grads(Q, K, V, theta_q, theta_k)
    f32 = dict(dtype=torch.float32, device=Q.device)
    dg = torch.empty(log_gate.shape, **f32)
    ws, wsb = _workspace(shape, ENTRY_GATED_CAUSAL_BWD, Q.device, workspace)
    if not state:
        _check(library().llops_linattn_gated_causal_bwd(
            ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta_q), _ptr(theta_k),
            _ptr(log_gate), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dtq), _ptr(dtk), _ptr(dg),
            _ptr(ws), wsb, _stream(Q)))
        return dQ, dK, dV, dtq, dtk, dg
    dS0, dz0 = torch.empty((B, H, m, dv), **f32), torch.empty((B, H, m), **f32)
    _check(library().llops_linattn_gated_causal_bwd_state(
        ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta_q), _ptr(theta_k),
        _ptr(log_gate), _ptr(S0), _ptr(z0), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dtq),
        _ptr(dtk), _ptr(dg), _ptr(dS0), _ptr(dz0), _ptr(ws), wsb, _stream(Q)))
    return dQ, dK, dV, dtq, dtk, dg, dS0, dz0


def llops_decode_step(q, k, v, theta_q, theta_k, S, z, *, square=False, normalize=True,
                      delta=0.0, out=None, workspace=None):
    """One token per (b, h): S, z updated in place; returns out [B, H, dv] fp32."""
    return _decode(None, q, k, v, theta_q, theta_k, S, z, square, normalize, delta, out, workspace)


def llops_gated_decode_step(q, k, v, theta_q, theta_k, log_gate, S, z, *, square=False,
                            normalize=True, delta=0.0, out=None, workspace=None):
    """llops_decode_step on a state first decayed by exp(log_gate) (fp32 [B, H])."""
    if log_gate is None:
        raise ValueError("log_gate is required")
    return _decode(log_gate, q, k, v, theta_q, theta_k, S, z, square, normalize, delta, out,
                   workspace)


def llops_decode_step_noalloc(q, k, v, theta_q, theta_k, S, z, *, square=False, normalize=True,
                              delta=0.0, out=None):
    """llops_decode_step with its scratch in the library's static per-GPU
    buffer (no workspace allocated). Calls overlapping in time on one GPU race
    on that buffer; S, z updated in place; returns out [B, H, dv] fp32."""
    q, k, v, theta_q, theta_k, _, shape = _decode_args(
        q, k, v, theta_q, theta_k, S, z, square, normalize, delta, out, None)
    _on_device(q=q, k=k, v=v, theta_q=theta_q, theta_k=theta_k, S=S, z=z, out=out)
    if out is None:
        out = torch.empty((shape.batch, shape.heads, shape.dv), dtype=torch.float32,
                          device=q.device)
    _check(library().llops_decode_step_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(theta_q), _ptr(theta_k), _ptr(S), _ptr(z),
                                               _ptr(out), _stream(q)))
    return out


def _decode_args(q, k, v, theta_q, theta_k, S, z, square, normalize, delta, out, log_gate):
    """Checked decode arguments and their llops_shape_t (metadata only)."""
    q, k, v = _t(q, "q"), _t(k, "k"), _t(v, "v")
    theta_q, theta_k = _t(theta_q, "theta_q"), _t(theta_k, "theta_k")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B, H, d] and v [B, H, dv]")
    B, H, d = q.shape
    dv = v.shape[2]
    p, t, m, ph = _two_thetas(theta_q, theta_k, H, d)
    if len({x.dtype for x in (q, k, v, theta_q, theta_k)}) != 1:
        raise ValueError("q, k, v and theta must share one dtype")
    idt = _dt(q)
    _out(S, "S", (B, H, m, dv), torch.float32)
    _out(z, "z", (B, H, m), torch.float32)
    if out is not None:
        _out(out, "out", (B, H, dv), torch.float32)
    if log_gate is not None:
        log_gate = _t(log_gate, "log_gate")
        _want(log_gate, "log_gate", (B, H), torch.float32)
    shape = make_shape(batch=B, heads=H, n=1, d=d, dv=dv, m=m, p=p, t=t, square=square,
                       normalize=normalize, delta=delta, theta_per_head=ph, in_dtype=idt,
                       out_dtype=F32)
    return q, k, v, theta_q, theta_k, log_gate, shape


def _decode(log_gate, q, k, v, theta_q, theta_k, S, z, square, normalize, delta, out, workspace):
    q, k, v, theta_q, theta_k, log_gate, shape = _decode_args(
        q, k, v, theta_q, theta_k, S, z, square, normalize, delta, out, log_gate)
    workspace = _ws_arg(workspace)
    _on_device(q=q, k=k, v=v, theta_q=theta_q, theta_k=theta_k, S=S, z=z, out=out,
               log_gate=log_gate, workspace=workspace)
    B, H, dv = shape.batch, shape.heads, shape.dv
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    if log_gate is None:
        ws, wsb = _workspace(shape, ENTRY_DECODE, q.device, workspace)
        _check(library().llops_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(theta_q), _ptr(theta_k), _ptr(S), _ptr(z),
                                           _ptr(out), _ptr(ws), wsb, _stream(q)))
    else:
        ws, wsb = _workspace(shape, ENTRY_GATED_DECODE, q.device, workspace)
        _check(library().llops_gated_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                                 _ptr(theta_q), _ptr(theta_k), _ptr(log_gate),
                                                 _ptr(S), _ptr(z), _ptr(out), _ptr(ws), wsb,
                                                 _stream(q)))
    return out


class KernelTimer:
    """Times every kernel the library launches inside a ``with`` block, with
    HIP events recorded on the launch stream (llops_profile_arm)."""

    def __init__(self, capacity: int = 4096):
        self.capacity = capacity
        self.events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(capacity)]
        # torch creates the underlying HIP event on first record; record each
        # once so every handle passed to the library is a live event
        for pair in self.events:
            for e in pair:
                e.record()
        torch.cuda.synchronize()
        self._ev = (ctypes.c_void_p * (2 * capacity))(
            *[e.cuda_event for pair in self.events for e in pair])
        self._names = (ctypes.c_char_p * capacity)()
        self.records = []

    def __enter__(self):
        _check(library().llops_profile_arm(self._ev, self._names, self.capacity))
        return self

    def __exit__(self, *exc):
        n = library().llops_profile_disarm()
        self.records = [(self._names[i].decode(), self.events[i]) for i in range(n)]
        return False

    def durations_ms(self) -> dict:
        """kernel name -> list of durations (ms); call after synchronising."""
        out = {}
        for name, (a, b) in self.records:
            out.setdefault(name, []).append(a.elapsed_time(b))
        return out
