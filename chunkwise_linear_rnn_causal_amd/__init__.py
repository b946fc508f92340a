"""Python binding of liblinattn: causal linear attention on MI355X (gfx950).

Thin ctypes layer over the C ABI declared in include/linattn.h, with the same
entry-point names. It only marshals arguments: PyTorch provides device memory
and the current stream; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is not built, or the device is not
gfx950, calls raise.

    o, state, z = la_chunk_fwd("decay", q, k, v, log_gate=lg, C=64, want_state=True)
    o = la_decode_step("decay", q, k, v, log_gate, state)   # state updated in place
    qc, kc, vc, *_ = la_short_conv(q, k, v, w_q, w_k, w_v)  # causal depthwise conv
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblinattn.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "linattn.h")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
VARIANTS = {"plain": 0, "normalized": 1, "decay": 2, "gated_delta": 3, "vector_decay": 4, "kda": 5}
# variants with one log-gate per key channel
_PER_CHANNEL = ("vector_decay", "kda")
EXPORTS = ("la_chunk_fwd_workspace_size", "la_chunk_fwd", "la_chunk_fwd_noalloc",
           "la_chunk_bwd_workspace_size", "la_chunk_bwd", "la_decode_step", "la_short_conv",
           "la_chunk_fwd_conv", "la_chunk_fwd_conv_workspace_size",
           "la_status_str", "la_abi_version")

_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {la_status_str(status)} ({status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblinattn.so (built in-tree by chunkwise_linear_rnn_causal_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m chunkwise_linear_rnn_causal_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.la_abi_version.restype = i
    lib.la_abi_version.argtypes = []
    lib.la_status_str.restype = ctypes.c_char_p
    lib.la_status_str.argtypes = [i]
    lib.la_chunk_fwd_workspace_size.restype = i
    lib.la_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_chunk_fwd.restype = i
    lib.la_chunk_fwd.argtypes = [i, i, i, vp, vp, vp, fp, fp, fp, fp, vp, fp, fp,
                                 i, i, i, i, i, i, vp, sz, vp]
    lib.la_chunk_fwd_noalloc.restype = i
    lib.la_chunk_fwd_noalloc.argtypes = [i, i, i, vp, vp, vp, fp, fp, fp, fp, vp, fp, fp,
                                         i, i, i, i, i, i, vp]
    lib.la_decode_step.restype = i
    lib.la_decode_step.argtypes = [i, i, i, vp, vp, vp, fp, fp, fp, vp, i, i, i, i, vp]
    lib.la_chunk_bwd_workspace_size.restype = i
    lib.la_chunk_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_chunk_bwd.restype = i
    lib.la_chunk_bwd.argtypes = [i, i, vp, vp, vp, fp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                 i, i, i, i, i, i, vp, sz, vp]
    lib.la_short_conv.restype = i
    lib.la_chunk_fwd_conv_workspace_size.restype = i
    lib.la_chunk_fwd_conv_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_chunk_fwd_conv.restype = i
    lib.la_chunk_fwd_conv.argtypes = [i, i, i, vp, vp, vp, fp, fp, fp, i, vp, vp, vp, vp, vp, vp, fp, fp, fp,
                                      vp, fp, i, i, i, i, i, i, vp, sz, vp]
    lib.la_short_conv.argtypes = [i, vp, vp, vp, fp, fp, fp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  i, i, i, i, i, i, vp]
    _lib = lib
    return lib


def la_abi_version() -> int:
    return load_library().la_abi_version()


def la_status_str(status: int) -> str:
    return load_library().la_status_str(int(status)).decode()


def _dt(x) -> int:
    import torch
    dtype = x if isinstance(x, torch.dtype) else x.dtype
    if dtype == torch.bfloat16:
        return 1
    if dtype == torch.float32:
        return 0
    raise TypeError(f"unsupported dtype {dtype}: use torch.bfloat16 or torch.float32")


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return x.data_ptr()


def _check(name: str, x, shape, dtype, device, required: bool = False) -> None:
    """Raise ValueError unless x is None (and not required) or a contiguous tensor of
    exactly this shape and dtype on this device. Every pointer the library reads or
    writes goes through here first, so a wrong shape, dtype or device is a Python
    error instead of an out-of-bounds device access."""
    if x is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if x.dtype != dtype:
        raise ValueError(f"{name} has dtype {x.dtype}, expected {dtype}")
    if x.device != device:
        raise ValueError(f"{name} is on {x.device}, expected {device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(device) -> None:
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")


def _stream(dev, stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def la_chunk_fwd_workspace_size(variant: str, dtype_code: int, B: int, H: int, L: int,
                                d_k: int, d_v: int, C: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().la_chunk_fwd_workspace_size(VARIANTS[variant], dtype_code, B, H, L, d_k,
                                                    d_v, C, ctypes.byref(out))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_fwd_workspace_size")
    return out.value


def la_chunk_fwd(variant: str, q, k, v, log_gate=None, beta=None, state_in=None, z_in=None, *,
                 C: int = 64, o=None, out_dtype=None, state_out=None, z_out=None,
                 want_state: bool = False, want_z: bool = False, workspace=None,
                 stream=None) -> Tuple:
    """Chunkwise causal linear-attention forward.

    q, k: [B, H, L, d_k]; v: [B, H, L, d_v] (bf16 or fp32, contiguous, on the GPU).
    log_gate, beta: [B, H, L] fp32 ("vector_decay", "kda": log_gate [B, H, L, d_k]);
    state_in: [B, H, d_k, d_v] fp32;
    z_in: [B, H, d_k] fp32. Returns (o, state_out or None, z_out or None).
    o is fp32 unless out_dtype=torch.bfloat16 (bf16 inputs only) or a bf16 ``o``
    is passed. Output buffers may be passed in (o, state_out, z_out); state_out
    may be state_in for an in-place carry.
    """
    import torch
    lib = load_library()
    B, H, L, d_k, d_v, o, state_out, z_out = _fwd_args(variant, q, k, v, log_gate, beta, state_in,
                                                       z_in, o, out_dtype, state_out, z_out,
                                                       want_state, want_z)
    dt = _dt(q)
    dev_ = q.device
    ws_bytes = 0
    if workspace is None:
        ws_bytes = la_chunk_fwd_workspace_size(variant, dt, B, H, L, d_k, d_v, C)
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    else:
        if workspace.device != dev_ or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.la_chunk_fwd(VARIANTS[variant], dt, _dt(o), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                          _ptr(beta), _ptr(state_in), _ptr(z_in), _ptr(o), _ptr(state_out),
                          _ptr(z_out), B, H, L, d_k, d_v, C, _ptr(workspace), ws_bytes,
                          _stream(q.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_fwd")
    return o, state_out, z_out


def _fwd_args(variant, q, k, v, log_gate, beta, state_in, z_in, o, out_dtype, state_out, z_out,
              want_state, want_z):
    """Check the tensors of a forward call and allocate the missing outputs.
    Returns (B, H, L, d_k, d_v, o, state_out, z_out)."""
    import torch
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, d_k = q.shape
    d_v = v.shape[-1]
    _dt(q)
    f32, dev_ = torch.float32, q.device
    _check("k", k, (B, H, L, d_k), q.dtype, dev_, required=True)
    _check("v", v, (B, H, L, d_v), q.dtype, dev_, required=True)
    gate_shape = (B, H, L, d_k) if variant in _PER_CHANNEL else (B, H, L)
    _check("log_gate", log_gate, gate_shape, f32, dev_)
    _check("beta", beta, (B, H, L), f32, dev_)
    _check("state_in", state_in, (B, H, d_k, d_v), f32, dev_)
    _check("z_in", z_in, (B, H, d_k), f32, dev_)
    if o is not None:
        _check("o", o, (B, H, L, d_v), o.dtype, dev_)
    _check("state_out", state_out, (B, H, d_k, d_v), f32, dev_)
    _check("z_out", z_out, (B, H, d_k), f32, dev_)
    _check_device(dev_)
    if o is None:
        o = torch.empty((B, H, L, d_v), dtype=out_dtype or torch.float32, device=dev_)
    if want_state and state_out is None:
        state_out = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=dev_)
    if want_z and z_out is None:
        z_out = torch.empty((B, H, d_k), dtype=torch.float32, device=dev_)
    return B, H, L, d_k, d_v, o, state_out, z_out


def la_chunk_fwd_noalloc(variant: str, q, k, v, log_gate=None, beta=None, state_in=None, z_in=None,
                         *, C: int = 64, o=None, out_dtype=None, state_out=None, z_out=None,
                         want_state: bool = False, want_z: bool = False, stream=None) -> Tuple:
    """la_chunk_fwd without a workspace: the library's static per-device scratch
    holds the delta rule's per-chunk products (for callers that cannot allocate).
    Same arguments and results as la_chunk_fwd; pass o (and state_out, z_out) to
    keep the call itself free of allocations. Calls that overlap on one device race."""
    lib = load_library()
    B, H, L, d_k, d_v, o, state_out, z_out = _fwd_args(variant, q, k, v, log_gate, beta, state_in,
                                                       z_in, o, out_dtype, state_out, z_out,
                                                       want_state, want_z)
    st = lib.la_chunk_fwd_noalloc(VARIANTS[variant], _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(log_gate), _ptr(beta), _ptr(state_in), _ptr(z_in), _ptr(o),
                                  _ptr(state_out), _ptr(z_out), B, H, L, d_k, d_v, C,
                                  _stream(q.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_fwd_noalloc")
    return o, state_out, z_out


def la_decode_step(variant: str, q, k, v, log_gate, state, *, o=None, out_dtype=None, beta=None,
                   stream=None):
    """One decode step for [N, H] sequence-heads; ``state`` [N, H, d_k, d_v] fp32 is
    updated in place. Returns o [N, H, d_v] (fp32 unless out_dtype/o say bf16)."""
    import torch
    lib = load_library()
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [N, H, d]")
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    f32, dev_ = torch.float32, q.device
    _dt(q)
    _check("k", k, (N, H, d_k), q.dtype, dev_, required=True)
    _check("v", v, (N, H, d_v), q.dtype, dev_, required=True)
    _check("log_gate", log_gate, (N, H, d_k) if variant in _PER_CHANNEL else (N, H), f32, dev_)
    _check("beta", beta, (N, H), f32, dev_)
    _check("state", state, (N, H, d_k, d_v), f32, dev_, required=True)
    if o is not None:
        _check("o", o, (N, H, d_v), o.dtype, dev_)
    _check_device(dev_)
    if o is None:
        o = torch.empty((N, H, d_v), dtype=out_dtype or torch.float32, device=q.device)
    st = lib.la_decode_step(VARIANTS[variant], _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                            _ptr(beta), _ptr(state), _ptr(o), N, H, d_k, d_v,
                            _stream(q.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_decode_step")
    return o


def la_chunk_bwd_workspace_size(variant: str, dtype_code: int, B: int, H: int, L: int,
                                d_k: int, d_v: int, C: int = 64) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().la_chunk_bwd_workspace_size(VARIANTS[variant], dtype_code, B, H, L, d_k,
                                                    d_v, C, ctypes.byref(out))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_bwd_workspace_size")
    return out.value


def la_chunk_bwd(variant: str, q, k, v, d_o, log_gate=None, state_in=None, d_state_out=None, *,
                 beta=None, z_in=None, d_z_out=None, C: int = 64, want_d_log_gate: bool = True,
                 want_d_state_in: bool = False, want_d_beta: bool = True, want_d_z_in: bool = False,
                 workspace=None, stream=None) -> Tuple:
    """Backward pass of la_chunk_fwd ("plain", "normalized", "decay", or
    "gated_delta" and "vector_decay" in bf16).

    q, k: [B, H, L, d_k]; v, d_o: [B, H, L, d_v] (bf16 or fp32, one dtype);
    log_gate: [B, H, L] fp32 ("decay"; optional for "gated_delta"; [B, H, L, d_k]
    for "vector_decay"); beta: [B, H, L]
    fp32 ("gated_delta"); state_in, d_state_out: [B, H, d_k, d_v] fp32.
    Returns (dq, dk, dv, d_log_gate or None, d_state_in or None), all fp32, and for
    "gated_delta" d_beta (or None) as a sixth entry. "normalized" takes z_in and
    d_z_out ([B, H, d_k] fp32) and returns d_z_in (or None) as the sixth entry.
    """
    import torch
    lib = load_library()
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, d_k = q.shape
    d_v = v.shape[-1]
    dt = _dt(q)
    dev_, f32 = q.device, torch.float32
    gdn = variant == "gated_delta"
    _check("k", k, (B, H, L, d_k), q.dtype, dev_, required=True)
    _check("v", v, (B, H, L, d_v), q.dtype, dev_, required=True)
    _check("d_o", d_o, (B, H, L, d_v), q.dtype, dev_, required=True)
    gshape = (B, H, L, d_k) if variant in _PER_CHANNEL else (B, H, L)
    _check("log_gate", log_gate, gshape, f32, dev_)
    _check("beta", beta, (B, H, L), f32, dev_, required=gdn)
    _check("state_in", state_in, (B, H, d_k, d_v), f32, dev_)
    _check("d_state_out", d_state_out, (B, H, d_k, d_v), f32, dev_)
    _check("z_in", z_in, (B, H, d_k), f32, dev_)
    _check("d_z_out", d_z_out, (B, H, d_k), f32, dev_)
    if not gdn and beta is not None:
        raise ValueError("beta is taken by the gated delta rule only")
    norm = variant == "normalized"
    if not norm and (z_in is not None or d_z_out is not None):
        raise ValueError("z_in and d_z_out are taken by the normalized variant only")
    _check_device(dev_)
    if workspace is not None and (workspace.device != dev_ or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    dq = torch.empty((B, H, L, d_k), dtype=torch.float32, device=dev_)
    dk = torch.empty((B, H, L, d_k), dtype=torch.float32, device=dev_)
    dv = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev_)
    dlg = (torch.empty(gshape, dtype=torch.float32, device=dev_)
           if (log_gate is not None and variant in ("decay", "gated_delta", "vector_decay") and want_d_log_gate)
           else None)
    dbe = torch.empty((B, H, L), dtype=torch.float32, device=dev_) if (gdn and want_d_beta) else None
    dsi = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=dev_) if want_d_state_in else None
    dzi = torch.empty((B, H, d_k), dtype=torch.float32, device=dev_) if (norm and want_d_z_in) else None
    if workspace is None:
        ws_bytes = la_chunk_bwd_workspace_size(variant, dt, B, H, L, d_k, d_v, C)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev_)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.la_chunk_bwd(VARIANTS[variant], dt, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(beta),
                          _ptr(state_in), _ptr(z_in), _ptr(d_o), _ptr(d_state_out), _ptr(d_z_out), _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(dlg), _ptr(dbe), _ptr(dsi), _ptr(dzi), B, H, L, d_k, d_v, C,
                          _ptr(workspace), ws_bytes, _stream(dev_, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_bwd")
    if gdn:
        return dq, dk, dv, dlg, dsi, dbe
    if norm:
        return dq, dk, dv, None, dsi, dzi
    return dq, dk, dv, dlg, dsi


def la_chunk_fwd_conv_workspace_size(variant: str, dtype_code: int, B: int, H: int, L: int, d_k: int,
                                     d_v: int, C: int = 64, K: int = 4) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().la_chunk_fwd_conv_workspace_size(VARIANTS[variant], dtype_code, B, H, L, d_k, d_v, C,
                                                         K, ctypes.byref(out))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_fwd_conv_workspace_size")
    return out.value


def la_chunk_fwd_conv(variant: str, q, k, v, w_q, w_k, w_v, log_gate=None, beta=None, state_in=None, *,
                      q_win_in=None, k_win_in=None, v_win_in=None, want_windows: bool = False,
                      q_win_out=None, k_win_out=None, v_win_out=None, C: int = 64,
                      want_state: bool = False, out_dtype=None, o=None, state_out=None, workspace=None,
                      stream=None) -> Tuple:
    """The gated delta rule's forward with the short convolution of q, k, v fused in
    front (raw bf16 inputs; taps w_*: [H, d, K] fp32; windows [B, H, K-1, d] bf16).

    Returns (o, state_out or None, (q_win, k_win, v_win) or None).
    """
    import torch
    lib = load_library()
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, d_k = q.shape
    d_v = v.shape[-1]
    K = w_q.shape[-1]
    dt = _dt(q)
    dev_, f32 = q.device, torch.float32
    _check("k", k, (B, H, L, d_k), q.dtype, dev_, required=True)
    _check("v", v, (B, H, L, d_v), q.dtype, dev_, required=True)
    _check("w_q", w_q, (H, d_k, K), f32, dev_, required=True)
    _check("w_k", w_k, (H, d_k, K), f32, dev_, required=True)
    _check("w_v", w_v, (H, d_v, K), f32, dev_, required=True)
    _check("log_gate", log_gate, (B, H, L), f32, dev_)
    _check("beta", beta, (B, H, L), f32, dev_, required=L > 0)
    _check("state_in", state_in, (B, H, d_k, d_v), f32, dev_)
    for nm, x, d in (("q_win_in", q_win_in, d_k), ("k_win_in", k_win_in, d_k), ("v_win_in", v_win_in, d_v),
                     ("q_win_out", q_win_out, d_k), ("k_win_out", k_win_out, d_k), ("v_win_out", v_win_out, d_v)):
        _check(nm, x, (B, H, K - 1, d), q.dtype, dev_)
    _check_device(dev_)
    if o is None:
        o = torch.empty((B, H, L, d_v), dtype=out_dtype if out_dtype is not None else torch.float32, device=dev_)
    elif o.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o must be float32 or bfloat16")
    _check("o", o, (B, H, L, d_v), o.dtype, dev_)
    s_out = state_out
    if s_out is None and want_state:
        s_out = torch.empty((B, H, d_k, d_v), dtype=f32, device=dev_)
    _check("state_out", s_out, (B, H, d_k, d_v), f32, dev_)
    if want_windows:
        q_win_out = q_win_out if q_win_out is not None else torch.empty((B, H, K - 1, d_k), dtype=q.dtype, device=dev_)
        k_win_out = k_win_out if k_win_out is not None else torch.empty((B, H, K - 1, d_k), dtype=q.dtype, device=dev_)
        v_win_out = v_win_out if v_win_out is not None else torch.empty((B, H, K - 1, d_v), dtype=q.dtype, device=dev_)
    if workspace is None:
        ws_bytes = la_chunk_fwd_conv_workspace_size(variant, dt, B, H, L, d_k, d_v, C, K)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev_)
    elif workspace.device != dev_ or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.la_chunk_fwd_conv(VARIANTS[variant], dt, _dt(o), _ptr(q), _ptr(k), _ptr(v), _ptr(w_q), _ptr(w_k),
                               _ptr(w_v), K, _ptr(q_win_in), _ptr(k_win_in), _ptr(v_win_in), _ptr(q_win_out),
                               _ptr(k_win_out), _ptr(v_win_out), _ptr(log_gate), _ptr(beta), _ptr(state_in),
                               _ptr(o), _ptr(s_out), B, H, L, d_k, d_v, C, _ptr(workspace), ws_bytes,
                               _stream(dev_, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_chunk_fwd_conv")
    wins = (q_win_out, k_win_out, v_win_out) if want_windows else None
    return o, s_out, wins


def la_short_conv(q=None, k=None, v=None, w_q=None, w_k=None, w_v=None, *, q_state_in=None,
                  k_state_in=None, v_state_in=None, q_out=None, k_out=None, v_out=None,
                  q_state_out=None, k_state_out=None, v_state_out=None, want_state: bool = False,
                  stream=None) -> Tuple:
    """Causal depthwise short convolution of any of q, k, v in one launch.

    q, k: [B, H, L, d_k]; v: [B, H, L, d_v] (bf16 or fp32, all the same dtype);
    w_*: [H, d, K] fp32 taps (tap tau multiplies the input tau tokens back);
    *_state_in: [B, H, K-1, d] windows of preceding inputs (None = zeros).
    Returns (q_out, k_out, v_out, q_state_out, k_state_out, v_state_out); entries
    of skipped tensors are None, windows are None unless requested (want_state or
    a passed *_state_out, which may be the same tensor's *_state_in).
    """
    import torch
    lib = load_library()
    xs = [q, k, v]
    ws = [w_q, w_k, w_v]
    given = [x for x in xs if x is not None]
    if not given or any((x is None) != (w is None) for x, w in zip(xs, ws)):
        raise ValueError("la_short_conv needs at least one of q, k, v, each with its taps")
    ref = given[0]
    if ref.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L = ref.shape[:3]
    d_k = q.shape[-1] if q is not None else (k.shape[-1] if k is not None else 8)
    d_v = v.shape[-1] if v is not None else 8
    K = next(w for w, x in zip(ws, xs) if x is not None).shape[-1]
    outs = [q_out, k_out, v_out]
    sins = [q_state_in, k_state_in, v_state_in]
    souts = [q_state_out, k_state_out, v_state_out]
    dev_, f32 = ref.device, torch.float32
    _dt(ref)
    for i, (nm, x, w) in enumerate(zip("qkv", xs, ws)):
        if x is None:
            for extra, what in ((sins[i], "state_in"), (outs[i], "out"), (souts[i], "state_out")):
                if extra is not None:
                    raise ValueError(f"{nm}_{what} given without {nm}")
            continue
        d = d_v if nm == "v" else d_k
        _check(nm, x, (B, H, L, d), ref.dtype, dev_, required=True)
        _check(f"w_{nm}", w, (H, d, K), f32, dev_, required=True)
        _check(f"{nm}_state_in", sins[i], (B, H, K - 1, d), ref.dtype, dev_)
        _check(f"{nm}_out", outs[i], (B, H, L, d), ref.dtype, dev_)
        _check(f"{nm}_state_out", souts[i], (B, H, K - 1, d), ref.dtype, dev_)
    _check_device(dev_)
    for i, x in enumerate(xs):
        if x is None:
            continue
        if outs[i] is None:
            outs[i] = torch.empty_like(x)
        if want_state and souts[i] is None:
            souts[i] = torch.empty((B, H, K - 1, x.shape[-1]), dtype=x.dtype, device=x.device)
    st = lib.la_short_conv(_dt(ref), *[_ptr(x) for x in xs], *[_ptr(w) for w in ws],
                           *[_ptr(x) for x in sins], *[_ptr(x) for x in outs],
                           *[_ptr(x) for x in souts], B, H, L, d_k, d_v, K,
                           _stream(ref.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_short_conv")
    return (*outs, *souts)


__all__ = ["la_chunk_fwd", "la_chunk_fwd_workspace_size", "la_chunk_fwd_noalloc", "la_chunk_bwd", "la_chunk_bwd_workspace_size",
           "la_chunk_fwd_conv", "la_chunk_fwd_conv_workspace_size",
           "la_decode_step", "la_short_conv",
           "la_status_str", "la_abi_version", "LinAttnError", "VARIANTS", "load_library"]
