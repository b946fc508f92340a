"""fp64 CPU oracle for causal linear attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and its
binding in ``chunkwise_linear_rnn_causal_amd``) never imports, links or calls it,
and the oracle imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C, float64, naive per-token recurrence;
see that file's header for the definitions and the passages they follow). This
module is a ctypes wrapper: it converts arrays to contiguous float64 and calls it.
All functions here are pinned by ``tests/test_oracle_pins.py``; no function is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

VARIANT_ID = {"plain": 0, "normalized": 1, "decay": 2, "gated_delta": 3, "vector_decay": 4, "kda": 5}

_lib = None
_lib_path = None


def load(path: Optional[str] = None):
    """Load (building first if missing or stale) the oracle shared library."""
    global _lib, _lib_path
    path = path or _build.LIB
    if _lib is not None and _lib_path == path:
        return _lib
    if path == _build.LIB and _build.stale():
        _build.build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.oracle_forward.argtypes = [ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                   L, L, L, L, ctypes.c_int]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_decode_step.argtypes = [ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, L, L, L, ctypes.c_int]
    lib.oracle_decode_step.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                    L, L, L, L, ctypes.c_int]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_backward_gdn.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                        L, L, L, L, ctypes.c_int]
    lib.oracle_backward_gdn.restype = ctypes.c_int
    lib.oracle_backward_norm.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                         ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_int]
    lib.oracle_backward_norm.restype = ctypes.c_int
    lib.oracle_short_conv.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, ctypes.c_int]
    lib.oracle_short_conv.restype = ctypes.c_int
    lib.oracle_abi_version.restype = ctypes.c_int
    _lib, _lib_path = lib, path
    return lib


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _c64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def forward(variant: str, q, k, v, log_gate=None, beta=None, state_in=None, z_in=None,
            threads: int = 0, lib=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Run the recurrence over every leading (batch, head) slice.

    q, k: [..., L, dk]; v: [..., L, dv]; log_gate, beta: [..., L]
    ("vector_decay", "kda": log_gate [..., L, dk]); state_in: [..., dk, dv]; z_in: [..., dk]. Returns (o [..., L, dv],
    state_out [..., dk, dv], z_out [..., dk]) in float64.
    """
    lib = lib or load()
    q, k, v = _c64(q), _c64(k), _c64(v)
    lead = q.shape[:-2]
    L, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    assert k.shape == q.shape and v.shape[:-1] == q.shape[:-1]
    lg, be = _c64(log_gate), _c64(beta)
    s_in, zi = _c64(state_in), _c64(z_in)
    lg_shape = lead + ((L, dk) if variant in ("vector_decay", "kda") else (L,))
    for x, shp in ((lg, lg_shape), (be, lead + (L,)), (s_in, lead + (dk, dv)), (zi, lead + (dk,))):
        assert x is None or x.shape == shp, (x.shape, shp)
    o = np.zeros(lead + (L, dv), np.float64)
    s_out = np.zeros(lead + (dk, dv), np.float64)
    z_out = np.zeros(lead + (dk,), np.float64)
    st = lib.oracle_forward(VARIANT_ID[variant], _p(q), _p(k), _p(v), _p(lg), _p(be), _p(s_in),
                            _p(zi), _p(o), _p(s_out), _p(z_out), BH, L, dk, dv, int(threads))
    if st != 0:
        raise ValueError(f"oracle_forward failed with status {st}")
    return o, s_out, z_out


def decode_step(variant: str, q, k, v, log_gate, state, beta=None, threads: int = 0, lib=None,
                copy: bool = True):
    """One in-place decode step on a copy of ``state``; returns (o, new_state).

    q, k: [..., dk]; v: [..., dv]; log_gate, beta: [...] ("vector_decay", "kda":
    log_gate [..., dk]); state: [..., dk, dv].
    beta is required for "gated_delta" (log_gate may then be None: alpha = 1).
    copy=False updates ``state`` itself (a C-contiguous float64 array) in place.
    """
    lib = lib or load()
    q, k, v = _c64(q), _c64(k), _c64(v)
    lead = q.shape[:-1]
    dk, dv = q.shape[-1], v.shape[-1]
    NH = int(np.prod(lead)) if lead else 1
    if copy:
        S = np.array(state, dtype=np.float64, copy=True, order="C")
    else:
        assert state.dtype == np.float64 and state.flags.c_contiguous
        S = state
    lg = _c64(log_gate)
    be = _c64(beta)
    o = np.zeros(lead + (dv,), np.float64)
    st = lib.oracle_decode_step(VARIANT_ID[variant], _p(q), _p(k), _p(v), _p(lg), _p(be), _p(S),
                                _p(o), NH, dk, dv, int(threads))
    if st != 0:
        raise ValueError(f"oracle_decode_step failed with status {st}")
    return o, S


def short_conv(x, w, state_in=None, threads: int = 0, lib=None):
    """Causal depthwise short convolution over tokens (see ``oracle_short_conv``).

    x: [B, H, L, d]; w: [H, d, K] (tap tau multiplies the input tau tokens back);
    state_in: [B, H, K-1, d] previous inputs, oldest first (None = zeros).
    Returns (y [B, H, L, d], state_out [B, H, K-1, d]) in float64.
    """
    lib = lib or load()
    x, w = _c64(x), _c64(w)
    B, H, L, d = x.shape
    K = w.shape[-1]
    assert w.shape == (H, d, K), (w.shape, (H, d, K))
    s_in = _c64(state_in)
    assert s_in is None or s_in.shape == (B, H, K - 1, d), s_in.shape
    y = np.zeros((B, H, L, d), np.float64)
    s_out = np.zeros((B, H, K - 1, d), np.float64)
    st = lib.oracle_short_conv(_p(x), _p(w), _p(s_in), _p(y), _p(s_out), B, H, L, d, K, int(threads))
    if st != 0:
        raise ValueError(f"oracle_short_conv failed with status {st}")
    return y, s_out


def backward(variant: str, q, k, v, do, log_gate=None, state_in=None, d_state_out=None,
             threads: int = 0, lib=None, beta=None, z_in=None, d_z_out=None):
    """Gradients through the forward recurrence (see ``oracle_backward`` and, for
    "gated_delta", ``oracle_backward_gdn``).

    q, k: [..., L, dk]; v, do: [..., L, dv]; log_gate: [..., L] ("vector_decay":
    [..., L, dk]); state_in, d_state_out: [..., dk, dv]; beta: [..., L]
    ("gated_delta" only). Returns (dq, dk, dv, d_log_gate or None, d_state_in) in
    float64, and for "gated_delta" d_beta as a sixth entry. For "normalized" (z_in,
    d_z_out: [..., dk]) the sixth entry is d_z_in and the fourth is None.
    """
    lib = lib or load()
    if variant == "gated_delta":
        return _backward_gdn(q, k, v, do, log_gate, beta, state_in, d_state_out, threads, lib)
    if variant == "normalized":
        return _backward_norm(q, k, v, do, state_in, z_in, d_state_out, d_z_out, threads, lib)
    q, k, v, do = _c64(q), _c64(k), _c64(v), _c64(do)
    lead = q.shape[:-2]
    L, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    lg, s_in, dso = _c64(log_gate), _c64(state_in), _c64(d_state_out)
    dq = np.zeros(q.shape, np.float64)
    dkk = np.zeros(k.shape, np.float64)
    dvv = np.zeros(v.shape, np.float64)
    dlg = np.zeros(lg.shape, np.float64) if lg is not None else None
    dsi = np.zeros(lead + (dk, dv), np.float64)
    st = lib.oracle_backward(VARIANT_ID[variant], _p(q), _p(k), _p(v), _p(lg), _p(s_in), _p(do), _p(dso),
                             _p(dq), _p(dkk), _p(dvv), _p(dlg), _p(dsi), BH, L, dk, dv, int(threads))
    if st != 0:
        raise ValueError(f"oracle_backward failed with status {st}")
    return dq, dkk, dvv, dlg, dsi


def _backward_gdn(q, k, v, do, log_gate, beta, state_in, d_state_out, threads, lib):
    q, k, v, do = _c64(q), _c64(k), _c64(v), _c64(do)
    lead = q.shape[:-2]
    L, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    lg, be, s_in, dso = _c64(log_gate), _c64(beta), _c64(state_in), _c64(d_state_out)
    assert be is not None and be.shape == lead + (L,)
    dq = np.zeros(q.shape, np.float64)
    dkk = np.zeros(k.shape, np.float64)
    dvv = np.zeros(v.shape, np.float64)
    dlg = np.zeros(lg.shape, np.float64) if lg is not None else None
    dbe = np.zeros(be.shape, np.float64)
    dsi = np.zeros(lead + (dk, dv), np.float64)
    st = lib.oracle_backward_gdn(_p(q), _p(k), _p(v), _p(lg), _p(be), _p(s_in), _p(do), _p(dso),
                                 _p(dq), _p(dkk), _p(dvv), _p(dlg), _p(dbe), _p(dsi), BH, L, dk, dv,
                                 int(threads))
    if st != 0:
        raise ValueError(f"oracle_backward_gdn failed with status {st}")
    return dq, dkk, dvv, dlg, dsi, dbe


def _backward_norm(q, k, v, do, state_in, z_in, d_state_out, d_z_out, threads, lib):
    q, k, v, do = _c64(q), _c64(k), _c64(v), _c64(do)
    lead = q.shape[:-2]
    L, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    s_in, zi, dso, dzo = _c64(state_in), _c64(z_in), _c64(d_state_out), _c64(d_z_out)
    dq = np.zeros(q.shape, np.float64)
    dkk = np.zeros(k.shape, np.float64)
    dvv = np.zeros(v.shape, np.float64)
    dsi = np.zeros(lead + (dk, dv), np.float64)
    dzi = np.zeros(lead + (dk,), np.float64)
    st = lib.oracle_backward_norm(_p(q), _p(k), _p(v), _p(s_in), _p(zi), _p(do), _p(dso), _p(dzo), _p(dq),
                                  _p(dkk), _p(dvv), _p(dsi), _p(dzi), BH, L, dk, dv, int(threads))
    if st != 0:
        raise ValueError(f"oracle_backward_norm failed with status {st}")
    return dq, dkk, dvv, None, dsi, dzi
