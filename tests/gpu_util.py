"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP
path through the C ABI, run the oracle on the same values, compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import chunkwise_linear_rnn_causal_amd as la
import oracle
import workloads as W

# Tolerances: max |err| <= TOL * RMS(reference), over the whole compared tensor.
# bf16 inputs: 2e-2; fp32 inputs: 1e-4 (the normwise form of "1e-4 relative").
TOL = {"bf16": 2e-2, "f32": 1e-4}


def dev(x: np.ndarray | None, device="cuda"):
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t is not None else None


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = math.sqrt(float(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(got - ref))) / (rms if rms > 0 else 1.0)


def assert_close(got, ref, tol, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max|err|/RMS = {e:.3e} > {tol:.1e}"
    return e


def gpu_chunk(inp: W.ChunkInputs, C: int, want_state=True, state_in=True, z_in=True, stream=None):
    """Run la_chunk_fwd on the inputs; returns (o, state, z) as float64 numpy."""
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    lg, be = dev(inp.log_gate), dev(inp.beta)
    s_in = dev(inp.state_in) if state_in else None
    zi = dev(inp.z_in) if (z_in and inp.variant == "normalized") else None
    want_z = inp.variant == "normalized"
    o, s, z = la.la_chunk_fwd(inp.variant, q, k, v, lg, be, s_in, zi, C=C, want_state=want_state,
                              want_z=want_z, stream=stream)
    torch.cuda.synchronize()
    return host64(o), host64(s), host64(z)


def oracle_chunk(inp: W.ChunkInputs, state_in=True, z_in=True, threads=0):
    o, s, z = oracle.forward(inp.variant, inp.f64("q"), inp.f64("k"), inp.f64("v"),
                             log_gate=inp.f64("log_gate"), beta=inp.f64("beta"),
                             state_in=inp.f64("state_in") if state_in else None,
                             z_in=inp.f64("z_in") if (z_in and inp.variant == "normalized") else None,
                             threads=threads)
    return o, s, z
