"""Seeded synthetic inputs for the causal linear-attention workloads.

This module is shared by the tests, the benchmark and the oracle checks. It holds
none of the method's arithmetic: it only draws random tensors, applies the
input-side transforms each workload prescribes (the elu(x)+1 feature map, per-token
L2 normalisation, sigmoid gates stored as log-gates) and rounds to the storage
dtype. The feature map is applied here, on the host, because the pages place it
before the attention product (ai-master glossary "Linear Attention", kernel-map
bullet; wln20 "LLM注意力优化：线性注意力", first section).

Random streams. Every (tensor, b, h) slice of a chunk-forward workload has its own
PCG64 stream seeded with SeedSequence([seed, tag, b, h]); tags are
q=1, k=2, v=3, gate=4, beta=5, state=6. A slice can therefore be regenerated alone
(the oracle checks sampled heads at full size) and the full tensors can be filled
from several threads. Decode workloads draw their initial state from
SeedSequence([seed, 6, n]) per sequence n and the inputs of step i from
SeedSequence([seed, tag, 1000 + i]) as whole [N, H, d] arrays. Short-convolution
inputs draw each (tensor, b, h) slice like the chunk workloads (tags 1-3), their
taps per tensor from SeedSequence([seed, 7, tensor]) and their incoming windows
per slice from SeedSequence([seed, 8, tensor, b, h]).

bf16 values are produced by round-to-nearest-even from float32 and kept as their
raw uint16 bit patterns; ``bf16_bits_to_f32`` widens them exactly.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_GATE, TAG_BETA, TAG_STATE = 1, 2, 3, 4, 5, 6
TAG_CONV_W, TAG_CONV_WINDOW = 7, 8
TAG_DOUT = 9

VARIANTS = ("plain", "normalized", "decay", "gated_delta", "vector_decay", "kda")

# The five workloads, each named by what it is. "recipe" selects the input
# distribution (see _draw_slice); sizes are the ones the workloads are quoted at.
CONFIGS: Dict[str, dict] = {
    "plain_f32_b1h1_l256_d32": dict(
        kind="chunk", variant="plain", dtype="f32", B=1, H=1, L=256, dk=32, dv=32, C=64,
        recipe="gauss_scaled"),
    "normalized_bf16_b8h16_l2048_d64": dict(
        kind="chunk", variant="normalized", dtype="bf16", B=8, H=16, L=2048, dk=64, dv=64, C=64,
        recipe="elu1"),
    "decay_bf16_b4h32_l8192_d128": dict(
        kind="chunk", variant="decay", dtype="bf16", B=4, H=32, L=8192, dk=128, dv=128, C=64,
        recipe="gauss_scaled_gate", o_dtype="bf16"),
    "decode_decay_bf16_n512h32_d128": dict(
        kind="decode", variant="decay", dtype="bf16", N=512, H=32, dk=128, dv=128, steps=100,
        recipe="decode"),
    "gated_delta_bf16_b2h16_l8192_d128": dict(
        kind="chunk", variant="gated_delta", dtype="bf16", B=2, H=16, L=8192, dk=128, dv=128, C=64,
        recipe="gdn"),
    # the decay workload's shapes with one gate per key channel (GLA-style gates)
    "vector_decay_bf16_b4h32_l8192_d128": dict(
        kind="chunk", variant="vector_decay", dtype="bf16", B=4, H=32, L=8192, dk=128, dv=128, C=64,
        recipe="gla"),
    # Kimi Delta Attention at the delta-rule workload's shapes: its inputs, with the
    # gate drawn independently for every key channel
    "kda_bf16_b2h16_l8192_d128": dict(
        kind="chunk", variant="kda", dtype="bf16", B=2, H=16, L=8192, dk=128, dv=128, C=64,
        recipe="kda"),
    # the backward pass of the decay workload (output gradient dO ~ N(0, 1))
    "decay_bwd_bf16_b4h32_l8192_d128": dict(
        kind="bwd", variant="decay", dtype="bf16", B=4, H=32, L=8192, dk=128, dv=128, C=64,
        recipe="gauss_scaled_gate"),
    # the backward pass of the delta-rule workload (output gradient dO ~ N(0, 1))
    "gated_delta_bwd_bf16_b2h16_l8192_d128": dict(
        kind="bwd", variant="gated_delta", dtype="bf16", B=2, H=16, L=8192, dk=128, dv=128, C=64,
        recipe="gdn"),
    # the backward pass of the per-key-channel decay workload (output gradient dO ~ N(0, 1))
    "vector_decay_bwd_bf16_b4h32_l8192_d128": dict(
        kind="bwd", variant="vector_decay", dtype="bf16", B=4, H=32, L=8192, dk=128, dv=128, C=64,
        recipe="gla"),
    # the backward pass of the normalized workload (output gradient dO ~ N(0, 1))
    "normalized_bwd_bf16_b8h16_l2048_d64": dict(
        kind="bwd", variant="normalized", dtype="bf16", B=8, H=16, L=2048, dk=64, dv=64, C=64,
        recipe="elu1"),
    # the delta-rule workload with a K = 4 short convolution of q, k, v fused in front
    "conv_gated_delta_bf16_b2h16_l8192_d128_k4": dict(
        kind="convfwd", variant="gated_delta", dtype="bf16", B=2, H=16, L=8192, dk=128, dv=128, C=64, K=4,
        recipe="gdn"),
    # the short convolution in front of the delta rule, at that workload's q, k, v shapes
    "short_conv_qkv_bf16_b2h16_l8192_d128_k4": dict(
        kind="conv", dtype="bf16", B=2, H=16, L=8192, dk=128, dv=128, K=4, recipe="conv"),
}

# Recipe used for each variant when a test builds a small case of that variant.
DEFAULT_RECIPE = {
    "plain": "gauss_scaled",
    "normalized": "elu1",
    "decay": "gauss_scaled_gate",
    "gated_delta": "gdn",
    "vector_decay": "gla",
    "kda": "kda",
}


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def stream(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def _sigmoid_log(g: np.ndarray) -> np.ndarray:
    """log(sigmoid(g)) evaluated in float64, stored as float32."""
    g = g.astype(np.float64)
    return (-np.log1p(np.exp(-g))).astype(np.float32)


def _sigmoid(g: np.ndarray) -> np.ndarray:
    g = g.astype(np.float64)
    return (1.0 / (1.0 + np.exp(-g))).astype(np.float32)


def _l2_rows(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (x64 / np.linalg.norm(x64, axis=-1, keepdims=True)).astype(np.float32)


def _elu1(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return np.where(x64 > 0, x64 + 1.0, np.exp(np.minimum(x64, 0.0))).astype(np.float32)


# ----------------------------------------------------------------------------
# Chunk-forward workloads
# ----------------------------------------------------------------------------
def _draw_slice(recipe: str, tag: int, seed: int, b: int, h: int, L: int, d: int) -> np.ndarray:
    """One (b, h) slice of one tensor as float32, before storage rounding."""
    rng = stream(seed, tag, b, h)
    if tag in (TAG_Q, TAG_K, TAG_V):
        x = rng.standard_normal((L, d), dtype=np.float32)
        if recipe in ("gauss_scaled", "gauss_scaled_gate", "gla", "gla_strong"):
            return (x / np.float32(math.sqrt(d))).astype(np.float32)
        if recipe == "elu1":
            return _elu1(x) if tag in (TAG_Q, TAG_K) else x
        if recipe in ("gdn", "kda", "kda_gla", "kda_strong"):
            return _l2_rows(x) if tag in (TAG_Q, TAG_K) else x
        raise ValueError(recipe)
    if tag == TAG_GATE:
        if recipe == "gauss_scaled_gate" or recipe == "gdn":
            return _sigmoid_log(rng.normal(4.0, 1.0, size=L))
        if recipe == "gla":
            # alpha = sigmoid(x)^(1/tau) per key channel, tau = 16: l = log sigmoid(x) / 16
            return (_sigmoid_log(rng.normal(0.0, 1.0, size=(L, d))).astype(np.float64) / 16.0).astype(np.float32)
        if recipe == "gla_strong" or recipe == "kda_strong":
            # per-channel gates spread over the whole supported range [-10, 0]
            return (-10.0 * rng.random((L, d)) ** 3).astype(np.float32)
        if recipe == "kda":
            # the delta rule's gate alpha = sigmoid(N(4, 1)), one per key channel
            return _sigmoid_log(rng.normal(4.0, 1.0, size=(L, d)))
        if recipe == "kda_gla":
            return (_sigmoid_log(rng.normal(0.0, 1.0, size=(L, d))).astype(np.float64) / 16.0).astype(np.float32)
        raise ValueError(recipe)
    if tag == TAG_BETA:
        return _sigmoid(rng.normal(0.0, 1.0, size=L))
    raise ValueError(tag)


KDA_RECIPES = ("kda", "kda_gla", "kda_strong")


def recipe_has_gate(recipe: str) -> bool:
    return recipe in ("gauss_scaled_gate", "gdn", "gla", "gla_strong") + KDA_RECIPES


def recipe_gate_width(recipe: str, dk: int) -> int:
    """Gates per token: one (scalar decay) or one per key channel."""
    return dk if recipe in ("gla", "gla_strong") + KDA_RECIPES else 1


def recipe_has_beta(recipe: str) -> bool:
    return recipe in ("gdn",) + KDA_RECIPES


@dataclass
class ChunkInputs:
    """Inputs of one chunk-forward call.

    q, k: [B, H, L, dk]; v: [B, H, L, dv] in the storage dtype (float32, or uint16
    bf16 bits). log_gate, beta: [B, H, L] float32 or None. state_in: [B, H, dk, dv]
    float32 or None.
    """
    variant: str
    dtype: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_gate: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    state_in: Optional[np.ndarray] = None
    z_in: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    def f64(self, name: str) -> Optional[np.ndarray]:
        """Exact float64 copy of a stored tensor (what the GPU reads)."""
        x = getattr(self, name)
        if x is None:
            return None
        if x.dtype == np.uint16:
            return bf16_bits_to_f32(x).astype(np.float64)
        return x.astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32.astype(np.float32)


def make_chunk_inputs(variant: str, dtype: str, B: int, H: int, L: int, dk: int, dv: int,
                      seed: int = 0, recipe: Optional[str] = None,
                      heads: Optional[Sequence[Tuple[int, int]]] = None,
                      threads: Optional[int] = None, with_state: bool = False,
                      with_z: bool = False) -> ChunkInputs:
    """Build seeded inputs of one chunk-forward call.

    heads: if given, only these (b, h) slices are drawn and the result has shape
    [1, len(heads), ...] (used to regenerate sampled heads of a full-size case).
    with_state / with_z: also draw an initial state (N(0, 0.1^2) fp32) and, for the
    normalized variant, a positive initial normalizer.
    """
    recipe = recipe or DEFAULT_RECIPE[variant]
    pairs = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    nb, nh = (1, len(pairs)) if heads is not None else (B, H)
    sdt = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((nb * nh, L, dk), sdt)
    k = np.empty((nb * nh, L, dk), sdt)
    v = np.empty((nb * nh, L, dv), sdt)
    has_gate = recipe_has_gate(recipe)
    has_beta = recipe_has_beta(recipe)
    gw = recipe_gate_width(recipe, dk)
    lg = (np.empty((nb * nh, L, gw) if gw > 1 else (nb * nh, L), np.float32)) if has_gate else None
    be = np.empty((nb * nh, L), np.float32) if has_beta else None

    def fill(i: int) -> None:
        b, h = pairs[i]
        q[i] = _store(_draw_slice(recipe, TAG_Q, seed, b, h, L, dk), dtype)
        k[i] = _store(_draw_slice(recipe, TAG_K, seed, b, h, L, dk), dtype)
        v[i] = _store(_draw_slice(recipe, TAG_V, seed, b, h, L, dv), dtype)
        if lg is not None:
            lg[i] = _draw_slice(recipe, TAG_GATE, seed, b, h, L, gw)
        if be is not None:
            be[i] = _draw_slice(recipe, TAG_BETA, seed, b, h, L, 1)

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    if len(pairs) > 1 and nthr > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(len(pairs))))
    else:
        for i in range(len(pairs)):
            fill(i)

    st = None
    z = None
    if with_state:
        st = np.empty((nb * nh, dk, dv), np.float32)
        for i, (b, h) in enumerate(pairs):
            st[i] = stream(seed, TAG_STATE, b, h).normal(0.0, 0.1, size=(dk, dv)).astype(np.float32)
        st = st.reshape(nb, nh, dk, dv)
    if with_z:
        z = np.empty((nb * nh, dk), np.float32)
        for i, (b, h) in enumerate(pairs):
            z[i] = (1.0 + stream(seed, TAG_STATE + 100, b, h).random(dk)).astype(np.float32)
        z = z.reshape(nb, nh, dk)

    return ChunkInputs(
        variant=variant, dtype=dtype, B=nb, H=nh, L=L, dk=dk, dv=dv,
        q=q.reshape(nb, nh, L, dk), k=k.reshape(nb, nh, L, dk), v=v.reshape(nb, nh, L, dv),
        log_gate=None if lg is None else lg.reshape((nb, nh) + lg.shape[1:]),
        beta=None if be is None else be.reshape(nb, nh, L),
        state_in=st, z_in=z, meta=dict(seed=seed, recipe=recipe, heads=pairs))


def config_chunk_inputs(name: str, seed: int = 0, heads=None, threads=None) -> ChunkInputs:
    c = CONFIGS[name]
    assert c["kind"] == "chunk", name
    return make_chunk_inputs(c["variant"], c["dtype"], c["B"], c["H"], c["L"], c["dk"], c["dv"],
                             seed=seed, recipe=c["recipe"], heads=heads, threads=threads)


# ----------------------------------------------------------------------------
# Decode workload
# ----------------------------------------------------------------------------
@dataclass
class DecodeStep:
    q: np.ndarray          # [N, H, dk] storage dtype
    k: np.ndarray          # [N, H, dk]
    v: np.ndarray          # [N, H, dv]
    log_gate: np.ndarray   # [N, H] float32
    beta: Optional[np.ndarray] = None  # [N, H] float32 (delta rule), when requested


def make_decode_state(N: int, H: int, dk: int, dv: int, seed: int = 0,
                      threads: Optional[int] = None) -> np.ndarray:
    """Initial fp32 state [N, H, dk, dv], entries N(0, 0.1^2)."""
    S = np.empty((N, H, dk, dv), np.float32)

    def fill(n: int) -> None:
        S[n] = stream(seed, TAG_STATE, n).normal(0.0, 0.1, size=(H, dk, dv)).astype(np.float32)

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill, range(N)))
    return S


def make_decode_step(N: int, H: int, dk: int, dv: int, step: int, seed: int = 0,
                     dtype: str = "bf16", with_beta: bool = False) -> DecodeStep:
    """Inputs of decode step ``step``: q,k,v ~ N(0,1)/sqrt(dk); gate log sigmoid(N(4,1));
    with_beta: also beta = sigmoid(N(0,1)) (delta rule)."""
    def qkv(tag: int, d: int) -> np.ndarray:
        x = stream(seed, tag, 1000 + step).standard_normal((N, H, d), dtype=np.float32)
        return _store((x / np.float32(math.sqrt(dk))).astype(np.float32), dtype)

    q = qkv(TAG_Q, dk)
    k = qkv(TAG_K, dk)
    v = qkv(TAG_V, dv)
    lg = _sigmoid_log(stream(seed, TAG_GATE, 1000 + step).normal(4.0, 1.0, size=(N, H)))
    beta = _sigmoid(stream(seed, TAG_BETA, 1000 + step).normal(0.0, 1.0, size=(N, H))) if with_beta else None
    return DecodeStep(q=q, k=k, v=v, log_gate=lg, beta=beta)


def to_f64(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


# ----------------------------------------------------------------------------
# Short causal depthwise convolution
# ----------------------------------------------------------------------------
@dataclass
class ConvInputs:
    """Inputs of one short-convolution call over q, k and v.

    x[i], window[i]: storage dtype (uint16 bf16 bits or float32); taps: float32.
    i = 0, 1, 2 for q, k, v."""
    dtype: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    K: int
    x: list
    taps: list
    window: list

    def f64(self, what: str, i: int) -> Optional[np.ndarray]:
        arr = getattr(self, what)[i]
        return None if arr is None else to_f64(arr)


def make_conv_inputs(dtype: str, B: int, H: int, L: int, dk: int, dv: int, K: int = 4,
                     seed: int = 0, with_window: bool = False,
                     threads: Optional[int] = None) -> ConvInputs:
    """q, k, v ~ N(0, 1) (the projections' outputs before the convolution); taps
    U(-1/sqrt(K), 1/sqrt(K)) per channel, the usual initialisation of a depthwise
    1-D convolution (fan-in K); windows N(0, 1) when requested."""
    sdt = np.uint16 if dtype == "bf16" else np.float32
    ds = (dk, dk, dv)
    xs = [np.empty((B * H, L, d), sdt) for d in ds]

    def fill(j: int) -> None:
        i, bh = divmod(j, B * H)
        b, h = divmod(bh, H)
        xs[i][bh] = _store(stream(seed, (TAG_Q, TAG_K, TAG_V)[i], b, h).standard_normal(
            (L, ds[i]), dtype=np.float32), dtype)

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill, range(3 * B * H)))
    bound = 1.0 / math.sqrt(K)
    taps = [stream(seed, TAG_CONV_W, i).uniform(-bound, bound, size=(H, ds[i], K)).astype(np.float32)
            for i in range(3)]
    win = [None, None, None]
    if with_window:
        for i in range(3):
            w = np.empty((B * H, K - 1, ds[i]), sdt)
            for bh in range(B * H):
                b, h = divmod(bh, H)
                w[bh] = _store(stream(seed, TAG_CONV_WINDOW, i, b, h).standard_normal(
                    (K - 1, ds[i]), dtype=np.float32), dtype)
            win[i] = w.reshape(B, H, K - 1, ds[i])
    return ConvInputs(dtype=dtype, B=B, H=H, L=L, dk=dk, dv=dv, K=K,
                      x=[x.reshape(B, H, L, d) for x, d in zip(xs, ds)], taps=taps, window=win)


def config_conv_inputs(name: str, seed: int = 0) -> ConvInputs:
    c = CONFIGS[name]
    assert c["kind"] == "conv", name
    return make_conv_inputs(c["dtype"], c["B"], c["H"], c["L"], c["dk"], c["dv"], c["K"], seed=seed)


# ----------------------------------------------------------------------------
# Backward pass
# ----------------------------------------------------------------------------
def make_backward_dout(dtype: str, B: int, H: int, L: int, dv: int, seed: int = 0,
                       threads: Optional[int] = None) -> np.ndarray:
    """Output gradient dO ~ N(0, 1) per (b, h) slice (stream [seed, 9, b, h]), in the
    storage dtype."""
    sdt = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((B * H, L, dv), sdt)

    def fill(i: int) -> None:
        b, h = divmod(i, H)
        out[i] = _store(stream(seed, TAG_DOUT, b, h).standard_normal((L, dv), dtype=np.float32), dtype)

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill, range(B * H)))
    return out.reshape(B, H, L, dv)
