"""Pins of the fp64 oracle against facts other than itself.

Each pin takes the loaded oracle library and raises AssertionError when the oracle
disagrees with a closed form, an invariant, a special case that reduces to a
textbook formula, or an exact rational brute force. None of them re-types the
oracle's recurrence: the references here are the parallel (quadratic) forms, the
explicit product expansion, the retrieve/merge/overwrite form and a chunkwise WY
form, each written from the passage it cites.

Used twice: tests/test_oracle_pins.py runs every pin on the real oracle, and
tests/test_oracle_mutants.py runs them on deliberately broken copies of the
oracle to show that each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = math.sqrt(float(np.mean(b * b))) or 1.0
    return float(np.max(np.abs(a - b))) / scale


def _mask(L):
    # inclusive causal mask j <= t (tensorplay section 2.1, sum over j = 1..t)
    return np.tril(np.ones((L, L)))


# ---------------------------------------------------------------------------
# PLAIN
# ---------------------------------------------------------------------------
def pin_plain_quadratic(lib):
    """O = (Q K^T (.) M) V  (tensorplay section 2.1, parallel form)."""
    r = _rng(1)
    q, k = r.standard_normal((3, 37, 5)), r.standard_normal((3, 37, 5))
    v = r.standard_normal((3, 37, 4))
    o, _, _ = oracle.forward("plain", q, k, v, lib=lib)
    ref = (q @ k.transpose(0, 2, 1) * _mask(37)) @ v
    assert _rel(o, ref) <= 1e-12, _rel(o, ref)


def pin_plain_fraction_bruteforce(lib):
    """o_t = sum_{j<=t} (q_t . k_j) v_j in exact integer arithmetic
    (tensorplay section 2.1, per-token sum form). Small integers make every fp64
    operation of the oracle exact, so agreement must be bit-exact."""
    r = _rng(2)
    L, dk, dv = 7, 3, 2
    q = r.integers(-3, 4, (L, dk))
    k = r.integers(-3, 4, (L, dk))
    v = r.integers(-3, 4, (L, dv))
    ref = np.zeros((L, dv), dtype=object)
    for t in range(L):
        for j in range(t + 1):
            w = sum(int(q[t, i]) * int(k[j, i]) for i in range(dk))
            for c in range(dv):
                ref[t, c] += w * int(v[j, c])
    o, _, _ = oracle.forward("plain", q.astype(float), k.astype(float), v.astype(float), lib=lib)
    assert np.array_equal(o, ref.astype(np.float64)), (o, ref)


def pin_plain_final_state(lib):
    """With S_0 given, S_L = S_0 + K^T V: the re-associated product of the
    non-causal form (proig-chaa notes section 3; tensorplay section 2.1)."""
    r = _rng(3)
    q, k = r.standard_normal((2, 19, 6)), r.standard_normal((2, 19, 6))
    v = r.standard_normal((2, 19, 3))
    s0 = r.standard_normal((2, 6, 3))
    o, s, _ = oracle.forward("plain", q, k, v, state_in=s0, lib=lib)
    assert _rel(s, s0 + k.transpose(0, 2, 1) @ v) <= 1e-12
    # outputs with a carried-in state: Q S_0 + (Q K^T (.) M) V
    ref = q @ s0 + (q @ k.transpose(0, 2, 1) * _mask(19)) @ v
    assert _rel(o, ref) <= 1e-12


# ---------------------------------------------------------------------------
# NORMALIZED
# ---------------------------------------------------------------------------
def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def pin_normalized_quadratic(lib):
    """y_i = sum_{j<=i} (phi_i . phi_j) v_j / sum_{j<=i} phi_i . phi_j, with an
    optional carried-in (S_0, z_0) adding phi_i^T S_0 and phi_i . z_0
    (proig-chaa notes sections 13-14)."""
    r = _rng(4)
    q, k = _phi(r.standard_normal((2, 29, 5))), _phi(r.standard_normal((2, 29, 5)))
    v = r.standard_normal((2, 29, 3))
    A = q @ k.transpose(0, 2, 1) * _mask(29)
    o, s, z = oracle.forward("normalized", q, k, v, lib=lib)
    ref = (A @ v) / A.sum(-1, keepdims=True)
    assert _rel(o, ref) <= 1e-12, _rel(o, ref)
    assert _rel(z, k.sum(1)) <= 1e-13
    s0 = r.standard_normal((2, 5, 3))
    z0 = 1.0 + r.random((2, 5))
    o2, s2, z2 = oracle.forward("normalized", q, k, v, state_in=s0, z_in=z0, lib=lib)
    num = q @ s0 + A @ v
    den = (q * z0[:, None, :]).sum(-1, keepdims=True) + A.sum(-1, keepdims=True)
    assert _rel(o2, num / den) <= 1e-12
    assert _rel(z2, z0 + k.sum(1)) <= 1e-13
    assert _rel(s2, s0 + k.transpose(0, 2, 1) @ v) <= 1e-12


def pin_normalized_constant_v(lib):
    """The normalised output is a weighted average of v_1..v_i (weights sum to
    one), so v == c gives o == c (proig-chaa notes section 13)."""
    r = _rng(5)
    q, k = _phi(r.standard_normal((1, 40, 4))), _phi(r.standard_normal((1, 40, 4)))
    v = np.broadcast_to(np.array([2.5, -1.0, 0.125]), (1, 40, 3)).copy()
    o, _, _ = oracle.forward("normalized", q, k, v, lib=lib)
    assert np.max(np.abs(o - v)) <= 1e-13


def pin_normalized_hull(lib):
    """Positive weights summing to one: each o_i lies within the per-column range
    of v_1..v_i."""
    r = _rng(6)
    q, k = _phi(r.standard_normal((1, 50, 4))), _phi(r.standard_normal((1, 50, 4)))
    v = r.standard_normal((1, 50, 3))
    o, _, _ = oracle.forward("normalized", q, k, v, lib=lib)
    lo = np.minimum.accumulate(v[0], axis=0)
    hi = np.maximum.accumulate(v[0], axis=0)
    assert np.all(o[0] >= lo - 1e-12) and np.all(o[0] <= hi + 1e-12)


# ---------------------------------------------------------------------------
# DECAY
# ---------------------------------------------------------------------------
def pin_decay_quadratic(lib):
    """Cumulative decay b_t = prod_{j<=t} gamma_j turns the recurrence into
    O = ((Q K^T) (.) D) V with D_ij = b_i / b_j for j <= i (tensorplay section 5.2),
    evaluated here with the global log cumsum G; a carried-in S_0 adds
    diag(b) Q S_0 and the final state is b_L S_0 + sum_j (b_L/b_j) k_j v_j^T."""
    r = _rng(7)
    L = 33
    q, k = r.standard_normal((2, L, 5)), r.standard_normal((2, L, 5))
    v = r.standard_normal((2, L, 4))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(2.0, 1.0, (2, L)))))
    s0 = r.standard_normal((2, 5, 4))
    G = np.cumsum(lg, axis=1)
    D = np.exp(G[:, :, None] - G[:, None, :]) * _mask(L)
    ref = np.exp(G)[:, :, None] * (q @ s0) + (q @ k.transpose(0, 2, 1) * D) @ v
    o, s, _ = oracle.forward("decay", q, k, v, log_gate=lg, state_in=s0, lib=lib)
    assert _rel(o, ref) <= 1e-12, _rel(o, ref)
    sref = np.exp(G[:, -1])[:, None, None] * s0 + \
        (k * np.exp(G[:, -1:] - G)[:, :, None]).transpose(0, 2, 1) @ v
    assert _rel(s, sref) <= 1e-12


def pin_decay_zero_gate_is_plain(lib):
    """gamma == 1 (log-gate 0) reduces the decayed recurrence to the plain one."""
    r = _rng(8)
    q, k, v = (r.standard_normal((2, 21, 4)) for _ in range(3))
    o1, s1, _ = oracle.forward("decay", q, k, v, log_gate=np.zeros((2, 21)), lib=lib)
    o2, s2, _ = oracle.forward("plain", q, k, v, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def pin_decay_fraction_half(lib):
    """Constant gamma = 1/2 with integer inputs: o_t = sum_{j<=t} 2^{-(t-j)}
    (q_t . k_j) v_j in exact rationals (wln20, data-independent decay with a
    constant 0 < gamma < 1). The oracle forms gamma = exp(log 1/2), which may be
    one ulp off, hence a 1e-13 relative bound instead of equality."""
    r = _rng(9)
    L, dk, dv = 8, 3, 2
    q = r.integers(-3, 4, (L, dk))
    k = r.integers(-3, 4, (L, dk))
    v = r.integers(-3, 4, (L, dv))
    ref = np.zeros((L, dv), dtype=object)
    for t in range(L):
        for j in range(t + 1):
            w = Fraction(sum(int(q[t, i]) * int(k[j, i]) for i in range(dk)), 2 ** (t - j))
            for c in range(dv):
                ref[t, c] += w * int(v[j, c])
    o, _, _ = oracle.forward("decay", q.astype(float), k.astype(float), v.astype(float),
                             log_gate=np.full(L, math.log(0.5)), lib=lib)
    assert _rel(o, ref.astype(np.float64)) <= 1e-13


# ---------------------------------------------------------------------------
# GATED DELTA
# ---------------------------------------------------------------------------
def _gdn_retrieve_merge_overwrite(q, k, v, alpha, beta, s0=None):
    """DeltaNet written as retrieve / merge / overwrite on the decayed state, in the
    pages' v k^T orientation (S' is d_v x d_k): S~ = alpha S'; v_old = S~ k;
    v_new = beta v + (1 - beta) v_old; S' = S~ - v_old k^T + v_new k^T; o = S' q
    (tensorplay section 6.1; wln20 DeltaNet and Gated DeltaNet sections)."""
    L, dk = q.shape
    dv = v.shape[1]
    Sp = np.zeros((dv, dk)) if s0 is None else s0.T.copy()
    o = np.zeros((L, dv))
    for t in range(L):
        St = alpha[t] * Sp
        v_old = St @ k[t]
        v_new = beta[t] * v[t] + (1.0 - beta[t]) * v_old
        Sp = St - np.outer(v_old, k[t]) + np.outer(v_new, k[t])
        o[t] = Sp @ q[t]
    return o, Sp.T


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def pin_gdn_retrieve_merge_overwrite(lib):
    r = _rng(10)
    L, dk, dv = 31, 6, 5
    q, k = _unit(r.standard_normal((L, dk))), _unit(r.standard_normal((L, dk)))
    v = r.standard_normal((L, dv))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, L))))
    beta = 1.0 / (1.0 + np.exp(-r.normal(0.0, 1.0, L)))
    s0 = r.standard_normal((dk, dv))
    ref_o, ref_s = _gdn_retrieve_merge_overwrite(q, k, v, np.exp(lg), beta, s0)
    o, s, _ = oracle.forward("gated_delta", q[None], k[None], v[None], log_gate=lg[None],
                             beta=beta[None], state_in=s0[None], lib=lib)
    assert _rel(o[0], ref_o) <= 1e-12, _rel(o[0], ref_o)
    assert _rel(s[0], ref_s) <= 1e-12


def pin_gdn_alpha_one_is_deltanet(lib):
    """alpha == 1 gives DeltaNet (tensorplay section 6.2); an absent log-gate means
    alpha == 1."""
    r = _rng(11)
    L, dk, dv = 17, 4, 3
    q, k = _unit(r.standard_normal((1, L, dk))), _unit(r.standard_normal((1, L, dk)))
    v = r.standard_normal((1, L, dv))
    beta = r.random((1, L))
    o1, s1, _ = oracle.forward("gated_delta", q, k, v, log_gate=None, beta=beta, lib=lib)
    o2, s2, _ = oracle.forward("gated_delta", q, k, v, log_gate=np.zeros((1, L)), beta=beta, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    ref_o, _ = _gdn_retrieve_merge_overwrite(q[0], k[0], v[0], np.ones(L), beta[0])
    assert _rel(o1[0], ref_o) <= 1e-12


def pin_gdn_beta_zero_pure_decay(lib):
    """beta == 0: nothing is written, S_t = (prod alpha) S_0 and o_t = S_t^T q_t."""
    r = _rng(12)
    L, dk, dv = 15, 4, 3
    q, k = r.standard_normal((1, L, dk)), _unit(r.standard_normal((1, L, dk)))
    v = r.standard_normal((1, L, dv))
    lg = -r.random((1, L)) * 0.3
    s0 = r.standard_normal((1, dk, dv))
    o, s, _ = oracle.forward("gated_delta", q, k, v, log_gate=lg, beta=np.zeros((1, L)),
                             state_in=s0, lib=lib)
    a = np.exp(np.cumsum(lg[0]))
    assert _rel(o[0], a[:, None] * (q[0] @ s0[0])) <= 1e-12
    assert _rel(s[0], a[-1] * s0[0]) <= 1e-12


RECALL_FIXTURES = ("recall_a4b3c6.txt", "recall_rebind.txt")


def _read_golden_recall(name):
    """A tests/golden/recall_*.txt fixture: keys, values, queries, expected outputs."""
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            rows[key.strip()] = val.split()
    return rows


def pin_gdn_onehot_recall(lib):
    """Associative recall with orthonormal (one-hot) keys, beta = 1, alpha = 1:
    the delta rule returns exactly the last value bound to the queried key, while
    plain linear attention returns the sum of every value bound to it
    (tensorplay section 6: A4B3C6 -> A?C? -> 4,6; proig-chaa sections 18-19 on
    interference). Values from tests/golden/recall_*.txt."""
    for name in RECALL_FIXTURES:
        _check_recall(lib, _read_golden_recall(name))


def _check_recall(lib, g):
    alphabet = g["alphabet"]
    d = len(alphabet)
    writes = [(w[0], float(w[1:])) for w in g["writes"]]
    queries = g["queries"]
    toks = len(writes) + len(queries)
    q = np.zeros((1, toks, d)); k = np.zeros((1, toks, d)); v = np.zeros((1, toks, 1))
    for t, (key, val) in enumerate(writes):
        k[0, t, alphabet.index(key)] = 1.0
        v[0, t, 0] = val
    for i, key in enumerate(queries):
        q[0, len(writes) + i, alphabet.index(key)] = 1.0
    beta = np.ones((1, toks))
    o, _, _ = oracle.forward("gated_delta", q, k, v, beta=beta, lib=lib)
    got = o[0, len(writes):, 0]
    assert np.array_equal(got, np.array([float(x) for x in g["delta_expect"]])), got
    o2, _, _ = oracle.forward("plain", q, k, v, lib=lib)
    got2 = o2[0, len(writes):, 0]
    assert np.array_equal(got2, np.array([float(x) for x in g["plain_expect"]])), got2


def pin_gdn_unit_key_identity(lib):
    """With |k_t| = 1 the reparameterised rule gives S_t^T k_t =
    alpha_t (1 - beta_t) S_{t-1}^T k_t + beta_t v_t at every step (from
    S'_t = alpha S'_{t-1}(I - beta k k^T) + beta v k^T, tensorplay section 6.2:
    the written value is the beta-merge of old and new)."""
    r = _rng(13)
    L, dk, dv = 12, 5, 4
    q, k = r.standard_normal((L, dk)), _unit(r.standard_normal((L, dk)))
    v = r.standard_normal((L, dv))
    lg = -r.random(L) * 0.2
    beta = r.random(L)
    S = r.standard_normal((dk, dv))
    for t in range(L):
        _, S1, _ = oracle.forward("gated_delta", q[None, t:t + 1], k[None, t:t + 1],
                                  v[None, t:t + 1], log_gate=lg[None, t:t + 1],
                                  beta=beta[None, t:t + 1], state_in=S[None], lib=lib)
        lhs = S1[0].T @ k[t]
        rhs = math.exp(lg[t]) * (1 - beta[t]) * (S.T @ k[t]) + beta[t] * v[t]
        assert np.max(np.abs(lhs - rhs)) <= 1e-12
        S = S1[0]


def pin_gdn_fraction_product_expansion(lib):
    """Exact rationals: S_t = sum_{j<=t} [A_t ... A_{j+1}] beta_j k_j v_j^T with
    A_s = alpha_s (I - beta_s k_s k_s^T), o_t = S_t^T q_t: the unrolled
    identity-plus-low-rank products (tensorplay sections 6.2 and 7.1, canonical
    d_k x d_v orientation). The oracle receives alpha as log(alpha) and forms
    exp in fp64, hence a 1e-12 relative bound."""
    r = _rng(14)
    L, dk, dv = 6, 3, 2
    Fr = Fraction
    q = [[Fr(int(x)) for x in row] for row in r.integers(-2, 3, (L, dk))]
    k = [[Fr(int(x)) for x in row] for row in r.integers(-1, 2, (L, dk))]
    v = [[Fr(int(x)) for x in row] for row in r.integers(-3, 4, (L, dv))]
    alpha = [Fr(int(a), 8) for a in r.integers(5, 9, L)]
    beta = [Fr(int(b), 4) for b in r.integers(0, 5, L)]

    def eye(n):
        return [[Fr(int(i == j)) for j in range(n)] for i in range(n)]

    def matmul(A, B):
        return [[sum((A[i][m] * B[m][j] for m in range(len(B))), Fr(0)) for j in range(len(B[0]))]
                for i in range(len(A))]

    def transition(s):
        return [[alpha[s] * ((1 if i == j else 0) - beta[s] * k[s][i] * k[s][j]) for j in range(dk)]
                for i in range(dk)]

    o_ref = []
    for t in range(L):
        S = [[Fr(0)] * dv for _ in range(dk)]
        for j in range(t + 1):
            P = eye(dk)
            for s in range(t, j, -1):
                P = matmul(P, transition(s))
            w = [[beta[j] * k[j][i] * v[j][c] for c in range(dv)] for i in range(dk)]
            PW = matmul(P, w)
            S = [[S[i][c] + PW[i][c] for c in range(dv)] for i in range(dk)]
        o_ref.append([sum((S[i][c] * q[t][i] for i in range(dk)), Fr(0)) for c in range(dv)])
    f = lambda M: np.array([[float(x) for x in row] for row in M])
    o, _, _ = oracle.forward("gated_delta", f(q)[None], f(k)[None], f(v)[None],
                             log_gate=np.log(np.array([float(a) for a in alpha]))[None],
                             beta=np.array([float(b) for b in beta])[None], lib=lib)
    assert _rel(o[0], f(o_ref)) <= 1e-12, _rel(o[0], f(o_ref))


def gdn_chunkwise_wy(q, k, v, lg, beta, C, s0=None):
    """Chunkwise WY/UT form of Gated DeltaNet (the tensorplay section 6.2 statement
    that Householder-style products become chunk-parallel accumulations, worked out
    for the canonical orientation). Per chunk, with G_r the within-chunk log-gate
    cumsum, a_r = exp(G_r) and Gamma_rs = exp(G_r - G_s):
      P = strict_lower(diag(beta) (Gamma (.) K K^T)),  T = (I + P)^-1
      W = T diag(beta a) K,   U~ = T diag(beta) V,   U = U~ - W S_0
      O = diag(a) Q S_0 + (Gamma (.) Q K^T (.) M) U
      S_C = a_C S_0 + (diag(a_C / a) K)^T U
    With lg == 0 this is DeltaNet; with T = I and U = V it is the decay form."""
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else s0.copy()
    o = np.zeros((L, dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = Q.shape[0]
        G = np.cumsum(lg[sl])
        a = np.exp(G)
        Gam = np.exp(G[:, None] - G[None, :])
        P = np.tril(b[:, None] * Gam * (K @ K.T), -1)
        T = np.linalg.inv(np.eye(n) + P)
        W = T @ ((b * a)[:, None] * K)
        U = T @ (b[:, None] * V) - W @ S
        o[sl] = a[:, None] * (Q @ S) + (np.tril(Gam * (Q @ K.T))) @ U
        S = a[-1] * S + ((a[-1] / a)[:, None] * K).T @ U
    return o, S


def pin_gdn_chunkwise_wy(lib):
    """The chunk algebra the GPU path uses equals the recurrence for C in
    {1, 4, 16, L} (tensorplay section 3.3: C = 1 is the recurrent form, C = L the
    parallel one)."""
    r = _rng(15)
    L, dk, dv = 48, 8, 6
    q, k = _unit(r.standard_normal((L, dk))), _unit(r.standard_normal((L, dk)))
    v = r.standard_normal((L, dv))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, L))))
    beta = 1.0 / (1.0 + np.exp(-r.normal(0.0, 1.0, L)))
    s0 = r.standard_normal((dk, dv)) * 0.3
    o, s, _ = oracle.forward("gated_delta", q[None], k[None], v[None], log_gate=lg[None],
                             beta=beta[None], state_in=s0[None], lib=lib)
    for C in (1, 4, 16, L):
        oc, sc = gdn_chunkwise_wy(q, k, v, lg, beta, C, s0)
        assert _rel(o[0], oc) <= 1e-10, (C, _rel(o[0], oc))
        assert _rel(s[0], sc) <= 1e-10, C


# ---------------------------------------------------------------------------
# KDA: the delta rule with a per-key-channel gate
# ---------------------------------------------------------------------------
def kda_chunkwise_wy(q, k, v, lg, beta, C, s0=None):
    """Chunk form of Kimi Delta Attention, S_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
    S_{t-1} + beta_t k_t v_t^T (wln20, Kimi Delta Attention section), worked out
    like the scalar-gate WY form: with the per-channel gate the update is
    S_t = Diag(alpha_t) S_{t-1} + k_t u_t^T, u_t = beta_t (v_t - S_{t-1}^T (alpha_t (.) k_t)).
    Within a chunk, with G_r the per-channel log-gate cumsum and Gam_r = exp(G_r),
    S_{t-1}^T (alpha_t (.) k_t) = S_0^T (Gam_t (.) k_t) + sum_{s<t} u_s (Gam_t (.) k_t).(k_s / Gam_s),
    so (I + diag(beta) A) U = diag(beta) (V - (K (.) Gam) S_0), A = strict_lower((K (.) Gam)(K / Gam)^T):
      T = (I + diag(beta) A)^-1,  W = T diag(beta) (K (.) Gam),  U~ = T diag(beta) V,  U = U~ - W S_0
      O = (Q (.) Gam) S_0 + tril((Q (.) Gam)(K / Gam)^T) U
      S_C = Diag(Gam_C) S_0 + (K (.) Gam_C / Gam)^T U"""
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else s0.copy()
    o = np.zeros((L, dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = Q.shape[0]
        Gam = np.exp(np.cumsum(lg[sl], axis=0))
        A = np.tril((K * Gam) @ (K / Gam).T, -1)
        T = np.linalg.inv(np.eye(n) + b[:, None] * A)
        W = T @ (b[:, None] * (K * Gam))
        U = T @ (b[:, None] * V) - W @ S
        o[sl] = (Q * Gam) @ S + np.tril((Q * Gam) @ (K / Gam).T) @ U
        S = Gam[-1][:, None] * S + (K * (Gam[-1] / Gam)).T @ U
    return o, S


def _kda_inputs(seed, L, dk, dv, gate_scale=1.0):
    r = _rng(seed)
    q, k = _unit(r.standard_normal((L, dk))), _unit(r.standard_normal((L, dk)))
    v = r.standard_normal((L, dv))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, (L, dk))))) * gate_scale
    beta = 1.0 / (1.0 + np.exp(-r.normal(0.0, 1.0, L)))
    s0 = r.standard_normal((dk, dv)) * 0.3
    return q, k, v, lg, beta, s0


def pin_kda_chunkwise_wy(lib):
    """The chunk algebra above equals the oracle's recurrence for C in {1, 4, 16, L}
    (tensorplay section 3.3: C = 1 is the recurrent form, C = L the parallel one)."""
    L, dk, dv = 48, 8, 6
    q, k, v, lg, beta, s0 = _kda_inputs(30, L, dk, dv)
    o, s, _ = oracle.forward("kda", q[None], k[None], v[None], log_gate=lg[None], beta=beta[None],
                             state_in=s0[None], lib=lib)
    for C in (1, 4, 16, L):
        oc, sc = kda_chunkwise_wy(q, k, v, lg, beta, C, s0)
        assert _rel(o[0], oc) <= 1e-10, (C, _rel(o[0], oc))
        assert _rel(s[0], sc) <= 1e-10, C


def pin_kda_uniform_gate_is_gdn(lib):
    """The same gate on every key channel is the scalar-gate delta rule: Diag(alpha)
    = alpha I commutes with (I - beta k k^T)."""
    L, dk, dv = 23, 6, 5
    q, k, v, lg, beta, s0 = _kda_inputs(31, L, dk, dv)
    g1 = lg[:, 0]
    o1, s1, _ = oracle.forward("kda", q[None], k[None], v[None], log_gate=np.repeat(g1[:, None], dk, 1)[None],
                               beta=beta[None], state_in=s0[None], lib=lib)
    o2, s2, _ = oracle.forward("gated_delta", q[None], k[None], v[None], log_gate=g1[None], beta=beta[None],
                               state_in=s0[None], lib=lib)
    assert _rel(o1, o2) <= 1e-12 and _rel(s1, s2) <= 1e-12


def pin_kda_beta_zero_pure_decay(lib):
    """beta == 0: nothing is written, S_t = Diag(prod alpha) S_0 channel by channel."""
    L, dk, dv = 15, 4, 3
    q, k, v, lg, _, s0 = _kda_inputs(32, L, dk, dv)
    o, s, _ = oracle.forward("kda", q[None], k[None], v[None], log_gate=lg[None], beta=np.zeros((1, L)),
                             state_in=s0[None], lib=lib)
    Gam = np.exp(np.cumsum(lg, axis=0))
    assert _rel(o[0], (q * Gam) @ s0) <= 1e-12
    assert _rel(s[0], Gam[-1][:, None] * s0) <= 1e-12


def pin_kda_unit_key_overwrite(lib):
    """beta = 1 with a unit key overwrites what the key retrieves, whatever the
    gate: S_t^T k_t = (Diag(alpha) S)^T (I - k k^T) k + v (k . k) = v_t."""
    L, dk, dv = 9, 5, 4
    q, k, v, lg, _, s0 = _kda_inputs(33, L, dk, dv, gate_scale=4.0)
    for t in range(1, L + 1):
        _, s, _ = oracle.forward("kda", q[None, :t], k[None, :t], v[None, :t], log_gate=lg[None, :t],
                                 beta=np.ones((1, t)), state_in=s0[None], lib=lib)
        assert np.max(np.abs(s[0].T @ k[t - 1] - v[t - 1])) <= 1e-12


def pin_kda_decode_and_resume(lib):
    """The decode step continues a prefill exactly, and a split sequence carried
    through the state equals one pass."""
    L, dk, dv = 20, 6, 5
    q, k, v, lg, beta, s0 = _kda_inputs(34, L, dk, dv)
    o, s, _ = oracle.forward("kda", q[None], k[None], v[None], log_gate=lg[None], beta=beta[None],
                             state_in=s0[None], lib=lib)
    t = 13
    op, sp, _ = oracle.forward("kda", q[None, :t], k[None, :t], v[None, :t], log_gate=lg[None, :t],
                               beta=beta[None, :t], state_in=s0[None], lib=lib)
    od, sd = oracle.decode_step("kda", q[None, t], k[None, t], v[None, t], lg[None, t], sp, beta=beta[None, t],
                                lib=lib)
    oc, _ = kda_chunkwise_wy(q[: t + 1], k[: t + 1], v[: t + 1], lg[: t + 1], beta[: t + 1], 4, s0)
    assert _rel(od[0], oc[t]) <= 1e-10
    ob, sb, _ = oracle.forward("kda", q[None, t:], k[None, t:], v[None, t:], log_gate=lg[None, t:],
                               beta=beta[None, t:], state_in=sp, lib=lib)
    assert _rel(np.concatenate([op[0], ob[0]]), o[0]) <= 1e-12 and _rel(sb, s) <= 1e-12


# ---------------------------------------------------------------------------
# DECODE and state carry
# ---------------------------------------------------------------------------
def pin_decode_one_decay_step(lib):
    """Decode step = S' = gamma S + k v^T, o = S'^T q, written out in numpy
    (wln20 data-dependent decay; tensorplay section 2.1 output read-out)."""
    r = _rng(16)
    NH, dk, dv = 6, 5, 4
    q, k = r.standard_normal((NH, dk)), r.standard_normal((NH, dk))
    v = r.standard_normal((NH, dv))
    lg = -r.random(NH)
    S = r.standard_normal((NH, dk, dv))
    o, S1 = oracle.decode_step("decay", q, k, v, lg, S, lib=lib)
    S_ref = np.exp(lg)[:, None, None] * S + k[:, :, None] * v[:, None, :]
    assert _rel(S1, S_ref) <= 1e-14
    assert _rel(o, np.einsum("nij,ni->nj", S_ref, q)) <= 1e-13


def pin_prefill_then_decode(lib):
    """The state is the whole memory (tensorplay section 2.2): prefill L tokens,
    then one decode step on token L+1, equals the forward over L+1 tokens."""
    r = _rng(17)
    L, dk, dv = 20, 4, 3
    q, k = r.standard_normal((2, L + 1, dk)), r.standard_normal((2, L + 1, dk))
    v = r.standard_normal((2, L + 1, dv))
    lg = -r.random((2, L + 1)) * 0.1
    o_full, s_full, _ = oracle.forward("decay", q, k, v, log_gate=lg, lib=lib)
    _, s_pre, _ = oracle.forward("decay", q[:, :L], k[:, :L], v[:, :L], log_gate=lg[:, :L], lib=lib)
    o_dec, s_dec = oracle.decode_step("decay", q[:, L], k[:, L], v[:, L], lg[:, L], s_pre, lib=lib)
    assert _rel(o_dec, o_full[:, L]) <= 1e-13 and _rel(s_dec, s_full) <= 1e-13


def pin_decode_gdn_step(lib):
    """Delta-rule decode step against the retrieve / merge / overwrite form of one
    token on the decayed state, written in the pages' v k^T orientation
    (tensorplay section 6.1; wln20 DeltaNet and Gated DeltaNet sections); also
    alpha = 1 when no log-gate is given."""
    r = _rng(21)
    NH, dk, dv = 5, 6, 4
    q, k = _unit(r.standard_normal((NH, dk))), _unit(r.standard_normal((NH, dk)))
    v = r.standard_normal((NH, dv))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, NH))))
    beta = 1.0 / (1.0 + np.exp(-r.normal(0.0, 1.0, NH)))
    S = r.standard_normal((NH, dk, dv))
    for gate in (lg, None):
        o, S1 = oracle.decode_step("gated_delta", q, k, v, gate, S, beta=beta, lib=lib)
        alpha = np.ones(NH) if gate is None else np.exp(gate)
        for h in range(NH):
            ro, rs = _gdn_retrieve_merge_overwrite(q[h:h + 1], k[h:h + 1], v[h:h + 1], alpha[h:h + 1],
                                                   beta[h:h + 1], S[h])
            assert _rel(o[h], ro[0]) <= 1e-13 and _rel(S1[h], rs) <= 1e-13


def pin_prefill_then_decode_gdn(lib):
    """Prefill L tokens with the delta rule, then one decode step on token L+1,
    equals the forward over L+1 tokens (the state is the whole memory)."""
    r = _rng(22)
    L, dk, dv = 17, 5, 3
    q, k = _unit(r.standard_normal((2, L + 1, dk))), _unit(r.standard_normal((2, L + 1, dk)))
    v = r.standard_normal((2, L + 1, dv))
    lg = np.log(1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, (2, L + 1)))))
    beta = 1.0 / (1.0 + np.exp(-r.normal(0.0, 1.0, (2, L + 1))))
    o_full, s_full, _ = oracle.forward("gated_delta", q, k, v, log_gate=lg, beta=beta, lib=lib)
    _, s_pre, _ = oracle.forward("gated_delta", q[:, :L], k[:, :L], v[:, :L], log_gate=lg[:, :L],
                                 beta=beta[:, :L], lib=lib)
    o_dec, s_dec = oracle.decode_step("gated_delta", q[:, L], k[:, L], v[:, L], lg[:, L], s_pre,
                                      beta=beta[:, L], lib=lib)
    assert _rel(o_dec, o_full[:, L]) <= 1e-12 and _rel(s_dec, s_full) <= 1e-12


def pin_resume_all_variants(lib):
    """Splitting a sequence and carrying (S, z) across the split gives the same
    result as one pass, for every variant."""
    r = _rng(18)
    L1, L2, dk, dv = 13, 11, 4, 3
    L = L1 + L2
    q = _phi(r.standard_normal((2, L, dk)))
    k = _unit(_phi(r.standard_normal((2, L, dk))))
    v = r.standard_normal((2, L, dv))
    lg = -r.random((2, L)) * 0.2
    beta = r.random((2, L))
    for var in ("plain", "normalized", "decay", "gated_delta"):
        kw = {}
        if var in ("decay", "gated_delta"):
            kw["log_gate"] = lg
        if var == "gated_delta":
            kw["beta"] = beta
        o, s, z = oracle.forward(var, q, k, v, lib=lib, **kw)
        k1 = {n: x[:, :L1] for n, x in kw.items()}
        k2 = {n: x[:, L1:] for n, x in kw.items()}
        oa, sa, za = oracle.forward(var, q[:, :L1], k[:, :L1], v[:, :L1], lib=lib, **k1)
        ob, sb, zb = oracle.forward(var, q[:, L1:], k[:, L1:], v[:, L1:], state_in=sa,
                                    z_in=za, lib=lib, **k2)
        assert _rel(np.concatenate([oa, ob], 1), o) <= 1e-12, var
        assert _rel(sb, s) <= 1e-12, var
        if var == "normalized":
            assert _rel(zb, z) <= 1e-13


# ---------------------------------------------------------------------------
# VECTOR_DECAY (one log-gate per key channel)
# ---------------------------------------------------------------------------
def pin_vector_decay_parallel_form(lib):
    """O = ((Q (.) B)(K / B)^T (.) M) V with B the per-channel cumulative product of
    the gates (tensorplay section 5.2, GLA parallel form), and the final state
    S_L = sum_s Diag(B_L / B_s) k_s v_s^T. Moderate gates keep K / B finite."""
    r = _rng(40)
    L, dk, dv = 37, 6, 5
    q, k = r.standard_normal((2, L, dk)), r.standard_normal((2, L, dk))
    v = r.standard_normal((2, L, dv))
    lg = -0.3 * r.random((2, L, dk))
    o, s, _ = oracle.forward("vector_decay", q, k, v, log_gate=lg, lib=lib)
    Bm = np.exp(np.cumsum(lg, axis=1))
    ref = ((q * Bm) @ (k / Bm).transpose(0, 2, 1) * _mask(L)) @ v
    assert _rel(o, ref) <= 1e-10, _rel(o, ref)
    sref = np.einsum("bsc,bsj->bcj", k * (Bm[:, -1:, :] / Bm), v)
    assert _rel(s, sref) <= 1e-12, _rel(s, sref)


def pin_vector_decay_uniform_is_scalar(lib):
    """The same gate on every key channel is the scalar decay, bit for bit; zero
    gates are the plain recurrence."""
    r = _rng(41)
    L, dk, dv = 23, 5, 4
    q, k, v = r.standard_normal((3, L, dk)), r.standard_normal((3, L, dk)), r.standard_normal((3, L, dv))
    lg1 = -r.random((3, L)) * 0.5
    s0 = r.standard_normal((3, dk, dv))
    ov, sv, _ = oracle.forward("vector_decay", q, k, v, log_gate=np.repeat(lg1[..., None], dk, -1),
                               state_in=s0, lib=lib)
    od, sd, _ = oracle.forward("decay", q, k, v, log_gate=lg1, state_in=s0, lib=lib)
    assert np.array_equal(ov, od) and np.array_equal(sv, sd)
    o0, _, _ = oracle.forward("vector_decay", q, k, v, log_gate=np.zeros((3, L, dk)), lib=lib)
    op, _, _ = oracle.forward("plain", q, k, v, lib=lib)
    assert np.array_equal(o0, op)


def pin_vector_decay_fraction(lib):
    """Exact rational brute force of o_t = sum_{s<=t} sum_c q_t[c] gamma_c^{t-s}
    k_s[c] v_s with constant per-channel gates gamma_c in {1, 1/2, 1/4}
    (the oracle forms gamma as exp(log gamma), so agreement is to rounding)."""
    r = _rng(42)
    L, dk, dv = 7, 3, 2
    q = r.integers(-3, 4, (1, L, dk)).astype(np.float64)
    k = r.integers(-3, 4, (1, L, dk)).astype(np.float64)
    v = r.integers(-3, 4, (1, L, dv)).astype(np.float64)
    gam = [Fraction(1), Fraction(1, 2), Fraction(1, 4)]
    lg = np.tile(np.array([math.log(float(g)) for g in gam]), (1, L, 1))
    o, _, _ = oracle.forward("vector_decay", q, k, v, log_gate=lg, lib=lib)
    for t in range(L):
        for j in range(dv):
            acc = Fraction(0)
            for s_ in range(t + 1):
                w = sum(Fraction(int(q[0, t, c])) * gam[c] ** (t - s_) * Fraction(int(k[0, s_, c]))
                        for c in range(dk))
                acc += w * Fraction(int(v[0, s_, j]))
            assert abs(o[0, t, j] - float(acc)) <= 1e-13 * max(1.0, abs(float(acc))), (t, j)


def pin_vector_decay_channel_isolation(lib):
    """A gate of exp(-200) on one key channel erases that channel's history at every
    step while the others keep theirs: o_t = sum_{s<=t} sum_{c != c0} q_t[c] k_s[c] v_s
    + q_t[c0] k_t[c0] v_t. This fails if the gate is applied along the value axis."""
    r = _rng(43)
    L, dk, dv, c0 = 11, 4, 6, 2
    q, k, v = r.standard_normal((1, L, dk)), r.standard_normal((1, L, dk)), r.standard_normal((1, L, dv))
    lg = np.zeros((1, L, dk))
    lg[:, :, c0] = -200.0
    o, s, _ = oracle.forward("vector_decay", q, k, v, log_gate=lg, lib=lib)
    keep = np.ones(dk)
    keep[c0] = 0.0
    ref = (((q * keep) @ k[0].T) * _mask(L)) @ v[0] + (q[0, :, c0] * k[0, :, c0])[:, None] * v[0]
    assert _rel(o, ref) <= 1e-12
    assert np.allclose(s[0, c0], k[0, -1, c0] * v[0, -1], rtol=1e-14, atol=0)


def pin_vector_decay_resume_and_decode(lib):
    """Splitting the sequence and carrying the state equals one pass, and one decode
    step on the carried state equals the next token of a longer pass."""
    r = _rng(44)
    L1, L2, dk, dv = 9, 8, 4, 3
    L = L1 + L2
    q, k, v = r.standard_normal((2, L, dk)), r.standard_normal((2, L, dk)), r.standard_normal((2, L, dv))
    lg = -r.random((2, L, dk)) * 0.4
    o, s, _ = oracle.forward("vector_decay", q, k, v, log_gate=lg, lib=lib)
    oa, sa, _ = oracle.forward("vector_decay", q[:, :L1], k[:, :L1], v[:, :L1], log_gate=lg[:, :L1], lib=lib)
    ob, sb, _ = oracle.forward("vector_decay", q[:, L1:], k[:, L1:], v[:, L1:], log_gate=lg[:, L1:],
                               state_in=sa, lib=lib)
    assert _rel(np.concatenate([oa, ob], 1), o) <= 1e-12 and _rel(sb, s) <= 1e-12
    t = L - 1
    o_prev, s_prev, _ = oracle.forward("vector_decay", q[:, :t], k[:, :t], v[:, :t], log_gate=lg[:, :t],
                                       lib=lib)
    od, sd = oracle.decode_step("vector_decay", q[:, t], k[:, t], v[:, t], lg[:, t], s_prev, lib=lib)
    assert _rel(od, o[:, t]) <= 1e-12 and _rel(sd, s) <= 1e-12


# ---------------------------------------------------------------------------
# Short causal depthwise convolution (wln20, DeltaNet section)
# ---------------------------------------------------------------------------
def pin_conv_library_convolve(lib):
    """Each channel's output is the head of the full 1-D convolution of its
    history (window, then inputs) with its own taps: numpy.convolve's
    definition sum_tau w[tau] x[n - tau] is the page's formula, with the window
    prepended (a textbook routine, not the oracle's loop)."""
    r = _rng(30)
    B, H, L, d, K = 2, 3, 19, 5, 4
    x = r.standard_normal((B, H, L, d))
    w = r.standard_normal((H, d, K))
    st = r.standard_normal((B, H, K - 1, d))
    y, so = oracle.short_conv(x, w, st, lib=lib)
    ref = np.empty_like(y)
    for b in range(B):
        for h in range(H):
            for c in range(d):
                hist = np.concatenate([st[b, h, :, c], x[b, h, :, c]])
                ref[b, h, :, c] = np.convolve(hist, w[h, c], mode="full")[K - 1:K - 1 + L]
    assert _rel(y, ref) <= 1e-13, _rel(y, ref)
    assert np.array_equal(so, x[:, :, L - K + 1:, :])
    # no window: the sequence starts from zeros
    y0, _ = oracle.short_conv(x, w, None, lib=lib)
    for c in range(d):
        ref0 = np.convolve(x[1, 2, :, c], w[2, c], mode="full")[:L]
        assert _rel(y0[1, 2, :, c], ref0) <= 1e-13


def pin_conv_fraction_bruteforce(lib):
    """Exact rational evaluation of y_t = sum_tau w_tau x_{t-tau} on small
    integers and halves (every fp64 step of the oracle is then exact)."""
    r = _rng(31)
    B, H, L, d, K = 1, 2, 7, 3, 3
    x = r.integers(-4, 5, (B, H, L, d)).astype(np.float64)
    w = r.integers(-3, 4, (H, d, K)).astype(np.float64) / 2
    st = r.integers(-4, 5, (B, H, K - 1, d)).astype(np.float64)
    y, _ = oracle.short_conv(x, w, st, lib=lib)
    for h in range(H):
        for c in range(d):
            hist = [Fraction(int(v)) for v in st[0, h, :, c]] + [Fraction(int(v)) for v in x[0, h, :, c]]
            for t in range(L):
                acc = Fraction(0)
                for tau in range(K):
                    acc += Fraction(w[h, c, tau]) * hist[K - 1 + t - tau]
                assert Fraction(y[0, h, t, c]) == acc, (h, c, t)


def pin_conv_delta_taps_shift(lib):
    """A one-hot tap at tau turns the convolution into a delay by tau tokens, with
    the window supplying the first tau outputs; K = 1 is a per-channel scale."""
    r = _rng(32)
    B, H, L, d, K = 2, 2, 9, 4, 4
    x = r.standard_normal((B, H, L, d))
    st = r.standard_normal((B, H, K - 1, d))
    hist = np.concatenate([st, x], axis=2)
    for tau in range(K):
        w = np.zeros((H, d, K))
        w[:, :, tau] = 1.0
        y, _ = oracle.short_conv(x, w, st, lib=lib)
        assert np.array_equal(y, hist[:, :, K - 1 - tau:K - 1 - tau + L, :]), tau
    w1 = r.standard_normal((H, d, 1))
    y1, s1 = oracle.short_conv(x, w1, None, lib=lib)
    assert np.array_equal(y1, x * w1[None, :, None, :, 0])
    assert s1.shape == (B, H, 0, d)


def pin_conv_chunked_carry(lib):
    """Convolving a sequence in pieces, carrying the window of the last K-1
    inputs, equals one pass; pieces shorter than the window shift it."""
    r = _rng(33)
    B, H, d, K = 2, 2, 3, 4
    x = r.standard_normal((B, H, 20, d))
    w = r.standard_normal((H, d, K))
    st0 = r.standard_normal((B, H, K - 1, d))
    y, s = oracle.short_conv(x, w, st0, lib=lib)
    for cuts in ((7,), (1, 2, 3), (2, 17)):
        parts, st, t0 = [], st0, 0
        for t1 in list(cuts) + [20]:
            yp, st = oracle.short_conv(x[:, :, t0:t1], w, st, lib=lib)
            parts.append(yp)
            t0 = t1
        assert np.array_equal(np.concatenate(parts, axis=2), y), cuts
        assert np.array_equal(st, s), cuts


# ---------------------------------------------------------------------------
# Backward pass (gradients through the recurrence)
# ---------------------------------------------------------------------------
def _bwd_case(r, variant, B=2, L=9, dk=4, dv=3):
    q, k = r.standard_normal((B, L, dk)), r.standard_normal((B, L, dk))
    v, do = r.standard_normal((B, L, dv)), r.standard_normal((B, L, dv))
    lg = None
    if variant == "decay":
        lg = -0.6 * r.random((B, L))
    elif variant == "vector_decay":
        lg = -0.6 * r.random((B, L, dk))
    s0 = r.standard_normal((B, dk, dv))
    dso = r.standard_normal((B, dk, dv))
    return q, k, v, do, lg, s0, dso


def pin_backward_finite_differences(lib):
    """Every gradient matches the central difference of the forward oracle's loss
    <do, O> + <dS_L, S_L> along a random direction (fp64, step 1e-6)."""
    r = _rng(50)
    for variant in ("plain", "decay", "vector_decay"):
        q, k, v, do, lg, s0, dso = _bwd_case(r, variant)

        def loss(q_, k_, v_, lg_, s0_):
            o, s, _ = oracle.forward(variant, q_, k_, v_, log_gate=lg_, state_in=s0_, lib=lib)
            return float((o * do).sum() + (s * dso).sum())

        dq, dk, dv, dlg, dsi = oracle.backward(variant, q, k, v, do, lg, s0, dso, lib=lib)
        eps = 1e-6
        args = [q, k, v, lg, s0]
        grads = [dq, dk, dv, dlg, dsi]
        for ai, (x, gx) in enumerate(zip(args, grads)):
            if x is None:
                continue
            u = r.standard_normal(x.shape)
            plus, minus = list(args), list(args)
            plus[ai], minus[ai] = x + eps * u, x - eps * u
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = float((gx * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (variant, ai, fd, an)


def _gdn_bwd_case(r, B=2, L=9, dk=4, dv=3, gated=True):
    q = r.standard_normal((B, L, dk))
    k = r.standard_normal((B, L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)          # unit keys, as the workload
    v, do = r.standard_normal((B, L, dv)), r.standard_normal((B, L, dv))
    lg = -0.6 * r.random((B, L)) if gated else None
    be = 0.1 + 0.8 * r.random((B, L))
    s0 = r.standard_normal((B, dk, dv))
    dso = r.standard_normal((B, dk, dv))
    return q, k, v, do, lg, be, s0, dso


def pin_backward_gdn_finite_differences(lib):
    """Gated delta rule: every gradient (q, k, v, log-gates, beta, initial state)
    matches the central difference of the forward oracle's loss
    <do, O> + <dS_L, S_L> along a random direction, with and without log-gates
    (fp64, step 1e-6)."""
    r = _rng(53)
    for gated in (True, False):
        q, k, v, do, lg, be, s0, dso = _gdn_bwd_case(r, gated=gated)

        def loss(q_, k_, v_, lg_, be_, s0_):
            o, s, _ = oracle.forward("gated_delta", q_, k_, v_, log_gate=lg_, beta=be_, state_in=s0_,
                                     lib=lib)
            return float((o * do).sum() + (s * dso).sum())

        dq, dk, dv, dlg, dsi, dbe = oracle.backward("gated_delta", q, k, v, do, lg, s0, dso, lib=lib,
                                                    beta=be)
        assert (dlg is None) == (not gated)
        eps = 1e-6
        args = [q, k, v, lg, be, s0]
        grads = [dq, dk, dv, dlg, dbe, dsi]
        for ai, (x, gx) in enumerate(zip(args, grads)):
            if x is None:
                continue
            u = r.standard_normal(x.shape)
            plus, minus = list(args), list(args)
            plus[ai], minus[ai] = x + eps * u, x - eps * u
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = float((gx * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gated, ai, fd, an)


def pin_backward_gdn_reductions(lib):
    """beta = 0 leaves only the decay S_t = alpha_t S_{t-1}: dq, the log-gate
    gradient and dS_0 equal the decay backward with zero keys, and dk, dv vanish.
    A zero log-gate equals the ungated rule (alpha = 1, DeltaNet)."""
    r = _rng(54)
    q, k, v, do, lg, be, s0, dso = _gdn_bwd_case(r, L=11)
    z = np.zeros_like(be)
    dq, dk, dv, dlg, dsi, dbe = oracle.backward("gated_delta", q, k, v, do, lg, s0, dso, lib=lib, beta=z)
    rq, _, _, rlg, rsi = oracle.backward("decay", q, np.zeros_like(k), v, do, lg, s0, dso, lib=lib)
    assert _rel(dq, rq) <= 1e-13 and _rel(dlg, rlg) <= 1e-13 and _rel(dsi, rsi) <= 1e-13
    assert np.abs(dk).max() == 0.0 and np.abs(dv).max() == 0.0
    g0 = oracle.backward("gated_delta", q, k, v, do, np.zeros_like(lg), s0, dso, lib=lib, beta=be)
    g1 = oracle.backward("gated_delta", q, k, v, do, None, s0, dso, lib=lib, beta=be)
    for i in (0, 1, 2, 4, 5):
        assert _rel(g0[i], g1[i]) <= 1e-14, i


def pin_backward_plain_closed_form(lib):
    """PLAIN with an initial state: O = (Q K^T (.) M) V + Q S_0 and S_L = S_0 + K^T V
    give dQ = (dO V^T (.) M) K + dO S_0^T, dK = (dO V^T (.) M)^T Q + V dS_L^T,
    dV = (Q K^T (.) M)^T dO + K dS_L and dS_0 = Q^T dO + dS_L (matrix calculus of the
    parallel form, tensorplay section 2.1)."""
    r = _rng(51)
    q, k, v, do, _, s0, dso = _bwd_case(r, "plain", B=2, L=23, dk=5, dv=4)
    dq, dk, dv, _, dsi = oracle.backward("plain", q, k, v, do, None, s0, dso, lib=lib)
    M = _mask(23)
    P = (do @ v.transpose(0, 2, 1)) * M
    A = (q @ k.transpose(0, 2, 1)) * M
    assert _rel(dq, P @ k + do @ s0.transpose(0, 2, 1)) <= 1e-12
    assert _rel(dk, P.transpose(0, 2, 1) @ q + v @ dso.transpose(0, 2, 1)) <= 1e-12
    assert _rel(dv, A.transpose(0, 2, 1) @ do + k @ dso) <= 1e-12
    assert _rel(dsi, q.transpose(0, 2, 1) @ do + dso) <= 1e-12


def pin_backward_gate_identity(lib):
    """The output and final state depend on the cumulative log-gates G only through
    differences G_r - G_s (and G_L for the final state), so
    dl_t = sum_{u >= t} (q_u . dq_u - k_u . dk_u) + <dS_L, S_L>, summed over the key
    channel for the scalar gate and per channel for the vector gate. The gate of
    token m multiplies only the state after token m - 1, so the sum may restart
    there: for t < m, dl_t = sum_{t <= u < m} (q_u . dq_u - k_u . dk_u) + <dS_m, S_m>,
    with S_m the state after the first m tokens and dS_m its gradient (from the
    backward of the remaining tokens started from S_m) -- the form the kernels use
    at every chunk end."""
    r = _rng(52)
    for variant in ("decay", "vector_decay"):
        q, k, v, do, lg, s0, dso = _bwd_case(r, variant, L=17)
        dq, dk, dv, dlg, _ = oracle.backward(variant, q, k, v, do, lg, s0, dso, lib=lib)
        _, sL, _ = oracle.forward(variant, q, k, v, log_gate=lg, state_in=s0, lib=lib)
        per = q * dq - k * dk                              # [B, L, dk]
        tail = (dso * sL).sum(-1)                          # [B, dk]
        if variant == "decay":
            per = per.sum(-1)
            tail = tail.sum(-1)[:, None]
        else:
            tail = tail[:, None, :]
        ref = np.flip(np.cumsum(np.flip(per, 1), 1), 1) + tail
        assert _rel(dlg, ref) <= 1e-12, (variant, _rel(dlg, ref))
        for m in (4, 8, 12):
            _, sm, _ = oracle.forward(variant, q[:, :m], k[:, :m], v[:, :m], log_gate=lg[:, :m], state_in=s0,
                                      lib=lib)
            dsm = oracle.backward(variant, q[:, m:], k[:, m:], v[:, m:], do[:, m:], lg[:, m:], sm, dso,
                                  lib=lib)[4]
            head = (dsm * sm).sum(-1)                      # [B, dk]
            head = head.sum(-1)[:, None] if variant == "decay" else head[:, None, :]
            restart = np.flip(np.cumsum(np.flip(per[:, :m], 1), 1), 1) + head
            assert _rel(dlg[:, :m], restart) <= 1e-12, (variant, m, _rel(dlg[:, :m], restart))


def pin_backward_gdn_gate_identity(lib):
    """Gated delta rule: in the variables S'_t = S_t e^{-G_t} the recurrence is
    gate-free with queries q_t e^{G_t} and values v_t e^{-G_t}, and the final state
    is e^{G_L} S'_L, so dl_t = sum_{u >= t} (q_u . dq_u - v_u . dv_u) + <dS_L, S_L>.
    The gate of token t + 1 multiplies only S_t, so the same sum from any token t + 1
    on is <dS_t, S_t> of the state after token t and its gradient: taking the state
    after token 7 from a forward run over the first 8 tokens and its gradient from
    the backward of the remaining tokens started from it."""
    r = _rng(55)
    q, k, v, do, lg, be, s0, dso = _gdn_bwd_case(r, L=17)
    dq, dk, dv, dlg, dsi, dbe = oracle.backward("gated_delta", q, k, v, do, lg, s0, dso, lib=lib, beta=be)
    _, sL, _ = oracle.forward("gated_delta", q, k, v, log_gate=lg, beta=be, state_in=s0, lib=lib)
    per = (q * dq).sum(-1) - (v * dv).sum(-1)
    ref = np.flip(np.cumsum(np.flip(per, 1), 1), 1) + (dso * sL).sum((-1, -2))[:, None]
    assert _rel(dlg, ref) <= 1e-12, _rel(dlg, ref)
    m = 8
    _, s8, _ = oracle.forward("gated_delta", q[:, :m], k[:, :m], v[:, :m], log_gate=lg[:, :m], beta=be[:, :m],
                              state_in=s0, lib=lib)
    tail = oracle.backward("gated_delta", q[:, m:], k[:, m:], v[:, m:], do[:, m:], lg[:, m:], s8, dso, lib=lib,
                           beta=be[:, m:])
    assert _rel(dlg[:, m], (tail[4] * s8).sum((-1, -2))) <= 1e-12


def _norm_bwd_case(r, B=2, L=9, dk=4, dv=3):
    """Positive features (elu + 1 of Gaussians), so every denominator is positive."""
    phi = lambda x: np.where(x > 0, x + 1.0, np.exp(x))
    q, k = phi(r.standard_normal((B, L, dk))), phi(r.standard_normal((B, L, dk)))
    v, do = r.standard_normal((B, L, dv)), r.standard_normal((B, L, dv))
    z0 = phi(r.standard_normal((B, dk)))
    s0 = r.standard_normal((B, dk, dv))
    dso, dzo = r.standard_normal((B, dk, dv)), r.standard_normal((B, dk))
    return q, k, v, do, s0, z0, dso, dzo


def pin_backward_norm_finite_differences(lib):
    """Normalized variant: every gradient (q, k, v, initial state and normalizer)
    matches the central difference of the forward oracle's loss
    <do, O> + <dS_L, S_L> + <dz_L, z_L> along a random direction (fp64, step 1e-6)."""
    r = _rng(56)
    q, k, v, do, s0, z0, dso, dzo = _norm_bwd_case(r)

    def loss(q_, k_, v_, s0_, z0_):
        o, s, z = oracle.forward("normalized", q_, k_, v_, state_in=s0_, z_in=z0_, lib=lib)
        return float((o * do).sum() + (s * dso).sum() + (z * dzo).sum())

    dq, dk, dv, dlg, dsi, dzi = oracle.backward("normalized", q, k, v, do, None, s0, dso, lib=lib, z_in=z0,
                                                d_z_out=dzo)
    assert dlg is None
    eps = 1e-6
    args = [q, k, v, s0, z0]
    for ai, (x, gx) in enumerate(zip(args, [dq, dk, dv, dsi, dzi])):
        u = r.standard_normal(x.shape)
        plus, minus = list(args), list(args)
        plus[ai], minus[ai] = x + eps * u, x - eps * u
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float((gx * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (ai, fd, an)


def pin_backward_norm_constant_v(lib):
    """Normalized variant with every value equal to c and S_0 = z_0 c^T: each output
    is exactly c whatever q and k are (the weights sum to one, proig-chaa section
    14), so the gradients of <do, O> with respect to q and k vanish, and dv_t is
    the sum over s >= t of (q_s . k_t / den_s) do_s."""
    r = _rng(57)
    q, k, _, do, _, z0, _, _ = _norm_bwd_case(r, L=7)
    c = r.standard_normal(3)
    v = np.broadcast_to(c, (2, 7, 3)).copy()
    s0 = z0[:, :, None] * c[None, None, :]
    dq, dk, dv, _, _, _ = oracle.backward("normalized", q, k, v, do, None, s0, None, lib=lib, z_in=z0)
    scale = np.abs(do).max() * np.abs(c).max() / min(q.min(), k.min())
    assert np.abs(dq).max() <= 1e-13 * scale and np.abs(dk).max() <= 1e-13 * scale
    z = z0[:, None, :] + np.cumsum(k, axis=1)
    den = (q * z).sum(-1)
    w = np.einsum("bsi,bti->bst", q, k) / den[:, :, None]          # [b, s, t]: q_s . k_t / den_s
    ref = np.einsum("bst,bsj->btj", np.triu(np.ones((7, 7)))[None].transpose(0, 2, 1) * w, do)
    assert _rel(dv, ref) <= 1e-12, _rel(dv, ref)


ALL_PINS = [
    pin_plain_quadratic, pin_plain_fraction_bruteforce, pin_plain_final_state,
    pin_normalized_quadratic, pin_normalized_constant_v, pin_normalized_hull,
    pin_decay_quadratic, pin_decay_zero_gate_is_plain, pin_decay_fraction_half,
    pin_gdn_retrieve_merge_overwrite, pin_gdn_alpha_one_is_deltanet,
    pin_gdn_beta_zero_pure_decay, pin_gdn_onehot_recall, pin_gdn_unit_key_identity,
    pin_gdn_fraction_product_expansion, pin_gdn_chunkwise_wy,
    pin_decode_one_decay_step, pin_prefill_then_decode, pin_resume_all_variants,
    pin_decode_gdn_step, pin_prefill_then_decode_gdn,
    pin_conv_library_convolve, pin_conv_fraction_bruteforce, pin_conv_delta_taps_shift,
    pin_conv_chunked_carry,
    pin_vector_decay_parallel_form, pin_vector_decay_uniform_is_scalar, pin_vector_decay_fraction,
    pin_vector_decay_channel_isolation, pin_vector_decay_resume_and_decode,
    pin_backward_finite_differences, pin_backward_plain_closed_form, pin_backward_gate_identity,
    pin_backward_gdn_finite_differences, pin_backward_gdn_reductions, pin_backward_gdn_gate_identity,
    pin_backward_norm_finite_differences, pin_backward_norm_constant_v,
    pin_kda_chunkwise_wy, pin_kda_uniform_gate_is_gdn, pin_kda_beta_zero_pure_decay,
    pin_kda_unit_key_overwrite, pin_kda_decode_and_resume,
]
