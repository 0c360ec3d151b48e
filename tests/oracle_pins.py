"""Pins that tie the fp64 oracle to facts fixed outside the oracle itself.

Each pin takes a loaded oracle (``oracle.Oracle``) and raises AssertionError if
the oracle disagrees with a closed form, an invariant of the gated delta rule,
a hand-worked example or a library routine.  ``tests/test_oracle_pins.py`` runs
them on the oracle; ``tests/test_oracle_mutations.py`` plants mistakes in a
copy of the oracle's C source and checks that every planted mistake fails at
least one pin.

The rule pinned (Gated Delta Networks, Yang et al., ICLR 2025; named in the
Qwen3.5-0.8B chat guide, section "Architektur"):
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = scale * S_t q_t
Shapes use d_k != d_v wherever possible, so a transposed state fails.
"""
from __future__ import annotations

import math

import numpy as np

RNG_SEED = 20260101


def _rng(tag: int) -> np.random.Generator:
    return np.random.default_rng([RNG_SEED, tag])


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 0.0)
    assert err <= tol * scale, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _unit(x):
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


# ---------------------------------------------------------------------------
# recurrence pins
# ---------------------------------------------------------------------------

def pin_handworked_two_tokens(orc):
    """Two tokens, d_k=3, d_v=2, worked by hand from the rule.

    Token 1: k=(1,0,0), v=(2,4), a=1/2, b=1/2, q=(1,1,1) from S0=0:
        S1 = b v k^T = [[1,0,0],[2,0,0]];  o1 = S1 q = (1, 2).
    Token 2: k=(0.6,0.8,0), v=(1,-1), a=1/4, b=1/4, q=(0,1,0):
        S1 k = (0.6, 1.2)
        S2 = a S1 - a b (S1 k) k^T + b v k^T
           = [[0.25,0,0],[0.5,0,0]] - (1/16)[[0.36,0.48,0],[0.72,0.96,0]]
             + (1/4)[[0.6,0.8,0],[-0.6,-0.8,0]]
           = [[0.3775, 0.17, 0], [0.305, -0.26, 0]];  o2 = S2 q = (0.17, -0.26).
    """
    q = np.array([[[1, 1, 1]], [[0, 1, 0]]], np.float32)
    k = np.array([[[1, 0, 0]], [[0.6, 0.8, 0]]], np.float32)
    v = np.array([[[2, 4]], [[1, -1]]], np.float32)
    g = np.log(np.array([[0.5], [0.25]])).astype(np.float32)
    b = np.array([[0.5], [0.25]], np.float32)
    o, S = orc.recurrence(q, k, v, g, b, np.array([0, 2]))
    _close(o[:, 0, :], [[1, 2], [0.17, -0.26]], 1e-6, "hand-worked outputs")
    _close(S[0, 0], [[0.3775, 0.17, 0], [0.305, -0.26, 0]], 1e-6, "hand-worked state")


def pin_single_token_closed_form(orc):
    """From S0 = 0 one token gives S_1 = b v k^T and o_1 = scale b (k.q) v."""
    r = _rng(1)
    N, H, HV, dk, dv = 5, 1, 2, 8, 6
    q = _unit(r.standard_normal((N, H, dk)))
    k = _unit(r.standard_normal((N, H, dk)))
    v = r.standard_normal((N, HV, dv)).astype(np.float32)
    g = -r.random((N, HV)).astype(np.float32)
    b = r.random((N, HV)).astype(np.float32)
    scale = 0.75
    o, S = orc.recurrence(q, k, v, g, b, np.arange(N + 1), scale=scale)
    qd, kd, vd, bd = (x.astype(np.float64) for x in (q, k, v, b))
    for n in range(N):
        for h in range(HV):
            kk, qq = kd[n, 0], qd[n, 0]
            _close(S[n, h], bd[n, h] * np.outer(vd[n, h], kk), 1e-14, "S_1 = b v k^T")
            _close(o[n, h], scale * bd[n, h] * (kk @ qq) * vd[n, h], 1e-14, "o_1")


def pin_decay_only(orc):
    """With b = 0 the state only decays: S_t = (prod a) S0, o_t = scale S_t q_t."""
    r = _rng(2)
    T, H, HV, dk, dv = 9, 1, 1, 7, 5
    q = _unit(r.standard_normal((T, H, dk)))
    k = _unit(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, HV, dv)).astype(np.float32)
    g = (-0.3 * r.random((T, HV))).astype(np.float32)
    b = np.zeros((T, HV), np.float32)
    s0 = r.standard_normal((1, HV, dv, dk))
    o, S = orc.recurrence(q, k, v, g, b, np.array([0, T]), s0=s0, scale=1.5)
    cum = np.cumsum(g[:, 0].astype(np.float64))
    for t in range(T):
        _close(o[t, 0], 1.5 * math.exp(cum[t]) * (s0[0, 0] @ q[t, 0].astype(np.float64)),
               1e-13, f"decayed readout t={t}")
    _close(S[0, 0], math.exp(cum[-1]) * s0[0, 0], 1e-13, "decay-only final state")


def pin_exact_retrieval(orc):
    """a = 1, b = 1 and orthonormal keys: S k_i = v_i for every stored pair.

    Keys are the rows of the 16 x 16 Hadamard matrix divided by 4 (orthonormal,
    and exact in bf16).  Reading with q_t = k_t retrieves v_t at once."""
    Hd = np.array([[1.0]])
    while Hd.shape[0] < 16:
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])
    keys = (Hd / 4.0).astype(np.float32)
    r = _rng(3)
    T, dv = 16, 12
    perm = r.permutation(16)
    k = keys[perm][:, None, :]
    v = r.standard_normal((T, 1, dv)).astype(np.float32)
    g = np.zeros((T, 1), np.float32)
    b = np.ones((T, 1), np.float32)
    o, S = orc.recurrence(k, k, v, g, b, np.array([0, T]))
    _close(o[:, 0], v[:, 0], 1e-14, "o_t = v_t when q_t = k_t")
    for i in range(T):
        _close(S[0, 0] @ k[i, 0].astype(np.float64), v[i, 0], 1e-14, f"S k_{i} = v_{i}")


def pin_linear_readout(orc):
    """a = 1, b = 0: the state never changes and o_t = scale S0 q_t."""
    r = _rng(4)
    T, dk, dv = 5, 6, 9
    q = r.standard_normal((T, 1, dk)).astype(np.float32)
    k = r.standard_normal((T, 1, dk)).astype(np.float32)
    v = r.standard_normal((T, 1, dv)).astype(np.float32)
    s0 = r.standard_normal((1, 1, dv, dk))
    o, S = orc.recurrence(q, k, v, np.zeros((T, 1), np.float32), np.zeros((T, 1), np.float32),
                          np.array([0, T]), s0=s0, scale=-2.0)
    _close(o[:, 0], -2.0 * (q[:, 0].astype(np.float64) @ s0[0, 0].T), 1e-14, "o = scale S0 q")
    _close(S, s0, 0.0, "state unchanged")


def _prefix_batch(q, k, v, g, b):
    """Pack sequences 0..T where sequence j is the first j tokens."""
    T = q.shape[0]
    idx = np.concatenate([np.arange(j) for j in range(T + 1)]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(np.arange(T + 1))]).astype(np.int32)
    return q[idx], k[idx], v[idx], g[idx], b[idx], cu


def pin_delta_rule_invariants(orc):
    """Characterising invariants of one step, checked token by token.

    For any k_t:  S_t k_t = a_t (1 - b_t |k_t|^2) S_{t-1} k_t + b_t |k_t|^2 v_t
    and for x orthogonal to k_t:  S_t x = a_t S_{t-1} x.
    Together these fix S_t.  Also o_t = scale S_t q_t (readout after the
    update).  S_{t-1} and S_t come from a packed batch of all prefixes, which
    also exercises the packed indexing."""
    r = _rng(5)
    T, H, HV, dk, dv = 6, 2, 4, 8, 5
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = (0.8 * _unit(r.standard_normal((T, H, dk)))).astype(np.float32)
    v = r.standard_normal((T, HV, dv)).astype(np.float32)
    g = (-r.random((T, HV))).astype(np.float32)
    b = r.random((T, HV)).astype(np.float32)
    s0 = r.standard_normal((T + 1, HV, dv, dk)) * 0.0 + r.standard_normal((1, HV, dv, dk))
    Q, K, V, G, B, cu = _prefix_batch(q, k, v, g, b)
    o, S = orc.recurrence(Q, K, V, G, B, cu, s0=s0, scale=0.5)
    r_of = HV // H
    for t in range(1, T + 1):
        for h in range(HV):
            hk = h // r_of
            kt = k[t - 1, hk].astype(np.float64)
            a = math.exp(float(g[t - 1, h]))
            bb = float(b[t - 1, h])
            Sp, Sn = S[t - 1, h], S[t, h]
            kk = kt @ kt
            want = a * (1 - bb * kk) * (Sp @ kt) + bb * kk * v[t - 1, h].astype(np.float64)
            _close(Sn @ kt, want, 1e-13, f"S_t k_t, t={t} h={h}")
            x = r.standard_normal(dk)
            x -= (x @ kt) / kk * kt
            _close(Sn @ x, a * (Sp @ x), 1e-13, f"S_t x for x orthogonal to k_t, t={t} h={h}")
            last = cu[t + 1] - 1
            _close(o[last, h], 0.5 * (Sn @ q[t - 1, hk].astype(np.float64)), 1e-13,
                   f"o_t = scale S_t q_t, t={t} h={h}")


def pin_scale_linearity(orc):
    """o(scale) = scale * o(1) exactly for powers of two; the state ignores scale."""
    r = _rng(6)
    T, dk, dv = 7, 4, 3
    q = r.standard_normal((T, 1, dk)).astype(np.float32)
    k = _unit(r.standard_normal((T, 1, dk)))
    v = r.standard_normal((T, 1, dv)).astype(np.float32)
    g = (-r.random((T, 1))).astype(np.float32)
    b = r.random((T, 1)).astype(np.float32)
    o1, S1 = orc.recurrence(q, k, v, g, b, np.array([0, T]), scale=1.0)
    o4, S4 = orc.recurrence(q, k, v, g, b, np.array([0, T]), scale=0.25)
    _close(o4, 0.25 * o1, 0.0, "scale linearity")
    _close(S4, S1, 0.0, "state independent of scale")


def pin_grouped_value_heads(orc):
    """HV = 2H with value head h reading key head h // 2 equals a call with
    H' = HV and q, k repeated per value head (the Core AI card's query/key
    head-repeat).  The mapping itself is a convention of this library."""
    r = _rng(7)
    T, H, HV, dk, dv = 11, 2, 4, 6, 5
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = _unit(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, HV, dv)).astype(np.float32)
    g = (-r.random((T, HV))).astype(np.float32)
    b = r.random((T, HV)).astype(np.float32)
    cu = np.array([0, 4, 11])
    og, Sg = orc.recurrence(q, k, v, g, b, cu)
    orr, Sr = orc.recurrence(np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1), v, g, b, cu)
    _close(og, orr, 0.0, "GVA outputs")
    _close(Sg, Sr, 0.0, "GVA states")
    # and a direct check that head 1 (key head 0) differs from head 2 (key head 1)
    one = orc.recurrence(q[:, :1], k[:, :1], v[:, 1:2], g[:, 1:2], b[:, 1:2], cu)[0]
    _close(og[:, 1:2], one, 1e-15, "value head 1 uses key head 0")


def pin_packed_isolation(orc):
    """A packed batch equals separate calls; an empty sequence keeps S0."""
    r = _rng(8)
    lens = [3, 0, 7, 1]
    T = sum(lens)
    H, HV, dk, dv = 1, 2, 5, 4
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = _unit(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, HV, dv)).astype(np.float32)
    g = (-r.random((T, HV))).astype(np.float32)
    b = r.random((T, HV)).astype(np.float32)
    s0 = r.standard_normal((len(lens), HV, dv, dk))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = orc.recurrence(q, k, v, g, b, cu, s0=s0)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        on, Sn = orc.recurrence(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], np.array([0, e - a]),
                                s0=s0[n:n + 1])
        _close(o[a:e], on, 0.0, f"packed outputs seq {n}")
        _close(S[n], Sn[0], 0.0, f"packed state seq {n}")
    _close(S[1], s0[1], 0.0, "empty sequence keeps S0")


def pin_contraction_bound(orc):
    """With |k| <= 1 and 0 <= b <= 1, |I - b k k^T|_2 <= 1, so
    |S_t|_2 <= a_t |S_{t-1}|_2 + b_t |v_t| |k_t|."""
    r = _rng(9)
    T, dk, dv = 12, 6, 6
    q = r.standard_normal((T, 1, dk)).astype(np.float32)
    k = (_unit(r.standard_normal((T, 1, dk))) * r.uniform(0.2, 1.0, (T, 1, 1))).astype(np.float32)
    v = r.standard_normal((T, 1, dv)).astype(np.float32)
    g = (-0.1 * r.random((T, 1))).astype(np.float32)
    b = r.random((T, 1)).astype(np.float32)
    s0 = r.standard_normal((T + 1, 1, dv, dk)) * 0 + r.standard_normal((1, 1, dv, dk))
    Q, K, V, G, B, cu = _prefix_batch(q, k, v, g, b)
    _, S = orc.recurrence(Q, K, V, G, B, cu, s0=s0)
    for t in range(1, T + 1):
        lhs = np.linalg.norm(S[t, 0], 2)
        rhs = (math.exp(float(g[t - 1, 0])) * np.linalg.norm(S[t - 1, 0], 2)
               + float(b[t - 1, 0]) * np.linalg.norm(v[t - 1, 0]) * np.linalg.norm(k[t - 1, 0]))
        assert lhs <= rhs * (1 + 1e-12), f"contraction bound fails at t={t}: {lhs} > {rhs}"


def chunked_reference(q, k, v, g, b, s0, C, scale=1.0):
    """An independent route to the same result: the chunked (WY/UT) form in
    numpy fp64, one sequence and one head.  Within a chunk with cumulative
    log-decays G, A_ts = b_t e^{G_t - G_s} (k_t . k_s) for s < t,
    T = (I + A)^-1, U = T (diag(b) V - diag(b e^G) K S^T);
    O = scale (diag(e^G) Q S^T + (tril(Q K^T) * e^{G_t - G_s}) U);
    S <- e^{G_n} S + U^T diag(e^{G_n - G}) K."""
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    g, b = g.astype(np.float64), b.astype(np.float64)
    S = s0.astype(np.float64).copy()
    T = q.shape[0]
    out = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, V, gg, bb = q[sl], k[sl], v[sl], g[sl], b[sl]
        G = np.cumsum(gg)
        D = np.exp(np.tril(G[:, None] - G[None, :]))
        A = np.tril(bb[:, None] * (K @ K.T) * D, -1)
        Tm = np.linalg.inv(np.eye(len(G)) + A)
        U = Tm @ (bb[:, None] * V - (bb * np.exp(G))[:, None] * (K @ S.T))
        P = np.tril(Q @ K.T) * D
        out[sl] = scale * (np.exp(G)[:, None] * (Q @ S.T) + P @ U)
        S = math.exp(G[-1]) * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
    return out, S


def pin_chunked_equals_step(orc):
    """The chunked (WY/UT) form, an independent algorithm, reaches the same
    outputs and final state as the oracle's step loop, for chunk sizes that
    leave a partial last chunk."""
    r = _rng(10)
    T, dk, dv = 70, 16, 12
    q = _unit(r.standard_normal((T, 1, dk)))
    k = _unit(r.standard_normal((T, 1, dk)))
    v = r.standard_normal((T, 1, dv)).astype(np.float32)
    g = (-0.05 * np.logaddexp(0, r.standard_normal((T, 1)))).astype(np.float32)
    b = (1 / (1 + np.exp(-r.standard_normal((T, 1))))).astype(np.float32)
    s0 = r.standard_normal((1, 1, dv, dk)) * 0.1
    o, S = orc.recurrence(q, k, v, g, b, np.array([0, T]), s0=s0, scale=0.5)
    for C in (16, 32, 64):
        oc, Sc = chunked_reference(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], s0[0, 0], C, 0.5)
        _close(o[:, 0], oc, 1e-12, f"chunked (C={C}) outputs")
        _close(S[0, 0], Sc, 1e-12, f"chunked (C={C}) state")


def pin_transition_product(orc):
    """S_T = S_0 M_1 ... M_T + sum_t b_t v_t k_t^T M_{t+1} ... M_T with
    M_t = a_t (I - b_t k_t k_t^T): the unrolled product form."""
    r = _rng(11)
    T, dk, dv = 8, 5, 3
    q = r.standard_normal((T, 1, dk)).astype(np.float32)
    k = _unit(r.standard_normal((T, 1, dk)))
    v = r.standard_normal((T, 1, dv)).astype(np.float32)
    g = (-r.random((T, 1))).astype(np.float32)
    b = r.random((T, 1)).astype(np.float32)
    s0 = r.standard_normal((1, 1, dv, dk))
    _, S = orc.recurrence(q, k, v, g, b, np.array([0, T]), s0=s0)
    kd, vd = k[:, 0].astype(np.float64), v[:, 0].astype(np.float64)
    M = [math.exp(float(g[t, 0])) * (np.eye(dk) - float(b[t, 0]) * np.outer(kd[t], kd[t]))
         for t in range(T)]
    acc = s0[0, 0].copy()
    for t in range(T):
        acc = acc @ M[t]
    for t in range(T):
        term = float(b[t, 0]) * np.outer(vd[t], kd[t])
        for r_ in range(t + 1, T):
            term = term @ M[r_]
        acc = acc + term
    _close(S[0, 0], acc, 1e-13, "transition-product form")


# ---------------------------------------------------------------------------
# RMSNormGated pins
# ---------------------------------------------------------------------------

def pin_norm_library(orc):
    """y = rms_norm(x, w, eps) * silu(z), with torch's CPU rms_norm and silu in fp64."""
    import torch
    r = _rng(20)
    x = r.standard_normal((7, 3, 16)) * 3.0
    z = r.standard_normal((7, 3, 16)).astype(np.float32)
    w = r.standard_normal(16).astype(np.float32)
    eps = 1e-6
    y = orc.rmsnorm_gated(x, z, w, eps=eps)
    xt = torch.from_numpy(x)
    want = torch.nn.functional.rms_norm(xt, (16,), torch.from_numpy(w.astype(np.float64)), eps)
    want = want * torch.nn.functional.silu(torch.from_numpy(z.astype(np.float64)))
    _close(y, want.numpy(), 1e-14, "RMSNormGated vs torch rms_norm * silu")


def pin_norm_closed_forms(orc):
    """z = 0 gives y = 0; a constant group x = c gives
    y = sign(c) * w * silu(z) * sqrt(c^2 / (c^2 + eps))."""
    r = _rng(21)
    x = r.standard_normal((4, 8))
    y = orc.rmsnorm_gated(x, np.zeros((4, 8), np.float32), np.ones(8, np.float32))
    _close(y, np.zeros_like(y), 0.0, "zero gate")
    c = np.array([0.5, -2.0, 1e-3, 3.0])
    xc = np.repeat(c[:, None], 8, axis=1)
    z = r.standard_normal((4, 8)).astype(np.float32)
    w = r.standard_normal(8).astype(np.float32)
    eps = 1e-6
    y = orc.rmsnorm_gated(xc, z, w, eps=eps)
    zd = z.astype(np.float64)
    silu = zd / (1 + np.exp(-zd))
    want = np.sign(c)[:, None] * w[None, :] * silu * np.sqrt(c ** 2 / (c ** 2 + eps))[:, None]
    _close(y, want, 1e-14, "constant group")


# ---------------------------------------------------------------------------
# decode-layer pins: gate activations, q/k L2 norm, slot table
# ---------------------------------------------------------------------------

def pin_gate_closed_forms(orc):
    """g = -exp(A_log) softplus(a_raw + dt_bias), beta = sigmoid(b_raw):
    softplus(0) = ln 2, softplus(x) - softplus(-x) = x, softplus(40) = 40 to
    1e-17, softplus(-40) = e^-40 to 1e-17; sigmoid(0) = 1/2,
    sigmoid(+-ln 3) = 3/4, 1/4; the per-head scale multiplies by exp(A_log)."""
    A = np.array([0.0, 0.6931471805599453, -1.25, 2.0], dtype=np.float32)
    sc = np.exp(A.astype(np.float64))
    dt = np.array([0.0, 0.25, -1.5, 3.0], dtype=np.float32)
    # a_raw + dt_bias = 0, 40, -40 (all exact in float32)
    a_raw = np.stack([-dt, 40.0 - dt, -40.0 - dt]).astype(np.float32)
    b_raw = np.array([[0.0] * 4, [math.log(3.0)] * 4, [-math.log(3.0)] * 4], dtype=np.float32)
    g, beta = orc.gates(a_raw, b_raw, A, dt)
    _close(g[0] / sc, -math.log(2.0) * np.ones(4), 1e-15, "softplus(0) = ln 2")
    _close(g[1] / sc, -40.0 * np.ones(4), 1e-15, "softplus(40)")
    _close(g[2] / (sc * math.exp(-40.0)), -np.ones(4), 1e-12, "softplus(-40) / e^-40")
    _close(beta[0], 0.5 * np.ones(4), 1e-15, "sigmoid(0)")
    b3 = np.float64(np.float32(math.log(3.0)))
    _close(beta[1], np.full(4, 1.0 / (1.0 + math.exp(-b3))), 1e-15, "sigmoid(ln 3)")
    _close(beta[1], 0.75 * np.ones(4), 1e-7, "sigmoid(ln 3) = 3/4")
    _close(beta[2], 0.25 * np.ones(4), 1e-7, "sigmoid(-ln 3) = 1/4")
    # odd part of softplus and the complement of sigmoid on random inputs
    r = _rng(30)
    x = r.standard_normal((5, 4)).astype(np.float32) * 4
    gp, bp = orc.gates(x, x, A, None)
    gm, bm = orc.gates(-x, -x, A, None)
    _close((gp - gm) / sc, -x.astype(np.float64), 1e-14, "softplus(x) - softplus(-x) = x")
    _close(bp + bm, np.ones_like(bp), 1e-15, "sigmoid(x) + sigmoid(-x) = 1")


def pin_gate_library(orc):
    """Against torch's CPU softplus (threshold beyond the range) and sigmoid in fp64."""
    import torch
    r = _rng(31)
    HV = 6
    a_raw = (r.standard_normal((9, HV)) * 3).astype(np.float32)
    b_raw = (r.standard_normal((9, HV)) * 3).astype(np.float32)
    A = r.uniform(0, math.log(16), HV).astype(np.float32)
    dt = r.standard_normal(HV).astype(np.float32)
    g, beta = orc.gates(a_raw, b_raw, A, dt)
    x = torch.from_numpy(a_raw.astype(np.float64)) + torch.from_numpy(dt.astype(np.float64))
    want_g = -torch.exp(torch.from_numpy(A.astype(np.float64))) * \
        torch.nn.functional.softplus(x, beta=1.0, threshold=1000.0)
    want_b = torch.sigmoid(torch.from_numpy(b_raw.astype(np.float64)))
    _close(g, want_g.numpy(), 1e-14, "g vs torch softplus")
    _close(beta, want_b.numpy(), 1e-15, "beta vs torch sigmoid")


def pin_l2norm(orc):
    """x / sqrt(sum x^2 + eps): (3, 4) -> (0.6, 0.8) at eps = 0 and
    (3, 4) / 6 at eps = 11; zero rows stay zero; torch's normalize at eps = 0."""
    import torch
    _close(orc.l2norm(np.array([[3.0, 4.0]]), eps=0.0), [[0.6, 0.8]], 1e-15, "3-4-5")
    _close(orc.l2norm(np.array([[3.0, 4.0]]), eps=11.0), [[0.5, 4.0 / 6.0]], 1e-15, "eps inside")
    _close(orc.l2norm(np.zeros((2, 5)), eps=1e-6), np.zeros((2, 5)), 0.0, "zero row")
    r = _rng(32)
    x = r.standard_normal((7, 16)).astype(np.float32)
    want = torch.nn.functional.normalize(torch.from_numpy(x.astype(np.float64)), dim=-1)
    _close(orc.l2norm(x, eps=0.0), want.numpy(), 1e-15, "vs torch normalize")


def _layer_inputs(tag, N, H, HV, dk, dv):
    r = _rng(tag)
    q = r.standard_normal((N, H, dk)).astype(np.float32)
    k = _unit(r.standard_normal((N, H, dk)))
    v = r.standard_normal((N, HV, dv)).astype(np.float32)
    g = (-r.random((N, HV)) * 0.5).astype(np.float32)
    b = r.random((N, HV)).astype(np.float32)
    return r, q, k, v, g, b


def pin_decode_layer_reduces_to_step(orc):
    """Without the slot table and the norm the layer step is the pinned
    recurrence; with a slot table each sequence advances its own slot, slots no
    sequence names keep their bits, and a skipped sequence reads 0."""
    N, H, HV, dk, dv = 5, 2, 4, 8, 6
    r, q, k, v, g, b = _layer_inputs(33, N, H, HV, dk, dv)
    S = r.standard_normal((N, HV, dv, dk))
    o_ref, s_ref = orc.decode(q, k, v, g, b, S, scale=0.7)
    o, pool = orc.decode_layer(q, k, v, g, b, S, scale=0.7)
    assert np.array_equal(o, o_ref) and np.array_equal(pool, s_ref), "identity slots"
    # pool of 9 slots; sequences 1 and 3 skipped (-1 and 9 lie outside [0, 9))
    slots = np.array([7, -1, 0, 9, 4], dtype=np.int32)
    pool0 = r.standard_normal((9, HV, dv, dk))
    o, pool = orc.decode_layer(q, k, v, g, b, pool0, slots=slots, scale=0.7)
    live = [0, 2, 4]
    o_ref, s_ref = orc.decode(q[live], k[live], v[live], g[live], b[live],
                              pool0[slots[live]], scale=0.7)
    assert np.array_equal(o[live], o_ref), "slot outputs"
    assert np.array_equal(pool[slots[live]], s_ref), "slot states"
    assert np.array_equal(o[[1, 3]], np.zeros((2, HV, dv))), "skipped outputs"
    untouched = [s for s in range(9) if s not in (7, 0, 4)]
    assert np.array_equal(pool[untouched], pool0[untouched]), "untouched slots"


def pin_decode_layer_l2norm(orc):
    """With the q/k norm the step equals the recurrence on normalised q and k
    (to float32 rounding of the normalised inputs) and is unchanged by a
    positive rescaling of q and k (eps = 0)."""
    N, H, HV, dk, dv = 4, 2, 4, 8, 6
    r, q, k, v, g, b = _layer_inputs(34, N, H, HV, dk, dv)
    k = (r.standard_normal((N, H, dk)) * 3).astype(np.float32)
    S = r.standard_normal((N, HV, dv, dk))
    o, pool = orc.decode_layer(q, k, v, g, b, S, l2norm=True, l2_eps=1e-6)
    o_ref, s_ref = orc.decode(orc.l2norm(q, eps=1e-6), orc.l2norm(k, eps=1e-6), v, g, b, S)
    _close(o, o_ref, 1e-6, "l2 outputs")
    _close(pool, s_ref, 1e-6, "l2 states")
    o0, p0 = orc.decode_layer(q, k, v, g, b, S, l2norm=True, l2_eps=0.0)
    o1, p1 = orc.decode_layer(q * 4, k * 0.5, v, g, b, S, l2norm=True, l2_eps=0.0)
    _close(o1, o0, 1e-13, "rescaled q, k")
    _close(p1, p0, 1e-13, "rescaled q, k (state)")
    o2, _ = orc.decode_layer(q, k, v, g, b, S, l2norm=False)
    assert np.max(np.abs(o2 - o0)) > 1e-3, "the norm changes the result"


def pin_decode_layer_gates(orc):
    """Layer step with activated gates: decay a = exp(g) in (0, 1) and, with
    beta = sigmoid(b_raw) and an orthonormal key on a zero state, the stored
    value is read back scaled by beta (the write strength)."""
    N, H, HV, dk, dv = 3, 1, 2, 8, 4
    r = _rng(35)
    a_raw = r.standard_normal((N, HV)).astype(np.float32)
    b_raw = r.standard_normal((N, HV)).astype(np.float32)
    A = np.array([0.5, 1.5], dtype=np.float32)
    g, beta = orc.gates(a_raw, b_raw, A, None)
    assert np.all(g < 0) and np.all(np.exp(g) > 0), "decay in (0, 1)"
    k = np.zeros((N, H, dk), np.float32)
    k[np.arange(N), 0, np.arange(N)] = 1.0
    v = r.standard_normal((N, HV, dv)).astype(np.float32)
    o, _ = orc.decode_layer(k, k, v, g, beta, np.zeros((N, HV, dv, dk)))
    _close(o, beta[:, :, None] * v.astype(np.float64), 1e-15, "read back b v")


# ---------------------------------------------------------------------------
# gated full attention (decode step) and its rotary embedding
# ---------------------------------------------------------------------------

def pin_rope_closed_forms(orc):
    """Position 0 is the identity; dimensions past rd pass unchanged; norms are
    kept; a unit vector on pair i at position p lands on (cos a, sin a) in
    dimensions (i, i + rd/2) with a = p theta^(-2i/rd)."""
    r = _rng(40)
    d, rd, th = 32, 16, 1e7
    x = r.standard_normal((5, d)).astype(np.float32)
    y0 = orc.rope(x, np.zeros(5, np.int32), rd=rd, theta=th)
    _close(y0, x.astype(np.float64), 0.0, "position 0")
    y = orc.rope(x, np.array([1, 7, 100, 4096, 65535]), rd=rd, theta=th)
    _close(y[:, rd:], x[:, rd:].astype(np.float64), 0.0, "unrotated tail")
    _close(np.linalg.norm(y, axis=1), np.linalg.norm(x.astype(np.float64), axis=1), 1e-14, "norm")
    for i, p in ((0, 1), (1, 1), (3, 37), (7, 1000)):
        e = np.zeros((1, d), np.float32)
        e[0, i] = 1.0
        a = p * th ** (-2.0 * i / rd)
        want = np.zeros(d)
        want[i], want[i + rd // 2] = math.cos(a), math.sin(a)
        _close(orc.rope(e, np.array([p]), rd=rd, theta=th)[0], want, 1e-13, f"pair {i} at {p}")


def pin_rope_relative(orc):
    """Rotated dot products depend on the position difference only:
    rope(q, p + s) . rope(k, t + s) = rope(q, p) . rope(k, t)."""
    r = _rng(41)
    d, rd = 64, 32
    q = r.standard_normal((6, d)).astype(np.float32)
    k = r.standard_normal((6, d)).astype(np.float32)
    p = np.array([0, 3, 10, 200, 5000, 1])
    t = np.array([0, 1, 17, 150, 4999, 30000])
    base = np.sum(orc.rope(q, p, rd=rd, theta=1e4) * orc.rope(k, t, rd=rd, theta=1e4), axis=1)
    for sft in (1, 123, 20000):
        moved = np.sum(orc.rope(q, p + sft, rd=rd, theta=1e4) * orc.rope(k, t + sft, rd=rd, theta=1e4), axis=1)
        _close(moved, base, 1e-9, f"shift {sft}")


def _attn_case(tag, N=3, Hq=4, Hkv=2, d=32, Lmax=40):
    r = _rng(tag)
    q = r.standard_normal((N, Hq, d)).astype(np.float32)
    gate = r.standard_normal((N, Hq, d)).astype(np.float32)
    kn = r.standard_normal((N, Hkv, d)).astype(np.float32)
    vn = r.standard_normal((N, Hkv, d)).astype(np.float32)
    kc = r.standard_normal((N, Hkv, Lmax, d)).astype(np.float32)
    vc = r.standard_normal((N, Hkv, Lmax, d)).astype(np.float32)
    pos = r.integers(1, Lmax - 1, N).astype(np.int32)
    return q, gate, kn, vn, kc, vc, pos


def pin_attn_closed_forms(orc):
    """Empty cache: o = v_new * sigmoid(gate) and the appended key is
    rope(k_new, 0) = k_new; q = 0: uniform weights, o = the mean of the
    cache's values and v_new; gate 0 halves o; a dominant score selects its
    value."""
    q, gate, kn, vn, kc, vc, pos = _attn_case(42)
    N, Hq, d = q.shape
    Hkv = kn.shape[1]
    grp = Hq // Hkv
    o, kr = orc.attn_decode(q, kn, vn, kc, vc, np.zeros(N, np.int32), gate=gate, rd=16)
    want = np.repeat(vn, grp, axis=1).astype(np.float64) / (1 + np.exp(-gate.astype(np.float64)))
    _close(o, want, 1e-15, "single position")
    _close(kr, kn.astype(np.float64), 0.0, "appended key at position 0")
    o, _ = orc.attn_decode(np.zeros_like(q), kn, vn, kc, vc, pos, rd=16)
    for n in range(N):
        vals = np.concatenate([vc[n, :, :pos[n]], vn[n, :, None]], axis=1).astype(np.float64)
        _close(o[n], np.repeat(vals.mean(axis=1), grp, axis=0), 1e-14, "uniform weights")
    o1, _ = orc.attn_decode(q, kn, vn, kc, vc, pos, rd=16, scale=0.3)
    o2, _ = orc.attn_decode(q, kn, vn, kc, vc, pos, gate=np.zeros_like(gate), rd=16, scale=0.3)
    _close(o2, 0.5 * o1, 1e-15, "gate 0")
    # cached key t* = q (rd = 0: no rotation), huge scale: softmax picks t*
    kc2 = kc.copy()
    kc2[:, :, 0, :] = np.repeat(q[:, ::grp], 1, axis=1) * 4
    o, _ = orc.attn_decode(q[:, ::grp], kn, vn, kc2, vc, pos, rd=0, scale=50.0)
    _close(o, vc[:, :, 0, :].astype(np.float64), 1e-9, "dominant score")


def pin_attn_library(orc):
    """Against torch's CPU softmax and matmul in fp64 on rotated inputs
    (the rotary embedding pinned above), with GQA by repeated heads."""
    import torch
    q, gate, kn, vn, kc, vc, pos = _attn_case(43, N=3, Hq=8, Hkv=2, d=32, Lmax=50)
    rd, th, sc = 16, 1e7, 32 ** -0.5
    o, kr = orc.attn_decode(q, kn, vn, kc, vc, pos, gate=gate, rd=rd, theta=th, scale=sc)
    N, Hq, d = q.shape
    grp = Hq // kn.shape[1]
    qr = orc.rope(q, np.repeat(pos[:, None], Hq, axis=1), rd=rd, theta=th)
    krw = orc.rope(kn, np.repeat(pos[:, None], kn.shape[1], axis=1), rd=rd, theta=th)
    _close(kr, krw, 0.0, "appended key")
    for n in range(N):
        K = np.concatenate([kc[n, :, :pos[n]].astype(np.float64), krw[n][:, None]], axis=1)
        V = np.concatenate([vc[n, :, :pos[n]], vn[n, :, None]], axis=1).astype(np.float64)
        K, V = np.repeat(K, grp, axis=0), np.repeat(V, grp, axis=0)
        s = torch.from_numpy(np.einsum("hd,htd->ht", qr[n], K) * sc)
        w = torch.softmax(s, dim=-1).numpy()
        want = np.einsum("ht,htd->hd", w, V) * torch.sigmoid(torch.from_numpy(gate[n].astype(np.float64))).numpy()
        _close(o[n], want, 1e-13, f"sequence {n}")


def pin_attn_gqa(orc):
    """Query head h reads key/value head h / (Hq / Hkv): equal to repeated heads."""
    q, gate, kn, vn, kc, vc, pos = _attn_case(44, N=2, Hq=6, Hkv=3, d=16, Lmax=20)
    o1, _ = orc.attn_decode(q, kn, vn, kc, vc, pos, gate=gate, rd=8)
    rep = lambda a: np.repeat(a, 2, axis=1)
    o2, _ = orc.attn_decode(q, rep(kn), rep(vn), rep(kc), rep(vc), pos, gate=gate, rd=8)
    assert np.array_equal(o1, o2), "GQA vs repeated heads"


RECURRENCE_PINS = [
    pin_handworked_two_tokens, pin_single_token_closed_form, pin_decay_only,
    pin_exact_retrieval, pin_linear_readout, pin_delta_rule_invariants, pin_scale_linearity,
    pin_grouped_value_heads, pin_packed_isolation, pin_contraction_bound,
    pin_chunked_equals_step, pin_transition_product,
]
NORM_PINS = [pin_norm_library, pin_norm_closed_forms]
LAYER_PINS = [pin_gate_closed_forms, pin_gate_library, pin_l2norm,
              pin_decode_layer_reduces_to_step, pin_decode_layer_l2norm, pin_decode_layer_gates]
ATTN_PINS = [pin_rope_closed_forms, pin_rope_relative, pin_attn_closed_forms, pin_attn_library,
             pin_attn_gqa]
ALL_PINS = RECURRENCE_PINS + NORM_PINS + LAYER_PINS + ATTN_PINS
