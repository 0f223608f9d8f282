"""Pins that tie the CPU oracle to what the pages and mathematics fix.

Each pin takes an oracle instance (the real one, or one compiled with a planted mistake)
and raises AssertionError when the oracle disagrees with something that does not come from
the oracle itself: a hand-computed example, a closed form, an invariant of the recurrence,
an explicit dense-matrix form, or the independent chunked derivation in chunked_ref.py.

Sources, by page title and section:
  "Kimi K3: Architecture, Training, and Million-Token Agentic RL" (the K3 note):
     §3.1 full recurrence S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, o = S^T q;
          Diag(alpha) scales rows (key channels)
     §3.2 edit/read order; read after the update
     §3.3 lower-bounded gate g = g_min Sigmoid(e^A z), g_min = -5; 16-token tile bound
          (-80, 0); chunked and recurrent forms compute the same update
"""
from __future__ import annotations

import math
import os

import numpy as np

from tests.chunked_ref import chunked_pair

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rand_pair(rng, L, dk, dv, g_lo=-5.0, g_hi=0.0, with_s0=True):
    q = rng.standard_normal((L, 1, dk)).astype(np.float32)
    k = rng.standard_normal((L, 1, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, 1, dv)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (L, 1)).astype(np.float32)
    g = rng.uniform(g_lo, g_hi, (L, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32) if with_s0 else None
    return q, k, v, beta, g, S0


# --- gate ([K3 note] §3.3) --------------------------------------------------------------

def pin_gate_midpoint(orc):
    """Sigmoid(0) = 1/2, so z = 0 gives g = g_min / 2 = -2.5 exactly, for any A."""
    rng = np.random.default_rng(10)
    A = rng.normal(0, 0.5, (3, 8)).astype(np.float32)
    z = np.zeros((5, 3, 8), np.float32)
    g = orc.gate(z, A)
    assert np.all(g == -2.5), f"g(z=0) = {np.unique(g)}"


def pin_gate_saturation(orc):
    """Sigmoid saturates: g -> g_min = -5 for large positive e^A z, -> 0 for large negative;
    no NaN at the extremes; range [-5, 0]."""
    A = np.zeros((1, 4), np.float32)
    z = np.array([[[1e4, -1e4, 50.0, -50.0]]], np.float32)
    g = orc.gate(z, A)[0, 0]
    assert g[0] == -5.0 and g[2] == -5.0, f"upper saturation {g}"
    assert g[1] == 0.0 and abs(g[3]) < 1e-20, f"lower saturation {g}"
    rng = np.random.default_rng(11)
    zz = rng.normal(0, 30, (64, 2, 16)).astype(np.float32)
    AA = rng.normal(0, 0.5, (2, 16)).astype(np.float32)
    gg = orc.gate(zz, AA)
    assert np.all(np.isfinite(gg)) and gg.min() >= -5.0 and gg.max() <= 0.0


def pin_gate_known_values(orc):
    """Sigmoid(ln 3) = 3/4 and Sigmoid(-ln 3) = 1/4, so with A = 0 (e^A = 1):
    g(ln 3) = -3.75 and g(-ln 3) = -1.25 (up to the fp32 rounding of z)."""
    A = np.zeros((1, 2), np.float32)
    z = np.array([[[math.log(3.0), -math.log(3.0)]]], np.float32)
    g = orc.gate(z, A)[0, 0]
    _close(g, [-3.75, -1.25], 1e-6, "g(+-ln3)")
    # e^A enters multiplicatively: A = ln 2 halves the z needed for the same g.
    A2 = np.full((1, 2), math.log(2.0), np.float32)
    z2 = np.array([[[math.log(3.0) / 2.0, -math.log(3.0) / 2.0]]], np.float32)
    _close(orc.gate(z2, A2)[0, 0], [-3.75, -1.25], 2e-6, "g with e^A = 2")


def pin_gate_symmetry_monotone(orc):
    """Sigmoid(x) + Sigmoid(-x) = 1 gives g(z) + g(-z) = -5; g decreases in z."""
    rng = np.random.default_rng(12)
    A = rng.normal(0, 0.5, (2, 16)).astype(np.float32)
    z = rng.normal(0, 2, (32, 2, 16)).astype(np.float32)
    _close(orc.gate(z, A) + orc.gate(-z, A), np.full(z.shape, -5.0), 1e-12, "g(z)+g(-z)")
    zs = np.sort(z, axis=0)
    gs = orc.gate(zs, A)
    assert np.all(np.diff(gs, axis=0) <= 0.0), "g not monotone decreasing in z"


# --- chunk-local cumulative log-decay -------------------------------------------------------

def pin_chunk_cumsum(orc):
    """Inclusive, restarting every 64 tokens from each sequence start (varlen aware)."""
    lens = [70, 10, 0, 5, 128]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = -np.ones((cu[-1], 1, 3))
    G = orc.chunk_cumsum(g, cu, chunk=64)
    exp = []
    for L in lens:
        exp += [-(p % 64 + 1) for p in range(L)]
    _close(G[:, 0, 0], exp, 0.0, "chunk cumsum")
    G1 = orc.chunk_cumsum(g[:100], None, chunk=16)
    _close(G1[:, 0, 1], [-(p % 16 + 1) for p in range(100)], 0.0, "chunk cumsum, one seq")


# --- worked examples ([K3 note] §3.1-§3.2) -----------------------------------------------

def _read_rows(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def pin_golden_scalar(orc):
    rows = _read_rows(os.path.join(GOLDEN, "scalar_worked_example.txt"))
    v = np.array([[[float(r[1])]] for r in rows], np.float32)
    L = len(rows)
    one = np.ones((L, 1, 1), np.float32)
    g = np.full((L, 1, 1), -math.log(2.0))
    o, S = orc.prefill(one, one, v, np.full((L, 1), 0.5, np.float32), g=g)
    _close(o[:, 0, 0], [float(r[2]) for r in rows], 1e-14, "scalar example o")
    _close(S[0, 0, 0, 0], float(rows[-1][3]), 1e-14, "scalar example S")


def pin_golden_two_channel(orc):
    rows = _read_rows(os.path.join(GOLDEN, "channel_decay_worked_example.txt"))
    toks = [r for r in rows if r[0] != "S"]
    Sexp = [float(x) for x in [r for r in rows if r[0] == "S"][0][1:]]
    f = lambda i, j: np.array([[[float(r[i]), float(r[j])]] for r in toks], np.float32)
    alpha = np.array([[[float(r[1]), float(r[2])]] for r in toks])
    g = np.log(alpha)
    k, q = f(3, 4), f(5, 6)
    v = np.array([[[float(r[7])]] for r in toks], np.float32)
    beta = np.array([[float(r[8])] for r in toks], np.float32)
    o, S = orc.prefill(q, k, v, beta, g=g)
    _close(o[:, 0, 0], [float(r[9]) for r in toks], 1e-14, "two-channel example o")
    _close(S[0, 0, :, 0], Sexp, 1e-14, "two-channel example S")


# --- brute force: the dense matrix form of [K3 note] §3.1 ---------------------------------

def pin_brute_force_matrix_form(orc):
    rng = np.random.default_rng(13)
    for L, dk, dv in [(8, 4, 4), (6, 3, 3), (7, 4, 4)]:
        q, k, v, beta, g, S0 = _rand_pair(rng, L, dk, dv)
        o, S = orc.prefill(q, k, v, beta, g=g, S0=S0)
        St = S0[0, 0].astype(np.float64)
        for t in range(L):
            kt = k[t, 0].astype(np.float64)
            M = (np.eye(dk) - beta[t, 0] * np.outer(kt, kt)) @ np.diag(np.exp(g[t, 0]))
            St = M @ St + beta[t, 0] * np.outer(kt, v[t, 0].astype(np.float64))
            _close(o[t, 0], St.T @ q[t, 0].astype(np.float64), 1e-13, f"brute o[{t}]")
        _close(S[0, 0], St, 1e-13, "brute S")


def pin_gate_in_recurrence(orc):
    """The recurrence driven by (z, A) equals the recurrence driven by the gate's g."""
    rng = np.random.default_rng(14)
    q, k, v, beta, _, S0 = _rand_pair(rng, 40, 8, 8)
    z = rng.normal(0, 1, (40, 1, 8)).astype(np.float32)
    A = rng.normal(0, 0.5, (1, 8)).astype(np.float32)
    o1, S1 = orc.prefill(q, k, v, beta, z=z, A=A, S0=S0)
    o2, S2 = orc.prefill(q, k, v, beta, g=orc.gate(z, A), S0=S0)
    _close(o1, o2, 0.0, "gate inside vs outside, o")
    _close(S1, S2, 0.0, "gate inside vs outside, S")


# --- invariants -------------------------------------------------------------------------

def pin_zero_beta_zero_state(orc):
    """beta = 0 and S0 = 0: no write ever happens, so o = 0 and S = 0."""
    rng = np.random.default_rng(15)
    q, k, v, _, g, _ = _rand_pair(rng, 50, 8, 8, with_s0=False)
    o, S = orc.prefill(q, k, v, np.zeros((50, 1), np.float32), g=g)
    assert np.all(o == 0.0) and np.all(S == 0.0)


def pin_unit_edit_reads_back_value(orc):
    """beta ||k||^2 = 1 and q = k: o = Sbar^T k + (v - Sbar^T k) k^T k beta = v, whatever the
    history and decay (read after the write, erase coupled to the write by beta)."""
    rng = np.random.default_rng(16)
    L, d = 30, 8
    q, k, v, _, g, S0 = _rand_pair(rng, L, d, d)
    k = rng.standard_normal((L, 1, d)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = (1.0 / np.sum(k.astype(np.float64) ** 2, axis=-1)).astype(np.float32)
    kk = k.astype(np.float64)
    # beta in fp32 is only ~1/||k||^2; fold the tiny residual into the expected value.
    o, _ = orc.prefill(k, k, v, beta, g=g, S0=S0)
    resid = np.abs(beta.astype(np.float64) * np.sum(kk * kk, axis=-1) - 1.0).max()
    _close(o, v, 50.0 * (resid + 1e-14), "o = v under unit edits")


def pin_no_write_pure_decay(orc):
    """k = 0: the state only decays, S_t = Diag(e^{Gamma_t}) S0 with Gamma_t the inclusive
    sequence-global sum of g, so o_t = S0^T (e^{Gamma_t} * q_t) (rows decayed, not columns)."""
    rng = np.random.default_rng(17)
    L, dk, dv = 20, 6, 5
    q, _, v, beta, g, S0 = _rand_pair(rng, L, dk, dv, g_lo=-0.5)
    k = np.zeros((L, 1, dk), np.float32)
    o, S = orc.prefill(q, k, v, beta, g=g, S0=S0)
    Gam = np.cumsum(g[:, 0, :], axis=0)
    S0d = S0[0, 0].astype(np.float64)
    exp_o = np.stack([S0d.T @ (np.exp(Gam[t]) * q[t, 0]) for t in range(L)])
    _close(o[:, 0], exp_o, 1e-14, "pure decay o")
    _close(S[0, 0], np.exp(Gam[-1])[:, None] * S0d, 1e-14, "pure decay S")


def pin_one_hot_keys(orc):
    """One-hot keys k_t = e_{c_t}: rows decouple into scalar exponential moving averages,
    row c_t <- (1 - beta) alpha_{c_t} row + beta v, every other row <- alpha_c row."""
    rng = np.random.default_rng(18)
    L, d = 40, 4
    c = rng.integers(0, d, L)
    k = np.zeros((L, 1, d), np.float32)
    k[np.arange(L), 0, c] = 1.0
    q = rng.standard_normal((L, 1, d)).astype(np.float32)
    v = rng.standard_normal((L, 1, d)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (L, 1)).astype(np.float32)
    g = rng.uniform(-1.0, 0.0, (L, 1, d))
    S0 = rng.standard_normal((1, 1, d, d)).astype(np.float32)
    o, S = orc.prefill(q, k, v, beta, g=g, S0=S0)
    St = S0[0, 0].astype(np.float64)
    for t in range(L):
        a = np.exp(g[t, 0])
        St = a[:, None] * St
        b = float(beta[t, 0])
        St[c[t]] = (1.0 - b) * St[c[t]] + b * v[t, 0].astype(np.float64)
        _close(o[t, 0], St.T @ q[t, 0], 1e-13, f"one-hot o[{t}]")
    _close(S[0, 0], St, 1e-13, "one-hot S")


# --- chunked == recurrent ([K3 note] §3.3) ------------------------------------------------

def pin_chunked_equals_recurrent(orc):
    rng = np.random.default_rng(19)
    for L, dk, dv, C in [(130, 16, 16, 16), (200, 16, 12, 32), (256, 8, 8, 64), (77, 8, 8, 64)]:
        q, k, v, beta, g, S0 = _rand_pair(rng, L, dk, dv)
        o, S = orc.prefill(q, k, v, beta, g=g, S0=S0)
        oc, Sc = chunked_pair(q[:, 0], k[:, 0], v[:, 0], beta[:, 0], g[:, 0], S0[0, 0], C)
        scale = max(1.0, float(np.abs(oc).max()))
        _close(o[:, 0] / scale, oc / scale, 1e-11, f"chunked C={C} o")
        _close(S[0, 0], Sc, 1e-11 * max(1.0, float(np.abs(Sc).max())), f"chunked C={C} S")


# --- state I/O, varlen, decode -----------------------------------------------------------

def pin_split_resume(orc):
    """prefill(x[:m]) -> S_m; prefill(x[m:], S0 = S_m) continues exactly (up to the fp32
    hand-over of the state, the form in which states cross the boundary)."""
    rng = np.random.default_rng(20)
    L, d, m = 90, 8, 37
    q, k, v, beta, g, S0 = _rand_pair(rng, L, d, d)
    o, S = orc.prefill(q, k, v, beta, g=g, S0=S0)
    o1, S1 = orc.prefill(q[:m], k[:m], v[:m], beta[:m], g=g[:m], S0=S0)
    o2, S2 = orc.prefill(q[m:], k[m:], v[m:], beta[m:], g=g[m:],
                         S0=S1.astype(np.float32))
    _close(o1, o[:m], 0.0, "split prefix o")
    tol = 1e-6 * max(1.0, float(np.abs(S).max()))
    _close(o2, o[m:], tol, "resumed o")
    _close(S2, S, tol, "resumed S")


def pin_varlen_equals_per_sequence(orc):
    rng = np.random.default_rng(21)
    lens = [33, 0, 64, 1, 100]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 8
    q = rng.standard_normal((T, H, d)).astype(np.float32)
    k = rng.standard_normal((T, H, d)).astype(np.float32) * 0.3
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    beta = rng.uniform(0, 1, (T, H)).astype(np.float32)
    z = rng.normal(0, 1, (T, H, d)).astype(np.float32)
    A = rng.normal(0, 0.5, (H, d)).astype(np.float32)
    S0 = rng.normal(0, 0.1, (len(lens), H, d, d)).astype(np.float32)
    o, S = orc.prefill(q, k, v, beta, z=z, A=A, S0=S0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        on, Sn = orc.prefill(q[s:e], k[s:e], v[s:e], beta[s:e], z=z[s:e], A=A,
                             S0=S0[n:n + 1])
        _close(o[s:e], on, 0.0, f"varlen seq {n} o")
        _close(S[n], Sn[0], 0.0, f"varlen seq {n} S")
    # a zero-length sequence hands its initial state through unchanged
    _close(S[1], S0[1], 0.0, "empty sequence state")


def pin_decode_equals_prefill(orc):
    """T single-token decode steps reproduce a T-token prefill ([K3 note] §3.3: the
    recurrent and chunked executions realise the same causal update)."""
    rng = np.random.default_rng(22)
    T, N, H, d = 12, 3, 2, 8
    q = rng.standard_normal((T, N, H, d)).astype(np.float32)
    k = (rng.standard_normal((T, N, H, d)) * 0.3).astype(np.float32)
    v = rng.standard_normal((T, N, H, d)).astype(np.float32)
    beta = rng.uniform(0, 1, (T, N, H)).astype(np.float32)
    z = rng.normal(0, 1, (T, N, H, d)).astype(np.float32)
    A = rng.normal(0, 0.5, (H, d)).astype(np.float32)
    S0 = rng.normal(0, 0.1, (N, H, d, d)).astype(np.float32)
    S = S0.astype(np.float64).copy()
    outs = [orc.decode_step(q[t], k[t], v[t], beta[t], z[t], A, S) for t in range(T)]
    pack = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1).reshape(N * T, *x.shape[2:]))
    cu = np.arange(0, N * T + 1, T, dtype=np.int32)
    o, Sp = orc.prefill(pack(q), pack(k), pack(v), pack(beta), z=pack(z), A=A, S0=S0,
                        cu_seqlens=cu)
    _close(np.stack(outs, 1).reshape(N * T, H, d), o, 0.0, "decode vs prefill o")
    _close(S, Sp, 0.0, "decode vs prefill S")


def pin_unit_retention_is_plain_delta_rule(orc):
    """alpha = 1 (g = 0) turns the recurrence of [K3 note] §3.1 into the plain delta rule of
    the same section: predict vhat = S^T k, correct S <- S + beta k (v - vhat)^T, read
    o = S^T q after the correction.  The gate reaches g = 0 exactly: e^A z = -1e4 e^A makes
    Sigmoid underflow to 0.  Checked with and without an initial state, and through both the
    (z, A) and the explicit-g entry of the oracle."""
    rng = np.random.default_rng(24)
    for L, dk, dv, with_s0 in [(24, 6, 5, True), (31, 8, 8, False), (9, 3, 7, True)]:
        q = rng.standard_normal((L, 1, dk)).astype(np.float32)
        k = rng.standard_normal((L, 1, dk)).astype(np.float32)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((L, 1, dv)).astype(np.float32)
        beta = rng.uniform(0.05, 0.95, (L, 1)).astype(np.float32)
        S0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32) if with_s0 else None
        z = np.full((L, 1, dk), -1e4, np.float32)
        A = rng.normal(0, 0.5, (1, dk)).astype(np.float32)
        assert np.all(orc.gate(z, A) == 0.0), "gate at z = -1e4 is not exactly 0"
        # the delta rule, written out on its own
        S = np.zeros((dk, dv)) if S0 is None else S0[0, 0].astype(np.float64)
        o_want = np.empty((L, dv))
        for t in range(L):
            kt = k[t, 0].astype(np.float64)
            vhat = S.T @ kt
            S = S + float(beta[t, 0]) * np.outer(kt, v[t, 0].astype(np.float64) - vhat)
            o_want[t] = S.T @ q[t, 0].astype(np.float64)
        for o, Sg in (orc.prefill(q, k, v, beta, z=z, A=A, S0=S0),
                      orc.prefill(q, k, v, beta, g=np.zeros((L, 1, dk)), S0=S0)):
            _close(o[:, 0], o_want, 1e-13, f"delta rule o (L={L})")
            _close(Sg[0, 0], S, 1e-13, f"delta rule S (L={L})")


def pin_linearity(orc):
    """o and S are jointly linear in (S0, v): scaling both by 2 scales o and S by 2."""
    rng = np.random.default_rng(23)
    q, k, v, beta, g, S0 = _rand_pair(rng, 50, 8, 8)
    o, S = orc.prefill(q, k, v, beta, g=g, S0=S0)
    o2, S2 = orc.prefill(q, k, 2 * v, beta, g=g, S0=2 * S0)
    _close(o2, 2 * o, 0.0, "linearity o")
    _close(S2, 2 * S, 0.0, "linearity S")


ALL_PINS = [
    pin_gate_midpoint, pin_gate_saturation, pin_gate_known_values, pin_gate_symmetry_monotone,
    pin_chunk_cumsum, pin_golden_scalar, pin_golden_two_channel, pin_brute_force_matrix_form,
    pin_gate_in_recurrence, pin_zero_beta_zero_state, pin_unit_edit_reads_back_value,
    pin_no_write_pure_decay, pin_one_hot_keys, pin_chunked_equals_recurrent, pin_split_resume,
    pin_varlen_equals_per_sequence, pin_decode_equals_prefill, pin_linearity,
    pin_unit_retention_is_plain_delta_rule,
]


def failing_pins(orc):
    bad = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:  # noqa: PERF203
            bad.append((pin.__name__, str(e)))
    return bad
