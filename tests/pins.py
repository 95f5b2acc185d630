"""Checks that pin the fp64 oracle to facts fixed outside the oracle itself.

Each ``check_*`` takes a loaded oracle library (so the mutation test can run
the same checks against deliberately broken builds) and raises
AssertionError on a mismatch.  The facts come from the pages and from the
algebra of the recurrence of the page "Kimi Delta Attention" (§03):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t                          (§02 read-out, after the update)

S is dk x dv here (math orientation); the oracle stores S^T.
"""
from __future__ import annotations

import json
import math
import os
import random
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    return float(np.max(np.abs(a - b)) / scale) if a.size else 0.0


def _run(lib, q, k, v, la, beta, cu, s0=None, **kw):
    return oracle.prefill(q, k, v, la, beta, np.asarray(cu, dtype=np.int64), s0, lib=lib, **kw)


def _rand_inputs(rng, T, H, dk, dv, unit_k=True, la_lo=-1.0):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = rng.uniform(la_lo, 0.0, (T, H, dk))
    beta = rng.uniform(0.0, 1.0, (T, H))
    return q, k, v, la, beta


# --------------------------------------------------------------------------
# 1. Exact rational brute force of the literal matrix recurrence (§03)
# --------------------------------------------------------------------------
def _brute_force_exact(alpha, beta, k, v, q, S0):
    """Literal (I - b k k^T) Diag(a) S + b k v^T in exact rationals.

    alpha, k, q: lists [T][dk]; v: [T][dv]; beta: [T]; S0: [dk][dv].
    Returns (outputs [T][dv], final S [dk][dv]).
    """
    T, dk, dv = len(alpha), len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        # M = (I - beta k k^T) Diag(alpha), built element by element
        M = [[((1 if i == c else 0) - beta[t] * k[t][i] * k[t][c]) * alpha[t][c]
              for c in range(dk)] for i in range(dk)]
        S = [[sum(M[i][c] * S[c][j] for c in range(dk)) + beta[t] * k[t][i] * v[t][j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(dk)) for j in range(dv)])
    return outs, S


def check_exact_bruteforce(lib, seed=7):
    rnd = random.Random(seed)
    for dk, dv, T in ((3, 4, 6), (4, 2, 5), (2, 3, 4)):
        fr = lambda lo, hi, den: Fraction(rnd.randint(lo, hi), den)
        alpha = [[fr(1, 9, 10) for _ in range(dk)] for _ in range(T)]
        beta = [fr(0, 8, 8) for _ in range(T)]
        k = [[fr(-4, 4, 8) for _ in range(dk)] for _ in range(T)]
        q = [[fr(-4, 4, 4) for _ in range(dk)] for _ in range(T)]
        v = [[fr(-6, 6, 3) for _ in range(dv)] for _ in range(T)]
        S0 = [[fr(-5, 5, 5) for _ in range(dv)] for _ in range(dk)]
        outs, S = _brute_force_exact(alpha, beta, k, v, q, S0)

        f = lambda M: np.array([[float(x) for x in row] for row in M])
        la = np.log(f(alpha))[:, None, :]
        s0 = f(S0).T[None, None]                     # stored as S^T
        o, fin = _run(lib, f(q)[:, None, :], f(k)[:, None, :], f(v)[:, None, :], la,
                      np.array([float(b) for b in beta])[:, None], [0, T], s0)
        exp_o = f(outs)
        exp_S = f(S).T
        assert _rel(o[:, 0, :], exp_o) < 1e-12, ("outputs vs exact brute force", dk, dv)
        assert _rel(fin[0, 0], exp_S) < 1e-12, ("final state vs exact brute force", dk, dv)


# --------------------------------------------------------------------------
# 2. Hand-worked two-token example (tests/golden)
# --------------------------------------------------------------------------
def check_golden_worked_example(lib):
    path = os.path.join(GOLDEN, "kda_two_token_worked_example.json")
    with open(path) as fh:
        G = json.load(fh)
    F = lambda x: float(Fraction(x))
    arr = lambda M: np.array([[F(x) for x in row] for row in M])
    alpha, k, v, q = arr(G["alpha"]), arr(G["k"]), arr(G["v"]), arr(G["q"])
    beta = np.array([F(b) for b in G["beta"]])
    S0 = arr(G["S0"])                  # dk x dv
    T = alpha.shape[0]
    o, fin = _run(lib, q[:, None], k[:, None], v[:, None], np.log(alpha)[:, None],
                  beta[:, None], [0, T], S0.T[None, None])
    for t, step in enumerate(G["steps"]):
        assert _rel(o[t, 0], np.array([F(x) for x in step["o"]])) < 1e-14, ("golden o", t)
    assert _rel(fin[0, 0], arr(G["steps"][-1]["S"]).T) < 1e-14, "golden final state"


# --------------------------------------------------------------------------
# 3. Special cases named by the recurrence and the pages
# --------------------------------------------------------------------------
def check_identity_no_write(lib, seed=1):
    """alpha == 1 and beta == 0: the state never changes; o_t = S0^T q_t."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 37, 2, 8, 5
    q, k, v, _, _ = _rand_inputs(rng, T, H, dk, dv)
    la = np.zeros((T, H, dk))
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((1, H, dv, dk))
    o, fin = _run(lib, q, k, v, la, beta, [0, T], s0)
    assert np.array_equal(fin, s0), "state must be bit-identical"
    exp_o = np.einsum("hji,thi->thj", s0[0], q)
    assert _rel(o, exp_o) < 1e-13


def check_deltanet(lib, seed=2):
    """alpha == 1 reduces KDA to the delta rule of §02:
    S_t = S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 29, 2, 6, 7
    q, k, v, _, beta = _rand_inputs(rng, T, H, dk, dv)
    la = np.zeros((T, H, dk))
    S = rng.standard_normal((H, dk, dv))
    s0 = np.transpose(S, (0, 2, 1))[None].copy()
    o, fin = _run(lib, q, k, v, la, beta, [0, T], s0)
    exp_o = np.zeros((T, H, dv))
    for t in range(T):
        for h in range(H):
            err = v[t, h] - S[h].T @ k[t, h]
            S[h] = S[h] + beta[t, h] * np.outer(k[t, h], err)
            exp_o[t, h] = S[h].T @ q[t, h]
    assert _rel(o, exp_o) < 1e-12
    assert _rel(fin[0], np.transpose(S, (0, 2, 1))) < 1e-12


def check_readback(lib, seed=3):
    """beta = 1 and a unit key: after the update the memory returns exactly
    v_t at k_t (§02: read, take the error, correct), whatever the decay.
    With q := k the read-out is therefore v_t."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 41, 3, 16, 9
    _, k, v, la, _ = _rand_inputs(rng, T, H, dk, dv, la_lo=-3.0)
    beta = np.ones((T, H))
    s0 = rng.standard_normal((1, H, dv, dk))
    o, _ = _run(lib, k, k, v, la, beta, [0, T], s0)
    assert _rel(o, v) < 1e-12


def _closed_form_additive(la, k, v, beta, q, S0):
    """Erase removed: S_t = Diag(G_t) S0 + sum_{i<=t} Diag(G_t / G_i) beta_i k_i v_i^T,
    G_t = prod_{s<=t} alpha_s (per key channel).  S0: [dk][dv]."""
    T = la.shape[0]
    cum = np.cumsum(la, axis=0)                       # log G_t
    outs = np.zeros((T, v.shape[1]))
    S = None
    for t in range(T):
        S = np.exp(cum[t])[:, None] * S0
        for i in range(t + 1):
            S = S + beta[i] * np.outer(np.exp(cum[t] - cum[i]) * k[i], v[i])
        outs[t] = S.T @ q[t]
    return outs, S


def check_additive_closed_form(lib, seed=4):
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 23, 2, 5, 6
    q, k, v, la, beta = _rand_inputs(rng, T, H, dk, dv, unit_k=False)
    s0 = rng.standard_normal((1, H, dv, dk))
    o, fin = _run(lib, q, k, v, la, beta, [0, T], s0, mode=oracle.MODE_ERASE_OFF)
    for h in range(H):
        eo, eS = _closed_form_additive(la[:, h], k[:, h], v[:, h], beta[:, h], q[:, h], s0[0, h].T)
        assert _rel(o[:, h], eo) < 1e-11, ("additive closed form o", h)
        assert _rel(fin[0, h], eS.T) < 1e-11, ("additive closed form S", h)
    # alpha == 1, beta == 1, S0 == 0: plain linear attention, S_T = sum k_i v_i^T
    la0 = np.zeros_like(la)
    o, fin = _run(lib, q, k, v, la0, np.ones((T, H)), [0, T], None, mode=oracle.MODE_ERASE_OFF)
    for h in range(H):
        assert _rel(fin[0, h], (k[:, h].T @ v[:, h]).T) < 1e-12


def check_pure_decay(lib, seed=5):
    """beta == 0: S_t = Diag(G_t) S0 and o_t = S0^T (G_t * q_t)."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 31, 2, 7, 4
    q, k, v, la, _ = _rand_inputs(rng, T, H, dk, dv, la_lo=-0.5)
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((1, H, dv, dk))
    o, fin = _run(lib, q, k, v, la, beta, [0, T], s0)
    G = np.exp(np.cumsum(la, axis=0))                 # [T,H,dk]
    exp_o = np.einsum("hji,thi->thj", s0[0], G * q)
    assert _rel(o, exp_o) < 1e-12
    assert _rel(fin[0], s0[0] * G[-1][:, None, :]) < 1e-12


def check_dictionary(lib, seed=6):
    """Basis keys, beta = 1, alpha = 1: a targeted overwrite (§02).  Reading at
    e_i returns the last value written at key i (zero if none); integer values
    make the result exact."""
    rnd = random.Random(seed)
    T, dk, dv = 24, 5, 3
    pi = [rnd.randrange(dk) for _ in range(T)]
    sigma = [rnd.randrange(dk) for _ in range(T)]
    k = np.zeros((T, 1, dk)); q = np.zeros((T, 1, dk))
    for t in range(T):
        k[t, 0, pi[t]] = 1.0
        q[t, 0, sigma[t]] = 1.0
    v = np.array([[rnd.randint(-9, 9) for _ in range(dv)] for _ in range(T)], dtype=np.float64)[:, None]
    o, _ = _run(lib, q, k, v, np.zeros((T, 1, dk)), np.ones((T, 1)), [0, T], None)
    for t in range(T):
        last = [s for s in range(t + 1) if pi[s] == sigma[t]]
        expect = v[last[-1], 0] if last else np.zeros(dv)
        assert np.array_equal(o[t, 0], expect), ("dictionary read", t)


def check_linearity(lib, seed=8):
    """For fixed q, k, alpha, beta the map (V, S0) -> (o, S_T) is linear."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 19, 2, 6, 5
    q, k, v1, la, beta = _rand_inputs(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    a = rng.standard_normal((1, H, dv, dk)); b = rng.standard_normal((1, H, dv, dk))
    o1, f1 = _run(lib, q, k, v1, la, beta, [0, T], a)
    o2, f2 = _run(lib, q, k, v2, la, beta, [0, T], b)
    o3, f3 = _run(lib, q, k, v1 - 2.5 * v2, la, beta, [0, T], a - 2.5 * b)
    assert _rel(o3, o1 - 2.5 * o2) < 1e-12
    assert _rel(f3, f1 - 2.5 * f2) < 1e-12


def check_column_permutation(lib, seed=9):
    """Value channels never mix: permuting v and S0 columns permutes o and S_T."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 17, 2, 8, 40
    q, k, v, la, beta = _rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    perm = rng.permutation(dv)
    o, f = _run(lib, q, k, v, la, beta, [0, T], s0)
    op, fp = _run(lib, q, k, v[..., perm], la, beta, [0, T], s0[:, :, perm, :])
    assert np.array_equal(op, o[..., perm])
    assert np.array_equal(fp, f[:, :, perm, :])


def check_continuation_and_packing(lib, seed=10):
    """Prefix checkpoint (§07): continuing from the state after a prefix is
    exact; sequences packed together do not interact."""
    rng = np.random.default_rng(seed)
    H, dk, dv = 2, 6, 5
    lens = [13, 0, 21, 1, 9]
    T = sum(lens)
    q, k, v, la, beta = _rand_inputs(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.standard_normal((len(lens), H, dv, dk))
    o, f = _run(lib, q, k, v, la, beta, cu, s0)
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        oi, fi = _run(lib, q[sl], k[sl], v[sl], la[sl], beta[sl], [0, L], s0[n:n + 1])
        assert np.array_equal(oi, o[sl]) and np.array_equal(fi[0], f[n]), ("packing", n)
        if L >= 2:
            c = L // 2
            sa = slice(cu[n], cu[n] + c)
            sb = slice(cu[n] + c, cu[n + 1])
            oa, fa = _run(lib, q[sa], k[sa], v[sa], la[sa], beta[sa], [0, c], s0[n:n + 1])
            ob, fb = _run(lib, q[sb], k[sb], v[sb], la[sb], beta[sb], [0, L - c], fa)
            assert np.array_equal(np.concatenate([oa, ob]), o[sl]), ("continuation o", n)
            assert np.array_equal(fb[0], f[n]), ("continuation state", n)
    # zero-length sequence: final state is the initial state
    assert np.array_equal(f[1], s0[1])


# --------------------------------------------------------------------------
# 12. Scalar gate (Gated DeltaNet): the literal scalar-gated delta rule
#     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
#     gate applied outside the erase, in exact rationals
# --------------------------------------------------------------------------
def _brute_force_gdn_exact(alpha, beta, k, v, q, S0):
    T, dk, dv = len(alpha), len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        E = [[(1 if i == c else 0) - beta[t] * k[t][i] * k[t][c] for c in range(dk)] for i in range(dk)]
        S = [[alpha[t] * sum(E[i][c] * S[c][j] for c in range(dk)) + beta[t] * k[t][i] * v[t][j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(dk)) for j in range(dv)])
    return outs, S


def check_scalar_gate_exact(lib, seed=13):
    rnd = random.Random(seed)
    for dk, dv, T in ((3, 2, 5), (2, 4, 6)):
        fr = lambda lo, hi, den: Fraction(rnd.randint(lo, hi), den)
        alpha = [fr(1, 9, 10) for _ in range(T)]
        beta = [fr(0, 8, 8) for _ in range(T)]
        k = [[fr(-4, 4, 8) for _ in range(dk)] for _ in range(T)]
        q = [[fr(-4, 4, 4) for _ in range(dk)] for _ in range(T)]
        v = [[fr(-6, 6, 3) for _ in range(dv)] for _ in range(T)]
        S0 = [[fr(-5, 5, 5) for _ in range(dv)] for _ in range(dk)]
        outs, S = _brute_force_gdn_exact(alpha, beta, k, v, q, S0)
        f = lambda M: np.array([[float(x) for x in row] for row in M])
        la = np.log(np.array([float(a) for a in alpha]))[:, None]          # [T, H=1]
        o, fin = oracle.prefill_scalar_gate(f(q)[:, None, :], f(k)[:, None, :], f(v)[:, None, :], la,
                                            np.array([float(b) for b in beta])[:, None],
                                            np.array([0, T], dtype=np.int64), f(S0).T[None, None], lib=lib)
        assert _rel(o[:, 0, :], f(outs)) < 1e-12, ("scalar gate outputs vs exact", dk, dv)
        assert _rel(fin[0, 0], f(S).T) < 1e-12, ("scalar gate state vs exact", dk, dv)


# --------------------------------------------------------------------------
# 13. Raw-input prologue: outputs do not depend on the length of q and k
#     (each is made unit length), and with unit q, k and beta = sigmoid(x)
#     the raw form is the plain recurrence
# --------------------------------------------------------------------------
def check_raw_prologue(lib, seed=14):
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 9, 2, 5, 3
    q, k, v, la, beta = _rand_inputs(rng, T, H, dk, dv)      # unit q, k
    logit = np.log(beta / (1.0 - beta))
    s0 = rng.standard_normal((1, H, dv, dk))
    o_plain, f_plain = _run(lib, q, k, v, la, beta, [0, T], s0)
    scale_q = rng.uniform(0.2, 5.0, (T, H, 1))
    scale_k = rng.uniform(0.2, 5.0, (T, H, 1))
    o_raw, f_raw = oracle.prefill_raw(q * scale_q, k * scale_k, v, la, logit, np.array([0, T]), s0, lib=lib)
    assert _rel(o_raw, o_plain) < 1e-12 and _rel(f_raw, f_plain) < 1e-12, "raw prologue"
    # a zero vector stays zero (the 1e-12 floor), which makes that token's write vanish
    kz = k.copy()
    kz[3] = 0.0
    o_z, _ = oracle.prefill_raw(q, kz, v, la, logit, np.array([0, T]), s0, lib=lib)
    o_ref, _ = _run(lib, q, kz, v, la, beta, [0, T], s0)
    assert _rel(o_z, o_ref) < 1e-12, "zero key"


ALL_CHECKS = [
    check_exact_bruteforce,
    check_golden_worked_example,
    check_identity_no_write,
    check_deltanet,
    check_readback,
    check_additive_closed_form,
    check_pure_decay,
    check_dictionary,
    check_linearity,
    check_column_permutation,
    check_continuation_and_packing,
    check_scalar_gate_exact,
    check_raw_prologue,
]
