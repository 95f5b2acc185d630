"""Checks that pin the fp64 gradient oracle (``oracle.prefill_grad``) to facts
fixed outside it.

The pages write no gradient out; what fixes it is the forward map itself
(the recurrence of the page "Kimi Delta Attention", §03, read out as in §02)
and the definition of a derivative:

* central finite differences of the (separately pinned) forward oracle,
  element by element, on small varlen cases that include an empty sequence
  and a sequence longer than the oracle's 64-token recompute segment;
* exact forward-mode differentiation (dual numbers over Fractions) of the
  literal matrix recurrence (I - b k k^T) Diag(a) S + b k v^T, along rational
  directions -- independent of both the rank-1 form and reverse mode;
* the closed form at beta = 0, where the state only decays.

Each ``check_*`` takes a loaded oracle library (the mutation test runs them on
deliberately broken builds) and raises AssertionError on a mismatch.  The
loss is L = sum(d_o * o) + sum(d_final * final_state).
"""
from __future__ import annotations

import random
from fractions import Fraction

import numpy as np

import oracle
from tests.pins import _rand_inputs, _rel

NAMES = ("q", "k", "v", "log_alpha", "beta", "init_state")


def _loss(lib, x, cu, d_o, d_final):
    o, fin = oracle.prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], np.asarray(cu, dtype=np.int64),
                            x["init_state"], lib=lib, nthreads=1)
    return float(np.sum(o * d_o) + np.sum(fin * d_final))


def _case(seed, lengths, H, dk, dv):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q, k, v, la, beta = _rand_inputs(rng, T, H, dk, dv, la_lo=-0.5)
    N = len(lengths)
    x = {"q": q, "k": k, "v": v, "log_alpha": la, "beta": beta,
         "init_state": 0.5 * rng.standard_normal((N, H, dv, dk))}
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    d_o = rng.standard_normal((T, H, dv))
    d_final = rng.standard_normal((N, H, dv, dk))
    return x, cu, d_o, d_final


def check_grad_finite_differences(lib, seed=21):
    """every gradient entry against a central difference of the forward oracle"""
    eps = 1e-6
    for lengths, H, dk, dv in (([0, 3, 70], 1, 2, 3), ([5, 4], 2, 3, 2)):
        x, cu, d_o, d_final = _case(seed, lengths, H, dk, dv)
        g = oracle.prefill_grad(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], cu, x["init_state"], d_o,
                                d_final, lib=lib, nthreads=2)
        for name in NAMES:
            fd = np.zeros_like(x[name])
            for idx in np.ndindex(x[name].shape):
                y = dict(x)
                y[name] = x[name].copy()
                y[name][idx] += eps
                lp = _loss(lib, y, cu, d_o, d_final)
                y[name][idx] -= 2 * eps
                lm = _loss(lib, y, cu, d_o, d_final)
                fd[idx] = (lp - lm) / (2 * eps)
            assert _rel(g[name], fd) < 1e-7, ("finite differences", name, lengths)


# --------------------------------------------------------------------------
# exact forward mode on the literal matrix recurrence
# --------------------------------------------------------------------------
class _Dual:
    """a + b eps with eps^2 = 0, over Fractions"""

    __slots__ = ("a", "b")

    def __init__(self, a, b=0):
        self.a, self.b = Fraction(a), Fraction(b)

    def __add__(self, o):
        o = o if isinstance(o, _Dual) else _Dual(o)
        return _Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __sub__(self, o):
        o = o if isinstance(o, _Dual) else _Dual(o)
        return _Dual(self.a - o.a, self.b - o.b)

    def __rsub__(self, o):
        return _Dual(o) - self

    def __mul__(self, o):
        o = o if isinstance(o, _Dual) else _Dual(o)
        return _Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__


def _literal_loss_dual(alpha, beta, k, v, q, S0, d_o, d_final):
    """L of the literal (I - b k k^T) Diag(a) S + b k v^T recurrence, o = S^T q,
    on dual numbers (S is dk x dv)."""
    T, dk, dv = len(alpha), len(S0), len(S0[0])
    S = [row[:] for row in S0]
    L = _Dual(0)
    for t in range(T):
        M = [[((1 if i == c else 0) - beta[t] * k[t][i] * k[t][c]) * alpha[t][c] for c in range(dk)]
             for i in range(dk)]
        S = [[sum((M[i][c] * S[c][j] for c in range(dk)), _Dual(0)) + beta[t] * k[t][i] * v[t][j]
              for j in range(dv)] for i in range(dk)]
        for j in range(dv):
            o = sum((S[i][j] * q[t][i] for i in range(dk)), _Dual(0))
            L = L + o * d_o[t][j]
    for i in range(dk):
        for j in range(dv):
            L = L + S[i][j] * d_final[i][j]
    return L


def check_grad_exact_directional(lib, seed=22):
    """sum(grad * direction) equals the exact derivative of the literal
    recurrence along that direction, for each input separately"""
    rnd = random.Random(seed)
    fr = lambda lo, hi, den: Fraction(rnd.randint(lo, hi), den)
    f = lambda M: np.array([[float(x) for x in row] for row in M])
    for dk, dv, T in ((2, 3, 4), (3, 2, 3)):
        alpha = [[fr(2, 9, 10) for _ in range(dk)] for _ in range(T)]
        beta = [fr(1, 8, 8) for _ in range(T)]
        k = [[fr(-4, 4, 8) for _ in range(dk)] for _ in range(T)]
        q = [[fr(-4, 4, 4) for _ in range(dk)] for _ in range(T)]
        v = [[fr(-6, 6, 3) for _ in range(dv)] for _ in range(T)]
        S0 = [[fr(-5, 5, 5) for _ in range(dv)] for _ in range(dk)]
        d_o = [[fr(-3, 3, 2) for _ in range(dv)] for _ in range(T)]
        d_final = [[fr(-3, 3, 2) for _ in range(dv)] for _ in range(dk)]
        g = oracle.prefill_grad(f(q)[:, None, :], f(k)[:, None, :], f(v)[:, None, :],
                                np.log(f(alpha))[:, None, :], np.array([float(b) for b in beta])[:, None],
                                [0, T], f(S0).T[None, None], f(d_o)[:, None, :], f(d_final).T[None, None],
                                lib=lib, nthreads=1)
        D = lambda rows, cols: [[fr(-5, 5, 4) for _ in range(cols)] for _ in range(rows)]
        plain = lambda M: [[_Dual(x) for x in row] for row in M]
        for name in NAMES:
            args = {"alpha": plain(alpha), "beta": [_Dual(b) for b in beta], "k": plain(k), "v": plain(v),
                    "q": plain(q), "S0": plain(S0)}
            if name == "q":
                d = D(T, dk)
                args["q"] = [[_Dual(q[t][i], d[t][i]) for i in range(dk)] for t in range(T)]
                got = float(np.sum(g["q"][:, 0, :] * f(d)))
            elif name == "k":
                d = D(T, dk)
                args["k"] = [[_Dual(k[t][i], d[t][i]) for i in range(dk)] for t in range(T)]
                got = float(np.sum(g["k"][:, 0, :] * f(d)))
            elif name == "v":
                d = D(T, dv)
                args["v"] = [[_Dual(v[t][j], d[t][j]) for j in range(dv)] for t in range(T)]
                got = float(np.sum(g["v"][:, 0, :] * f(d)))
            elif name == "log_alpha":
                d = D(T, dk)   # d alpha = alpha * d log_alpha
                args["alpha"] = [[_Dual(alpha[t][i], alpha[t][i] * d[t][i]) for i in range(dk)] for t in range(T)]
                got = float(np.sum(g["log_alpha"][:, 0, :] * f(d)))
            elif name == "beta":
                d = [fr(-5, 5, 4) for _ in range(T)]
                args["beta"] = [_Dual(beta[t], d[t]) for t in range(T)]
                got = float(np.sum(g["beta"][:, 0] * np.array([float(x) for x in d])))
            else:
                d = D(dk, dv)
                args["S0"] = [[_Dual(S0[i][j], d[i][j]) for j in range(dv)] for i in range(dk)]
                got = float(np.sum(g["init_state"][0, 0] * f(d).T))
            L = _literal_loss_dual(args["alpha"], args["beta"], args["k"], args["v"], args["q"], args["S0"],
                                   d_o, d_final)
            want = float(L.b)
            assert abs(got - want) <= 1e-11 * max(1.0, abs(want)), ("exact directional derivative", name, dk, dv)


def check_grad_beta_zero_closed_form(lib, seed=23):
    """beta = 0: S_t = Diag(Gamma_t) S0 with Gamma_t = exp(cumsum log_alpha),
    so the gradients have closed forms (dk = dv = 0 exactly)"""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 20, 2, 4, 5
    q, k, v, la, _ = _rand_inputs(rng, T, H, dk, dv, la_lo=-0.5)
    beta = np.zeros((T, H))
    S0 = rng.standard_normal((1, H, dv, dk))
    d_o = rng.standard_normal((T, H, dv))
    d_final = rng.standard_normal((1, H, dv, dk))
    g = oracle.prefill_grad(q, k, v, la, beta, [0, T], S0, d_o, d_final, lib=lib, nthreads=2)
    for h in range(H):
        s0 = S0[0, h].T                                   # dk x dv
        gam = np.exp(np.cumsum(la[:, h, :], axis=0))      # Gamma_t, [T, dk]
        St = gam[:, :, None] * s0[None]                   # [T, dk, dv]
        dq = np.einsum("tij,tj->ti", St, d_o[:, h])
        # dL/dS_t accumulated from the future, mapped back to S_t's own scale
        Gt = np.zeros((T, dk, dv))
        acc = d_final[0, h].T.copy()
        for t in range(T - 1, -1, -1):
            acc = acc + np.outer(q[t, h], d_o[t, h])
            Gt[t] = acc
            if t > 0:
                acc = acc * np.exp(la[t, h])[:, None]
        d_init = np.exp(la[0, h])[:, None] * Gt[0]
        # d log_alpha_t[i] = sum_{s >= t} sum_j (q_s[i] do_s[j] + [s = T-1] dS_T) S_s,ij
        contrib = np.einsum("ti,tj,tij->ti", q[:, h], d_o[:, h], St)
        contrib[-1] += np.sum(d_final[0, h].T * St[-1], axis=1)
        dla = np.cumsum(contrib[::-1], axis=0)[::-1]
        # d beta_t = (G_t^T k_t) . (v_t - D_t^T k_t) with D_t = S_t at beta = 0
        dbeta = np.array([np.dot(Gt[t].T @ k[t, h], v[t, h] - St[t].T @ k[t, h]) for t in range(T)])
        assert _rel(g["q"][:, h], dq) < 1e-12, "beta=0: dq"
        assert np.all(g["k"][:, h] == 0.0) and np.all(g["v"][:, h] == 0.0), "beta=0: dk, dv vanish"
        assert _rel(g["init_state"][0, h].T, d_init) < 1e-12, "beta=0: d init_state"
        assert _rel(g["log_alpha"][:, h], dla) < 1e-12, "beta=0: d log_alpha"
        assert _rel(g["beta"][:, h], dbeta) < 1e-12, "beta=0: d beta"


ALL_GRAD_CHECKS = [
    check_grad_finite_differences,
    check_grad_exact_directional,
    check_grad_beta_zero_closed_form,
]
