"""Oracle of the lifetime-aware bit allocation (test infrastructure only).

Written from the pages, not from the library: STEPQuant talk preview
(qingkeai.online), "STEPQuant 核心设计…" (time axis: each unit's error at each
width and how long the unit lives, under a fixed memory budget); e-cogni
STEPQuant analysis, "O que os autores propõem" (the allocation minimises a
lifetime-weighted reconstruction distortion under a fixed bit budget; the
riskiest units become binary16 pivots) and "Como funciona" (the lifetime
weight decays about exponentially); gpt-diffusion analysis, "Qué dice
realmente el «6-bit»" (pivots are counted apart from the nominal budget).

Readings (also in the library's contract): the lifetime weight of a unit with
gate half-life h tokens is the sum over future steps of the retained fraction,
sum_t 2^(-t/h) = 1 / (1 - 2^(-1/h)); the objective is sum_u w_u err_u(b_u)
over the quantized units (a pivot adds nothing); the pivots are the n_piv
units with the largest w_u err_u(8) (ties to the lower index); the widths
{4, 6, 8} of the other m units must satisfy sum_u b_u <= budget * m.
"""
import itertools

import numpy as np

WIDTHS = (4, 6, 8)


def lifetime_weight(h):
    """sum_{t>=0} 2^(-t/h), summed in closed form (geometric series)."""
    h = np.asarray(h, np.float64)
    return 1.0 / (1.0 - 2.0 ** (-1.0 / h))


def pivots(err, half_life, n_piv):
    """Indices of the n_piv riskiest units (largest w * err at 8 bits, ties to the lower index)."""
    risk = lifetime_weight(half_life) * np.asarray(err, np.float64)[:, 2]
    order = sorted(range(len(risk)), key=lambda u: (-risk[u], u))
    return sorted(order[:n_piv])


def _rest(err, half_life, n_piv):
    piv = pivots(err, half_life, n_piv)
    rest = [u for u in range(len(err)) if u not in set(piv)]
    return piv, rest, lifetime_weight(half_life)


def objective(err, half_life, bits):
    """Lifetime-weighted distortion of an assignment (binary16 pivots add nothing)."""
    w = lifetime_weight(half_life)
    err = np.asarray(err, np.float64)
    return float(sum(w[u] * err[u, WIDTHS.index(b)] for u, b in enumerate(bits) if b != 16))


def allocate_bruteforce(err, half_life, n_piv, budget):
    """Every assignment of {4, 6, 8} to the non-pivot units (tiny inputs only)."""
    err = np.asarray(err, np.float64)
    piv, rest, w = _rest(err, half_life, n_piv)
    cap = budget * len(rest)
    best, arg = np.inf, None
    for choice in itertools.product(range(3), repeat=len(rest)):
        if sum(WIDTHS[c] for c in choice) > cap:
            continue
        v = sum(w[u] * err[u, c] for u, c in zip(rest, choice))
        if v < best:
            best, arg = v, choice
    bits = np.full(len(err), 16, np.int32)
    for u, c in zip(rest, arg):
        bits[u] = WIDTHS[c]
    return bits, best


def allocate_milp(err, half_life, n_piv, budget):
    """The same problem as a 0/1 integer program (one binary per unit and width,
    one width per unit, the width budget), solved by scipy's MILP solver."""
    from scipy.optimize import Bounds, LinearConstraint, milp
    err = np.asarray(err, np.float64)
    piv, rest, w = _rest(err, half_life, n_piv)
    m = len(rest)
    c = np.concatenate([w[u] * err[u] for u in rest])
    one = np.zeros((m, 3 * m))
    for i in range(m):
        one[i, 3 * i:3 * i + 3] = 1.0
    wid = np.tile(np.array(WIDTHS, np.float64), m)[None, :]
    cons = [LinearConstraint(one, 1.0, 1.0), LinearConstraint(wid, -np.inf, budget * m)]
    r = milp(c, constraints=cons, integrality=np.ones(3 * m), bounds=Bounds(0, 1),
             options={"mip_rel_gap": 0.0})
    assert r.success, r.message
    x = np.round(r.x).reshape(m, 3)
    bits = np.full(len(err), 16, np.int32)
    for i, u in enumerate(rest):
        bits[u] = WIDTHS[int(np.argmax(x[i]))]
    return bits, float(r.fun)


def lp_bound(err, half_life, n_piv, budget):
    """Optimum of the linear relaxation: a lower bound on every feasible assignment."""
    from scipy.optimize import linprog
    err = np.asarray(err, np.float64)
    piv, rest, w = _rest(err, half_life, n_piv)
    m = len(rest)
    c = np.concatenate([w[u] * err[u] for u in rest])
    one = np.zeros((m, 3 * m))
    for i in range(m):
        one[i, 3 * i:3 * i + 3] = 1.0
    wid = np.tile(np.array(WIDTHS, np.float64), m)[None, :]
    r = linprog(c, A_ub=wid, b_ub=[budget * m], A_eq=one, b_eq=np.ones(m), bounds=(0, 1), method="highs")
    assert r.success
    return float(r.fun)
