"""The compact-fit oracle against its pins, and plausible mistakes planted in it (on the
CPU, for the duration of one test) that the pins must catch."""
import numpy as np
import pytest

from oracle import compact_fit as cf
from tests.oracle_pins_fit import PINS_FIT


@pytest.mark.parametrize("pin", PINS_FIT, ids=[p.__name__ for p in PINS_FIT])
def test_fit_oracle_pin(pin):
    pin(cf)


def _orig(name):
    return cf.__dict__["_orig_" + name]


def _stats_dist_transposed(A):
    col, _, ent = _orig("pattern_stats")(A)
    L = np.tril(np.asarray(A, float))
    return col, np.array([np.trace(L, offset=d) for d in range(L.shape[0])]), ent


def _stats_row_sums(A):
    _, dist, ent = _orig("pattern_stats")(A)
    return np.tril(np.asarray(A, float)).sum(axis=1), dist, ent


def _stats_entropy_sign(A):
    col, dist, ent = _orig("pattern_stats")(A)
    return col, dist, -ent


def _stats_entropy_by_rows(A):
    col, dist, _ = _orig("pattern_stats")(A)
    L = np.tril(np.asarray(A, float))
    return col, dist, -(L * np.log(np.where(L > 0, L, 1.0))).sum(axis=1)


def _grad_sign(alpha, rho, col, dist):
    ga, gr = _orig("objective_gradient")(alpha, rho, col, dist)
    return -ga, -gr


def _grad_no_T(alpha, rho, col, dist):
    ga, gr = _orig("objective_gradient")(alpha, rho, col, dist)
    T = np.shape(alpha)[0]
    return ga * T, gr * T


def _grad_swapped(alpha, rho, col, dist):
    ga, gr = _orig("objective_gradient")(alpha, rho, dist, col)
    return ga, gr


def _adam_factory(kind):
    def adam_fit(col, dist, alpha0, rho0, steps=cf.FIT_STEPS, lr=cf.ADAM_LR, beta1=cf.ADAM_BETA1,
                 beta2=cf.ADAM_BETA2, eps=cf.ADAM_EPS):
        x = [np.array(alpha0, float), np.array(rho0, float)]
        m = [np.zeros_like(x[0]), np.zeros_like(x[1])]
        v = [np.zeros_like(x[0]), np.zeros_like(x[1])]
        for t in range(1, steps + 1):
            g = cf.objective_gradient(x[0], x[1], col, dist)
            for p in range(2):
                m[p] = beta1 * m[p] + (1 - beta1) * g[p]
                v[p] = beta2 * v[p] + (1 - beta2) * g[p] ** 2
                if kind == "no_bias_correction":
                    x[p] = x[p] - lr * m[p] / (np.sqrt(v[p]) + eps)
                elif kind == "eps_inside_sqrt":
                    x[p] = x[p] - lr * (m[p] / (1 - beta1 ** t)) / np.sqrt(v[p] / (1 - beta2 ** t) + eps)
                else:   # "ascent"
                    x[p] = x[p] + lr * (m[p] / (1 - beta1 ** t)) / (np.sqrt(v[p] / (1 - beta2 ** t)) + eps)
        return x[0], x[1]
    return adam_fit


def _kl_is_ce(alpha, rho, A):
    return cf.row_cross_entropy(alpha, rho, A)


def _select_no_skip(s_var_all, kl_all, r, max_kl=cf.MAX_KL):
    s = np.asarray(s_var_all).reshape(-1)
    return cf.rank_heads(s)[: cf.n_selected(r, s.size)]


def _select_by_kl(s_var_all, kl_all, r, max_kl=cf.MAX_KL):
    return _orig("select_fitted")(kl_all, kl_all, r, max_kl)


MUTANTS = {
    "stats: distance marginal from the upper diagonals": ("pattern_stats", _stats_dist_transposed),
    "stats: column marginal replaced by row sums": ("pattern_stats", _stats_row_sums),
    "stats: entropy sign": ("pattern_stats", _stats_entropy_sign),
    "stats: entropy shares by rows, not columns": ("pattern_stats", _stats_entropy_by_rows),
    "gradient: sign flipped": ("objective_gradient", _grad_sign),
    "gradient: 1/T dropped": ("objective_gradient", _grad_no_T),
    "gradient: marginals swapped": ("objective_gradient", _grad_swapped),
    "adam: no bias correction": ("adam_fit", _adam_factory("no_bias_correction")),
    "adam: eps inside the square root": ("adam_fit", _adam_factory("eps_inside_sqrt")),
    "adam: ascent": ("adam_fit", _adam_factory("ascent")),
    "kl: cross-entropy without the entropy": ("row_kl", _kl_is_ce),
    "select: failed fits not skipped": ("select_fitted", _select_no_skip),
    "select: walks by KL instead of s_var": ("select_fitted", _select_by_kl),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_fit_pins_reject_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    for orig in ("pattern_stats", "objective_gradient", "select_fitted"):
        monkeypatch.setitem(cf.__dict__, "_orig_" + orig, getattr(cf, orig))
    monkeypatch.setattr(cf, attr, fn)
    caught = []
    for pin in PINS_FIT:
        try:
            pin(cf)
        except Exception:  # an assertion, or the mutant breaking the pin outright
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant '{name}'"
