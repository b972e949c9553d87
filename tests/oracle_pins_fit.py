"""Pins of the compact-fit oracle (part 二.3, Eq. (3)/(4), Appendix A.2): checks against
what the page and the mathematics fix, never a re-typing of the oracle's own formula.

Each pin takes the oracle module oracle.compact_fit and raises AssertionError if it
disagrees: a hand-worked golden example, a pure-Python brute force, finite differences of
the dense cross-entropy, torch's own Adam, exact recovery of a pattern Eq. (3) can
represent, a two-position closed form, the gauge symmetries and the selection rule on a
hand-made case. tests/test_oracle_fit.py runs them and plants mistakes they must catch.
"""
from __future__ import annotations

import math

import numpy as np

from tests.oracle_pins import _fd_grad, _read_golden, _rng


def _target(seed, T, N=6, D=8):
    """A realistic fit target: the mean causal softmax attention of N random sequences
    with a shared positional component (dense, fp64, row-stochastic)."""
    r = _rng(seed)
    pos = r.standard_normal((T, D))
    rows = []
    for _ in range(N):
        q = r.standard_normal((T, D)) + pos
        k = r.standard_normal((T, D)) + pos
        S = q @ k.T / math.sqrt(D)
        S[np.triu_indices(T, 1)] = -np.inf
        E = np.exp(S - S.max(axis=1, keepdims=True))
        rows.append(E / E.sum(axis=1, keepdims=True))
    return np.mean(rows, axis=0)


def _pattern(alpha, rho):
    """Eq. (3) written out with loops (pure Python), independent of the oracle."""
    T = len(alpha)
    P = [[0.0] * T for _ in range(T)]
    for i in range(T):
        w = [math.exp(alpha[j] + rho[i - j]) for j in range(i + 1)]
        z = sum(w)
        for j in range(i + 1):
            P[i][j] = w[j] / z
    return np.array(P)


def pin_stats_golden_T3(cf):
    """Hand-worked Eq. (4) statistics (tests/golden/fit_stats_T3.txt) and the columns'
    entropy shares in closed form."""
    g = _read_golden("fit_stats_T3.txt")
    col, dist, ent = cf.pattern_stats(g["A"])
    assert np.max(np.abs(col - g["col"])) < 1e-15
    assert np.max(np.abs(dist - g["dist"])) < 1e-15
    want = [0.25 * math.log(4) + math.log(6) / 6,
            0.75 * math.log(4 / 3) + math.log(3) / 3,
            0.5 * math.log(2)]
    assert np.max(np.abs(ent - want)) < 1e-15


def pin_stats_brute_force(cf):
    """Statistics of a random T=7 target against pure-Python loops; entries above the
    diagonal are ignored."""
    T = 7
    A = _target(1, T)
    A_noisy = A + np.triu(np.full((T, T), 5.0), 1)
    col, dist, ent = cf.pattern_stats(A_noisy)
    for j in range(T):
        assert abs(col[j] - sum(A[i][j] for i in range(j, T))) < 1e-14
        assert abs(ent[j] + sum(A[i][j] * math.log(A[i][j]) for i in range(j, T))) < 1e-14
    for d in range(T):
        assert abs(dist[d] - sum(A[i][i - d] for i in range(d, T))) < 1e-14


def pin_cross_entropy_and_kl(cf):
    """Cross-entropy and KL against a pure-Python evaluation of Eq. (3); KL is 0 on a
    representable target, positive otherwise, and equals CE minus the mean row entropy."""
    T = 9
    r = _rng(2)
    alpha, rho = r.standard_normal(T), r.standard_normal(T)
    A = _target(3, T)
    P = _pattern(list(alpha), list(rho))
    ce = -sum(A[i][j] * math.log(P[i][j]) for i in range(T) for j in range(i + 1)) / T
    assert abs(cf.row_cross_entropy(alpha, rho, A) - ce) < 1e-13
    kl = cf.row_kl(alpha, rho, A)
    assert kl > 0 and abs(kl - (ce - cf.pattern_stats(A)[2].sum() / T)) < 1e-13
    assert abs(cf.row_kl(alpha, rho, P)) < 1e-14


def pin_objective_from_stats(cf):
    """Eq. (4): the cross-entropy computed from the target's two marginals equals the one
    computed from the whole target."""
    T = 11
    r = _rng(4)
    alpha, rho = 2 * r.standard_normal(T), r.standard_normal(T)
    A = _target(5, T)
    col, dist, _ = cf.pattern_stats(A)
    assert abs(cf.objective_from_stats(alpha, rho, col, dist) - cf.row_cross_entropy(alpha, rho, A)) < 1e-13


def pin_gradient_finite_difference(cf):
    """The moment-matching gradient against central differences of the dense cross-entropy
    (relative error <= 1e-7); both gradients sum to 0 (the two shift gauges)."""
    T = 10
    r = _rng(6)
    alpha, rho = r.standard_normal(T), r.standard_normal(T)
    A = _target(7, T)
    col, dist, _ = cf.pattern_stats(A)
    ga, gr = cf.objective_gradient(alpha, rho, col, dist)
    na = _fd_grad(lambda: cf.row_cross_entropy(alpha, rho, A), alpha)
    nr = _fd_grad(lambda: cf.row_cross_entropy(alpha, rho, A), rho)
    assert np.max(np.abs(ga - na)) / np.max(np.abs(na)) < 1e-7
    assert np.max(np.abs(gr - nr)) / np.max(np.abs(nr)) < 1e-7
    assert abs(ga.sum()) < 1e-15 and abs(gr.sum()) < 1e-15


def pin_adam_matches_torch(cf):
    """adam_fit against torch.optim.Adam (float64, CPU) driven by the dense cross-entropy
    through autograd, 25 steps from a random start."""
    import torch
    T, steps = 8, 25
    r = _rng(8)
    a0, r0 = 0.3 * r.standard_normal(T), 0.3 * r.standard_normal(T)
    A = _target(9, T)
    col, dist, _ = cf.pattern_stats(A)
    alpha, rho = cf.adam_fit(col, dist, a0, r0, steps=steps, lr=0.05, beta1=0.8, beta2=0.99, eps=1e-6)
    ta = torch.tensor(a0, dtype=torch.float64, requires_grad=True)
    tr = torch.tensor(r0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([ta, tr], lr=0.05, betas=(0.8, 0.99), eps=1e-6)
    At = torch.tensor(np.tril(A))
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    causal = j <= i
    dd = torch.where(causal, i - j, torch.zeros_like(i - j))
    for _ in range(steps):
        opt.zero_grad()
        logits = torch.where(causal, ta[j.expand(T, T)] + tr[dd], torch.tensor(-math.inf, dtype=torch.float64))
        logp = torch.log_softmax(logits, dim=1)
        loss = -(At * torch.where(causal, logp, torch.zeros_like(logp))).sum() / T
        loss.backward()
        opt.step()
    assert np.max(np.abs(alpha - ta.detach().numpy())) < 1e-10
    assert np.max(np.abs(rho - tr.detach().numpy())) < 1e-10


def pin_fit_recovers_representable_pattern(cf):
    """A target that Eq. (3) represents exactly is recovered: KL ~ 0 and the same pattern."""
    T = 24
    r = _rng(10)
    a_star = 0.7 * r.standard_normal(T)
    a_star[0] = 3.0
    r_star = -0.8 * np.log1p(np.arange(T)) + 0.3 * r.standard_normal(T)
    A = _pattern(list(a_star), list(r_star))
    alpha, rho, kl = cf.fit_pattern(A)
    assert kl < 1e-6, kl
    assert np.max(np.abs(_pattern(list(alpha), list(rho)) - A)) < 1e-3


def pin_fit_two_positions(cf):
    """T = 2 closed form: row 1 of the target is (a, 1 - a); the fit reaches P-hat(1,0) = a
    (the logit gap alpha(0) + rho(1) - alpha(1) - rho(0) = log(a / (1 - a)))."""
    a = 0.8
    A = np.array([[1.0, 0.0], [a, 1 - a]])
    alpha, rho, kl = cf.fit_pattern(A)
    gap = alpha[0] + rho[1] - alpha[1] - rho[0]
    assert abs(gap - math.log(a / (1 - a))) < 1e-5, gap
    assert kl < 1e-10


def pin_fit_uniform_is_fixed_point(cf):
    """The uniform causal target is the starting pattern: the fit does not move, KL = 0;
    T = 1 is trivial."""
    T = 16
    A = np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None]
    alpha, rho, kl = cf.fit_pattern(A)
    assert np.max(np.abs(alpha)) < 1e-9 and np.max(np.abs(rho)) < 1e-9 and abs(kl) < 1e-14
    a1, r1, kl1 = cf.fit_pattern(np.ones((1, 1)))
    assert a1.shape == (1,) and kl1 == 0.0


def pin_selection_skips_failed_fits(cf):
    """Appendix A.2: walk ascending s_var, skip a head whose fit fails (KL > 0.2), stop at
    k = round(r n)."""
    s = np.array([0.3, 0.1, 0.2, 0.4, 0.25, 0.1])
    kl = np.array([0.1, 0.5, 0.15, 0.05, 0.2, 0.3])
    # order: 1, 5 (tie, lower index first), 2, 4, 0, 3; heads 1 and 5 fail
    assert list(cf.select_fitted(s, kl, 0.5)) == [2, 4, 0]       # k = 3
    assert list(cf.select_fitted(s, kl, 1.0)) == [2, 4, 0, 3]    # k = 6, only 4 pass
    assert list(cf.select_fitted(s, kl, 0.25, max_kl=0.6)) == [1, 5]


PINS_FIT = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
