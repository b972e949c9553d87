"""CPU oracle for the compact static pattern fit of SAF: Eq. (3) fitted to a target by
row-wise cross-entropy, with the target's Eq. (4) statistics.

TEST INFRASTRUCTURE ONLY. Nothing outside tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import or call this module. The product path (the HIP
library and its Python binding) never reaches it.

Plain numpy in float64; every function materialises the dense T x T pattern so that each
step can be checked against the page by eye.

Citations refer to the web page "When Can Attention Heads Be Statically Defined?:
中文精读笔记" (reading notes on the SAF paper), part 二.3 (Eq. (3), Eq. (4), Appendix A.2):
  * the static pattern is P-hat(i,j) = exp(alpha(j) + rho(i-j)) / Z(i) for j <= i, zero
    for j > i (Eq. (3));
  * alpha and rho are fitted to a target pattern A (the mean attention A-hat of part 二.1)
    by minimising the row-wise cross-entropy of P-hat relative to A; the target's absolute
    key-position marginal and distance marginal are sufficient statistics for that fit
    (Eq. (4));
  * each candidate head is fitted with 400 Adam steps and accepted when the mean row KL
    is at most 0.2 nat; a candidate that fails is skipped and the next one in variance
    order is tried (Appendix A.2).

Readings taken where the page is silent:
  * the objective is the mean over the T rows of -sum_{j<=i} A(i,j) log P-hat(i,j), and the
    acceptance measure is the mean over the T rows of KL(A_i || P-hat_i) (row 0 included,
    where both are 0);
  * Adam is the bias-corrected method of Kingma and Ba (2015) with lr 0.1, betas 0.9 and
    0.999, eps 1e-8, started from alpha = rho = 0 (the uniform causal pattern);
  * every candidate is fitted independently; the selection walks the candidates in
    ascending s_var order (ties to the lower index) and keeps those whose fit passes,
    until k = round(r L H) are kept or the candidates run out.

Parity: every function here is pinned by the -m "not gpu" tests in tests/ (a hand-worked
golden example, a pure-Python brute force, finite differences, torch's Adam, exact
recovery of a representable pattern, closed forms).
"""
from __future__ import annotations

import numpy as np

from .saf_oracle import frozen_probs, n_selected, rank_heads

# Appendix A.2 (part 二.3): 400 Adam steps, acceptance at a mean row KL of 0.2 nat.
FIT_STEPS = 400
MAX_KL = 0.2
# Adam hyper-parameters (a reading: the page names the optimiser only).
ADAM_LR, ADAM_BETA1, ADAM_BETA2, ADAM_EPS = 0.1, 0.9, 0.999, 1e-8


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def pattern_stats(A):
    """Eq. (4) statistics of a causal row-stochastic target A [T,T] (entries j > i unused).

    col(j)  = sum_{i >= j} A(i, j)             absolute key-position marginal;
    dist(d) = sum_{i >= d} A(i, i - d)         distance marginal;
    ent(j)  = -sum_{i >= j} A(i, j) log A(i, j) with 0 log 0 = 0, the column's share of the
              target's entropy: sum_j ent(j) / T is the mean row entropy, the constant that
              turns the mean row cross-entropy into the mean row KL.
    """
    A = _f64(A)
    T = A.shape[0]
    L = np.tril(A)
    col = L.sum(axis=0)
    dist = np.array([np.trace(L, offset=-d) for d in range(T)])
    logL = np.log(np.where(L > 0, L, 1.0))
    ent = -(L * logL).sum(axis=0)
    return col, dist, ent


def row_cross_entropy(alpha, rho, A):
    """The fit objective: mean over rows i of -sum_{j<=i} A(i,j) log P-hat(i,j)."""
    A = np.tril(_f64(A))
    T = A.shape[0]
    P, _ = frozen_probs(alpha, rho)
    pos = A > 0
    return float(-(A[pos] * np.log(P[pos])).sum() / T)


def row_kl(alpha, rho, A):
    """Acceptance measure: mean over rows i of KL(A_i || P-hat_i) = sum_j A log(A / P-hat)."""
    A = np.tril(_f64(A))
    T = A.shape[0]
    P, _ = frozen_probs(alpha, rho)
    pos = A > 0
    return float((A[pos] * (np.log(A[pos]) - np.log(P[pos]))).sum() / T)


def objective_from_stats(alpha, rho, col, dist):
    """The row cross-entropy written with the Eq. (4) statistics alone (rows of A sum to 1):
    -sum_j A(i,j) log P-hat(i,j) = log Z(i) - sum_j A(i,j) (alpha(j) + rho(i-j)), so the mean
    over rows is (1/T) [sum_i log Z(i) - sum_j alpha(j) col(j) - sum_d rho(d) dist(d)]."""
    alpha, rho = _f64(alpha), _f64(rho)
    T = alpha.shape[0]
    _, logZ = frozen_probs(alpha, rho)
    return float((logZ.sum() - alpha @ _f64(col) - rho @ _f64(dist)) / T)


def objective_gradient(alpha, rho, col, dist):
    """Gradient of objective_from_stats: the statistics of P-hat minus those of the target,
    over T (moment matching): d/d alpha(j) = (sum_i P-hat(i,j) - col(j)) / T and
    d/d rho(d) = (sum_i P-hat(i,i-d) - dist(d)) / T."""
    alpha = _f64(alpha)
    T = alpha.shape[0]
    P, _ = frozen_probs(alpha, rho)
    col_p, dist_p, _ = pattern_stats(P)
    return (col_p - _f64(col)) / T, (dist_p - _f64(dist)) / T


def adam_fit(col, dist, alpha0, rho0, steps=FIT_STEPS, lr=ADAM_LR, beta1=ADAM_BETA1,
             beta2=ADAM_BETA2, eps=ADAM_EPS):
    """Adam (Kingma and Ba, 2015, bias-corrected) on objective_from_stats from (alpha0, rho0).

    Per step t = 1..steps and parameter x with gradient g:
      m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
      x -= lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps).
    """
    x = [_f64(alpha0).copy(), _f64(rho0).copy()]
    m = [np.zeros_like(x[0]), np.zeros_like(x[1])]
    v = [np.zeros_like(x[0]), np.zeros_like(x[1])]
    for t in range(1, steps + 1):
        g = objective_gradient(x[0], x[1], col, dist)
        for p in range(2):
            m[p] = beta1 * m[p] + (1 - beta1) * g[p]
            v[p] = beta2 * v[p] + (1 - beta2) * g[p] ** 2
            m_hat = m[p] / (1 - beta1 ** t)
            v_hat = v[p] / (1 - beta2 ** t)
            x[p] = x[p] - lr * m_hat / (np.sqrt(v_hat) + eps)
    return x[0], x[1]


def fit_pattern(A, steps=FIT_STEPS, lr=ADAM_LR, beta1=ADAM_BETA1, beta2=ADAM_BETA2,
                eps=ADAM_EPS):
    """Compact fit of one candidate (part 二.3): Eq. (4) statistics of the target, Adam from
    the uniform pattern, and the mean row KL of the result. Returns alpha, rho, kl."""
    col, dist, _ = pattern_stats(A)
    T = np.shape(A)[0]
    alpha, rho = adam_fit(col, dist, np.zeros(T), np.zeros(T), steps, lr, beta1, beta2, eps)
    return alpha, rho, row_kl(alpha, rho, A)


def select_fitted(s_var_all, kl_all, r: float, max_kl: float = MAX_KL):
    """Selection with the fit's acceptance test (part 二.1 and Appendix A.2): walk all L*H
    heads by ascending s_var (ties to the lower index), keep a head when its fitted pattern
    has mean row KL <= max_kl, skip it otherwise, and stop once k = round(r L H) are kept.
    Returns the kept head indices in walk order (fewer than k if too few pass)."""
    s = np.asarray(s_var_all).reshape(-1)
    kl = np.asarray(kl_all).reshape(-1)
    k = n_selected(r, s.size)
    kept = []
    for h in rank_heads(s):
        if len(kept) == k:
            break
        if kl[h] <= max_kl:
            kept.append(int(h))
    return np.array(kept, dtype=np.int32)
