"""The stored oracle scores of the calibration workload (N = 64, H = 12, T = 1024, d_h = 64),
which the GPU parity test holds every head's s_var, s^KL and ranking to.

Checked here on the CPU: the stored rankings are the stable ascending orders of the stored
scores (part 二.1 sorts heads by s_var ascending); neighbouring scores are far enough apart
that the GPU's 1e-3 relative bar cannot swap two heads; the temperatures are the generator's;
sharper heads (lower temperature) vary more, so both rankings follow the temperatures from
hottest to coldest; and one head recomputed by the oracle reproduces the stored values."""
import math

import numpy as np

from hybrid_static_pattern_amd import inputs
from oracle import saf_oracle
from tests import golden_calibration


def test_golden_rankings_are_the_stored_orders():
    g = golden_calibration.load()
    assert g["rank_var"] == list(np.argsort(g["s_var"], kind="stable"))
    assert g["rank_kl"] == list(np.argsort(g["s_kl"], kind="stable"))
    for key in ("s_var", "s_kl"):
        s = np.sort(g[key])
        # a 1e-3 relative error on each side cannot reorder neighbours 1% apart
        assert np.all(s[1:] > s[:-1] * 1.01), key
    hot_to_cold = list(np.argsort(-g["tau"], kind="stable"))
    assert g["rank_var"] == hot_to_cold and g["rank_kl"] == hot_to_cold


def test_golden_temperatures_and_one_head_recomputed():
    g = golden_calibration.load()
    C = inputs.make_calibration(**inputs.CALIBRATION)
    assert np.array_equal(C["tau"], g["tau"])
    h = 5
    scale = 1.0 / math.sqrt(C["D"])
    A_hat, sv, _ = saf_oracle.var_score(C["q"][:, h:h + 1], C["k"][:, h:h + 1], scale)
    _, sk, _ = saf_oracle.kl_score(C["q"][:, h:h + 1], C["k"][:, h:h + 1], scale)
    assert abs(sv[0] - g["s_var"][h]) <= 1e-12 * g["s_var"][h]
    assert abs(sk[0] - g["s_kl"][h]) <= 1e-12 * g["s_kl"][h]
    assert abs((A_hat[0] ** 2).sum() - g["a_hat_sq"][h]) <= 1e-12 * g["a_hat_sq"][h]
