"""saf_attn_bwd_noalloc (the backward for callers that cannot allocate, its workspace in the
library's own device array) against saf_attn_bwd with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller layer, then one with shared key/value heads. The
kernels are the same and deterministic, so the results must be bit-identical; each call is
also held to the oracle at the bf16 bar."""
import math

import numpy as np
import pytest
import torch

from hybrid_static_pattern_amd import inputs
from oracle import saf_oracle
from tests.gpu_util import check, dev, down, layer_on_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    from hybrid_static_pattern_amd import saf
    saf.load()
    return saf


def _both(S, L):
    g = layer_on_device(L)
    fz = L["frozen"]
    o, lse = S.attn_fwd(g["q"], g["k"], g["v"], fz, g["alpha"], g["rho"])
    ref = S.attn_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, fz, g["alpha"], g["rho"],
                     dq=torch.full(tuple(g["do"].shape), float("nan"), device=dev()),
                     dk=torch.full(tuple(g["v"].shape), float("nan"), device=dev()))
    bufs = (torch.full(tuple(g["do"].shape), float("nan"), device=dev()),
            torch.full(tuple(g["v"].shape), float("nan"), device=dev()),
            torch.full(tuple(g["v"].shape), float("nan"), device=dev()))
    got = S.attn_bwd_noalloc(g["q"], g["k"], g["v"], o, g["do"], lse, fz, *bufs, alpha=g["alpha"], rho=g["rho"])
    torch.cuda.synchronize()
    return [down(t) for t in ref], [down(t) for t in got]


@pytest.mark.parametrize("case", [
    dict(B=2, H=4, T=300, D=64, frozen_heads=[1, 3]),
    dict(B=1, H=2, T=100, D=128, frozen_heads=[0]),        # smaller: the array keeps the last call's data
    dict(B=2, H=4, T=130, D=64, frozen_heads=[2], kv_heads=2),
])
def test_noalloc_matches_workspace_entry(S, case):
    L = inputs.make_layer(dtype="bf16", seed=71, **case)
    ref, got = _both(S, L)
    for name, r, x in zip(("dq", "dk", "dv"), ref, got):
        assert np.array_equal(np.isnan(r), np.isnan(x)), name   # the same entries written
        assert np.array_equal(np.nan_to_num(r), np.nan_to_num(x)), name
    dyn = L["frozen"] == 0
    scale = 1.0 / math.sqrt(L["D"])
    dq, dk, dv = saf_oracle.attn_bwd(L["q"], L["k"], L["v"], L["do"], L["frozen"], L["alpha"], L["rho"], scale)
    check(got[0][:, dyn], dq[:, dyn], "bf16", "dQ")
    if L["v"].shape[1] == L["H"]:
        check(got[1][:, dyn], dk[:, dyn], "bf16", "dK")
        check(got[2], dv, "bf16", "dV")
