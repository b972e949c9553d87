"""The seeded input generators: bf16 rounding, determinism and the stated distributions."""
import numpy as np
import torch

from hybrid_static_pattern_amd import inputs


def test_bf16_rounding_matches_torch_rne():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0, 65504.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(inputs.round_to_bf16(x), ref)
    bits = inputs.bf16_bits(inputs.round_to_bf16(x))
    assert np.array_equal(bits, torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_layer_generator_is_seeded_and_shaped():
    a = inputs.make_layer(2, 6, 64, 8, seed=5, n_frozen=2)
    b = inputs.make_layer(2, 6, 64, 8, seed=5, n_frozen=2)
    for key in ("q", "k", "v", "do", "alpha", "rho", "frozen"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (2, 6, 64, 8) and a["alpha"].shape == (6, 64)
    assert a["frozen"].sum() == 2 and np.all(a["alpha"][:, 0] == 4.0)
    assert np.array_equal(inputs.round_to_bf16(a["q"]), a["q"])
    c = inputs.make_layer(1, 4, 16, 8, dtype="fp32", frozen_heads=[3])
    assert list(c["frozen"]) == [0, 0, 0, 1]


def test_table_distributions():
    d = inputs.make_layer(1, 64, 4096, 8, seed=1, n_frozen=0)
    a = d["alpha"][:, 1:]
    assert abs(a.std() - 0.5) < 0.01 and abs(a.mean()) < 0.01
    resid = d["rho"] + 0.5 * np.log1p(np.arange(4096))[None]
    assert abs(resid.std() - 0.1) < 0.002


def test_calibration_temperatures_span():
    c = inputs.make_calibration(2, 12, 16, 8, seed=4)
    assert np.isclose(c["tau"].min(), 0.1) and np.isclose(c["tau"].max(), 4.0)
    assert not np.all(np.diff(c["tau"]) > 0)  # permuted, so rank order is not head order


def test_device_generator_is_seeded_bf16():
    """randn_bf16_device draws with torch's seeded generator (here on the CPU device): the same
    seed gives the same tensors in the same order, the values are bfloat16 N(0, 1)."""
    a = inputs.randn_bf16_device(torch, [(2, 3, 64, 8), (1, 3, 64, 8)], seed=7, device="cpu")
    b = inputs.randn_bf16_device(torch, [(2, 3, 64, 8), (1, 3, 64, 8)], seed=7, device="cpu")
    c = inputs.randn_bf16_device(torch, [(2, 3, 64, 8)], seed=8, device="cpu")
    assert [t.shape for t in a] == [(2, 3, 64, 8), (1, 3, 64, 8)]
    assert all(t.dtype == torch.bfloat16 for t in a)
    assert all(torch.equal(x, y) for x, y in zip(a, b)) and not torch.equal(a[0], c[0])
    x = a[0].float()
    assert abs(x.mean().item()) < 0.1 and abs(x.std().item() - 1.0) < 0.1
