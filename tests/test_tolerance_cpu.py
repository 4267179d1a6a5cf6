"""The bf16 parity bar itself (no GPU): 1e-2 below |ref| = 4; above it, half
a bf16 ulp of |ref| plus the 2.2e-3 compute slack, so that an output rounded
to the wrong bf16 neighbour fails."""
import numpy as np
import torch

from tests import gpu_util as U


def _bf16(x):
    return torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double().numpy()


def test_bar_values():
    ref = np.array([0.5, 3.99, 4.0, 7.9, 8.0, 20.0])
    bar = U.bf16_bar(ref)
    assert np.allclose(bar[:2], 1e-2)
    assert np.isclose(bar[2], 0.5 / 32 + 2.2e-3)
    assert np.isclose(bar[3], 0.5 / 32 + 2.2e-3)
    assert np.isclose(bar[4], 0.5 / 16 + 2.2e-3)
    assert np.isclose(bar[5], 0.5 / 8 + 2.2e-3)


def test_correct_rounding_passes_wrong_neighbour_fails():
    rng = np.random.default_rng(0)
    ref = rng.uniform(4.0, 60.0, size=20000) * rng.choice([-1.0, 1.0], size=20000)
    rounded = _bf16(ref)                      # correctly rounded (RNE)
    bar = U.bf16_bar(ref)
    assert np.all(np.abs(rounded - ref) <= bar)
    # The other neighbour: one ulp away from the correctly rounded value, on
    # the far side of ref.
    other = rounded + np.sign(ref - rounded) * U.bf16_ulp(rounded)
    far = np.abs(other - ref) > 0.5 * U.bf16_ulp(ref) + 2.2e-3
    # Wrong-neighbour outputs fail unless ref sits within 2.2e-3 of the
    # midpoint between the two neighbours.
    near_mid = np.abs(np.abs(ref - rounded) - 0.5 * U.bf16_ulp(rounded)) <= 2.2e-3
    assert np.all(far | near_mid)
    assert far.mean() > 0.7


def test_compare_counts_relaxed_elements():
    ref = np.zeros((1, 64))
    ref[0, :4] = [5.0, 0.1, -6.0, 1.0]
    delta = np.zeros((1, 64))
    delta[0, :4] = [0.015, 0.005, -0.017, 0.0]
    got = torch.tensor(ref + delta, dtype=torch.float32)
    mx, mean, n_relaxed = U.compare(got, ref, "bf16", "unit")
    assert n_relaxed == 2
