"""The per-element bar for bf16 outputs: the cache dtype's max-abs bar plus
half a bf16 ulp of the exact value, the most that rounding the result into a
bf16 output can move it."""
import numpy as np
import torch

from tests import gpu_case as G
from workloads import BF16, E4M3


def _bf16(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def test_half_ulp_bounds_bf16_rounding_and_is_reached():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * 3).astype(np.float32).astype(np.float64)  # one rounding
    r = np.abs(_bf16(x) - x)
    hu = G.bf16_half_ulp(x)
    assert np.all(r <= hu)
    # ties sit exactly half an ulp from both neighbours
    ties = np.array([1.0 + 2.0**-8, 2.0 + 2.0**-7, 4.0 + 3 * 2.0**-6, -6.0 - 2.0**-6])
    assert np.array_equal(np.abs(_bf16(ties) - ties), G.bf16_half_ulp(ties))


def test_half_ulp_values():
    x = np.array([0.0, 1.0, 1.5, 1.999, 2.0, 3.9, 4.0, 4.95, -4.95, 0.3])
    want = np.array([0.0, 2.0**-8, 2.0**-8, 2.0**-8, 2.0**-7, 2.0**-7, 2.0**-6, 2.0**-6, 2.0**-6,
                     2.0**-10])
    assert np.array_equal(G.bf16_half_ulp(x), want)


def test_bar_adds_the_rounding_to_the_dtype_bar():
    ref = np.array([0.25, 1.5, 4.95])
    assert np.allclose(G.out_bound(ref, BF16), 1e-2 + np.array([2.0**-10, 2.0**-8, 2.0**-6]))
    assert np.allclose(G.out_bound(ref, E4M3), 3e-2 + np.array([2.0**-10, 2.0**-8, 2.0**-6]))
