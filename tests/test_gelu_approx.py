"""The normal-CDF approximation the GPU epilogues use (Abramowitz and Stegun,
Handbook of Mathematical Functions, 7.1.26) with its published constants meets
its published error bound against float64 erf; a mistyped constant fails it."""
import math

import numpy as np

# The constants as they appear in csrc/epilogue.h.
P, A = 0.3275911, (0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429)


def _erf_7_1_26(x):
    t = 1.0 / (1.0 + P * x)
    poly = sum(a * t ** (k + 1) for k, a in enumerate(A))
    return 1.0 - poly * np.exp(-x * x)


def test_constants_match_the_source():
    import os
    src = open(os.path.join(os.path.dirname(__file__), "..", "tensor_transformer_mlp_03_amd", "csrc",
                            "epilogue.h")).read()
    for c in (P,) + A:
        assert repr(c).lstrip("-") in src


def test_error_bound():
    x = np.linspace(0.0, 6.0, 60001)
    err = np.abs(_erf_7_1_26(x) - np.array([math.erf(v) for v in x]))
    assert err.max() <= 1.5e-7
