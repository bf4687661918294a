"""The CPU oracle against page figures, closed forms, brute force, library
routines and invariants (no GPU)."""
import numpy as np
import pytest

import os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402
from oracle import gqa_oracle as O


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_float32_mode_matches_float64():
    res, x, w_qkv, qn, kn, w_o = P._layer_case(seed=20, b=2, l=16, hidden=64,
                                               hq=4, hkv=2, d=32)
    kw = dict(rope_theta=1e6, rms_eps=1e-6)
    a, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, **kw)
    b, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, dtype=np.float32, **kw)
    assert b.dtype == np.float32
    assert np.max(np.abs(a - b)) < 1e-4 * np.max(np.abs(a))
