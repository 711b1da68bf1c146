"""The CPU oracle against values fixed outside it: the stored E2M1 table, the
E8M0 closed form, torch's E4M3 / E8M0 / bf16 conversions, exact rational brute
force, one-hot activations, closed-form sums and the scale-bump invariant."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import oracle_pins as pins  # noqa: E402

CHECKS = dict(pins.all_checks())


@pytest.mark.parametrize("name", sorted(CHECKS))
def test_pin(name):
    CHECKS[name]()


@pytest.mark.parametrize("g", [1.0, 0.125, float(np.float32(1.0 / 2688.0))])
def test_nvfp4_exhaustive_decode_global_scales(g):
    pins.check_exhaustive_decode(oracle.NVFP4, g)


@pytest.mark.parametrize("fmt", pins.FMTS)
def test_random_decode_full_scale_range(fmt):
    pins.check_random_decode(fmt)


def test_moe_shared_x():
    for f in pins.FMTS:
        pins.check_moe_bruteforce(f, 0)


def test_result_independent_of_thread_count():
    rng = np.random.default_rng(2)
    codes, scales, g, x = pins._rand_case(oracle.MXFP4, rng, 64, 256)
    n0 = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        y1, _ = oracle.gemv(oracle.MXFP4, codes, scales, g, x, 64, 256)
        oracle.set_num_threads(max(2, n0))
        y2, _ = oracle.gemv(oracle.MXFP4, codes, scales, g, x, 64, 256)
    finally:
        oracle.set_num_threads(n0)
    assert (y1 == y2).all()


def test_tolerance_helper():
    y_ref = np.array([1.0, np.nan, np.inf, 100.0])
    a = np.array([10.0, np.nan, np.inf, 100.0])
    ok = oracle.within_tolerance(np.array([1.0 + 5e-5, np.nan, np.inf, 100.01]), y_ref, a)
    assert ok.tolist() == [True, True, True, False]
