"""The multi-step driver's learning-rate schedule: the oracle against closed
forms of its reading (warm-up line, half cosine, floor), and the library's
host function (lm_lr_schedule, no GPU involved) against the oracle."""
import ctypes
import math
import os

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_warmup_is_a_line_through_zero():
    for k in range(1, 11):
        assert oracle.lr_schedule(k, 10, 100, 3e-4, 3e-5) == pytest.approx(3e-4 * k / 10, rel=1e-15)
    # steps below 1 count as step 1
    assert oracle.lr_schedule(0, 10, 100, 3e-4, 0.0) == pytest.approx(3e-5, rel=1e-15)


def test_cosine_landmarks():
    lr, lo, W, S = 1e-3, 1e-4, 20, 220
    assert oracle.lr_schedule(W, W, S, lr, lo) == pytest.approx(lr, rel=1e-15)          # end of warm-up
    assert oracle.lr_schedule(W + 100, W, S, lr, lo) == pytest.approx((lr + lo) / 2, rel=1e-12)  # p = 1/2
    quarter = lo + (lr - lo) * (2 + math.sqrt(2)) / 4                                   # p = 1/4
    assert oracle.lr_schedule(W + 50, W, S, lr, lo) == pytest.approx(quarter, rel=1e-12)
    assert oracle.lr_schedule(S, W, S, lr, lo) == pytest.approx(lo, rel=1e-15)
    assert oracle.lr_schedule(S + 7, W, S, lr, lo) == pytest.approx(lo, rel=1e-15)


def test_decay_is_monotone_and_symmetric():
    lr, lo, W, S = 6e-4, 6e-5, 5, 105
    vals = [oracle.lr_schedule(k, W, S, lr, lo) for k in range(W, S + 1)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))
    # cos(pi p) = -cos(pi (1 - p)): points symmetric about the midpoint average to it
    for d in range(1, 50):
        a = oracle.lr_schedule(W + 50 - d, W, S, lr, lo)
        b = oracle.lr_schedule(W + 50 + d, W, S, lr, lo)
        assert (a + b) / 2 == pytest.approx((lr + lo) / 2, rel=1e-12)


def test_no_decay_phase_is_constant_after_warmup():
    assert oracle.lr_schedule(50, 10, 0, 2e-4, 0.0) == pytest.approx(2e-4, rel=1e-15)
    assert oracle.lr_schedule(50, 0, 0, 2e-4, 0.0) == pytest.approx(2e-4, rel=1e-15)


@pytest.fixture(scope="module")
def lib():
    so = os.path.join(ROOT, "scratch_decoder_only_amd", "liblmstep.so")
    if not os.path.exists(so):
        pytest.skip("library not built")
    L = ctypes.CDLL(so)
    L.lm_lr_schedule.restype = ctypes.c_float
    L.lm_lr_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float]
    return L


@pytest.mark.parametrize("W,S,lr,lo", [(10, 100, 3e-4, 3e-5), (0, 50, 6e-4, 0.0), (100, 1000, 1e-3, 1e-5),
                                       (10, 5, 5e-4, 1e-5), (0, 0, 5e-4, 0.0)])
def test_library_schedule_matches_oracle(lib, W, S, lr, lo):
    for k in list(range(0, 30)) + list(range(S - 5, S + 5)) + [S // 2, 3 * S // 4]:
        got = lib.lm_lr_schedule(k, W, S, lr, lo)
        ref = oracle.lr_schedule(k, W, S, ctypes.c_float(lr).value, ctypes.c_float(lo).value)
        # the library rounds its float64 value to fp32 once
        assert abs(got - ref) <= 2 ** -23 * abs(ref) + 1e-30, (k, got, ref)
