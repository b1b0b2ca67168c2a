"""Pins of the multi-step driver's and the generator's oracle functions:
the learning-rate schedule against closed forms of its reading (warm-up line,
half cosine, floor), the library's host schedule (lm_lr_schedule, no GPU
involved) against the oracle, and the next-token choice against closed forms
(ties, equal logits, the two-token logistic, top-1)."""
import ctypes
import math
import os

import numpy as np
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


# ------------------------------------------------------------- generation
# Pins of the oracle's next-token choice (closed forms of the sampler reading).

def test_greedy_takes_the_first_of_tied_maxima():
    z = [0.5, 2.0, -1.0, 2.0, 1.9]
    assert oracle.next_token(z, 0.0, 0, 0.3) == 1
    assert oracle.next_token(z, -1.0, 3, 0.9) == 1


def test_equal_logits_sample_uniformly_over_the_kept_ids():
    V, k = 40, 8
    z = [0.25] * V
    for j in range(k):
        u = (j + 0.5) / k
        # ties at the k-th value keep the smaller ids: ids 0..k-1, picked by floor(u k)
        assert oracle.next_token(z, 1.3, k, u) == j
    assert oracle.next_token(z, 1.3, 0, 0.999) == V - 1


def test_two_tokens_follow_the_logistic():
    a, b, T = 0.3, 1.1, 0.7
    p0 = 1.0 / (1.0 + math.exp((b - a) / T))
    assert oracle.next_token([a, b], T, 0, p0 * 0.999) == 0
    assert oracle.next_token([a, b], T, 0, p0 * 1.001) == 1


def test_top_1_is_greedy_and_top_k_drops_the_rest():
    z = [0.1, 3.0, 2.5, -4.0, 2.9]
    for u in (0.0, 0.3, 0.999):
        assert oracle.next_token(z, 2.0, 1, u) == 1
    # top 3 = {1, 2, 4}: ids 0 and 3 never come out
    picks = {oracle.next_token(z, 5.0, 3, u) for u in [i / 97 for i in range(97)]}
    assert picks == {1, 2, 4}


def test_low_temperature_approaches_greedy():
    z = [0.0, 1.0, 0.99, -2.0]
    assert oracle.next_token(z, 1e-3, 0, 0.5) == 1


def _brute_top_k(z, k):
    """Top k ids by (-value, id), by an insertion sort written out in plain
    Python (independent of the oracle's sort routines), in ascending id order."""
    chosen = []
    for i, v in enumerate(z):
        pos = len(chosen)
        while pos > 0 and (-z[chosen[pos - 1]], chosen[pos - 1]) > (-v, i):
            pos -= 1
        chosen.insert(pos, i)
        del chosen[k:]
    return sorted(chosen)


@pytest.mark.parametrize("V,k", [(300, 37), (300, 1), (1000, 250), (65, 64)])
def test_kept_ids_of_wide_vocabularies_match_a_brute_force_sort(V, k):
    """kept_ids for V > 64 (its library-sort branch) against the brute-force
    (-z, id) order, with values planted so that many tie at the k-th largest
    value: the kept ids must then be the smallest ids of that tie."""
    rng = np.random.default_rng(V + k)
    z = rng.integers(0, 6, V).astype(np.float64) * 0.5  # few distinct values: large ties
    kth = sorted(z, reverse=True)[k - 1]
    assert np.sum(z == kth) > 1  # the k-th value is tied
    got = oracle.kept_ids(z, k)
    assert list(got) == _brute_top_k(list(z), k)
    # the tie at the k-th value is cut at the smallest ids
    above = np.flatnonzero(z > kth)
    tied = np.flatnonzero(z == kth)
    assert set(got) == set(above) | set(tied[: k - above.size])


def test_cdf_bounds_of_equal_logits_are_j_over_k():
    V, k = 300, 12
    ids, lo, hi = oracle.cdf_bounds(np.full(V, -0.75), 0.8, k)
    assert list(ids) == list(range(k))
    j = np.arange(k)
    assert np.allclose(lo, j / k, rtol=0, atol=1e-15) and np.allclose(hi, (j + 1) / k, rtol=0, atol=1e-15)


def test_cdf_bounds_of_two_tokens_are_logistic():
    a, b, T = -0.4, 0.9, 1.7
    p0 = 1.0 / (1.0 + math.exp((b - a) / T))
    ids, lo, hi = oracle.cdf_bounds([a, b], T, 0)
    assert list(ids) == [0, 1]
    assert lo[0] == 0.0 and abs(hi[0] - p0) <= 1e-15 and abs(lo[1] - p0) <= 1e-15 and hi[1] == 1.0


def test_cdf_bounds_partition_the_unit_interval_by_softmax_weights():
    """V = 300 with ties planted at the k-th value: the intervals follow the
    kept ids in ascending order, tile [0, 1] without gaps, and each has the
    width of its id's tempered softmax weight over the kept set (computed by
    plain summation in Python)."""
    V, k, T = 300, 40, 0.6
    rng = np.random.default_rng(7)
    z = np.round(rng.normal(size=V), 1)
    ids, lo, hi = oracle.cdf_bounds(z, T, k)
    assert list(ids) == _brute_top_k(list(z), k)
    zmax = max(z)
    w = [math.exp((z[i] - zmax) / T) for i in ids]
    tot = math.fsum(w)
    assert lo[0] == 0.0 and abs(hi[-1] - 1.0) <= 1e-12
    assert np.array_equal(lo[1:], hi[:-1])
    assert np.allclose(hi - lo, np.array(w) / tot, rtol=1e-12, atol=0)
    # next_token picks the id whose interval holds u
    for j in range(0, k, 7):
        u = 0.5 * (lo[j] + hi[j])
        assert oracle.next_token(z, T, k, u) == ids[j]


# ------------------------------------------------------ dynamic loss scale

def test_loss_scale_rule_matches_torch_update_op():
    """The scaler's rule against torch's own loss-scale update operator (a
    library routine written independently), on a random finite / overflow
    sequence with a short interval and with the default one."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    for interval, growth, backoff in [(3, 2.0, 0.5), (2000, 2.0, 0.5), (5, 4.0, 0.25)]:
        flags = rng.random(400) < 0.93
        got = oracle.loss_scale_trace(65536.0, flags, growth, backoff, interval)
        s = torch.tensor([65536.0])
        g = torch.tensor([0], dtype=torch.int32)
        f = torch.tensor([0.0])
        for i, fin in enumerate(flags):
            f.fill_(0.0 if fin else 1.0)
            torch._amp_update_scale_(s, g, f, growth, backoff, interval)
            assert got[i] == (s.item(), g.item()), (interval, i)


def test_loss_scale_closed_forms():
    """k finite steps from a fresh run multiply S by growth^(k // interval);
    each overflow divides it by 1/backoff and restarts the run."""
    tr = oracle.loss_scale_trace(1024.0, [True] * 10, interval=3)
    assert [s for s, _ in tr] == [1024, 1024, 2048, 2048, 2048, 4096, 4096, 4096, 8192, 8192]
    assert [g for _, g in tr] == [1, 2, 0, 1, 2, 0, 1, 2, 0, 1]
    tr = oracle.loss_scale_trace(1024.0, [True, True, False, False, True], interval=3)
    assert tr == [(1024, 1), (1024, 2), (512, 0), (256, 0), (256, 1)]
