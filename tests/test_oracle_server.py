"""Pins of the oracle's model-delta direction (3LC page, "Proposed method",
fourth item: the same pipeline compresses model deltas as well as
gradients).  The server's state change is the mean of the workers' decoded
payloads, acc / workers in fp32, compressed with the server's own error
buffer.

Checked against: the pinned compress path where the definition reduces to it
(one worker; a power-of-two worker count, where the division is an exact
scaling), an exact rational-arithmetic rounding of acc / workers for other
worker counts, the error-feedback invariant, the decoded values being 0 or
+-M*s, and the argument checks."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def f32_round(fr: Fraction) -> np.float32:
    """The float32 nearest to a rational (ties to even), by exact comparison
    with the neighbouring float32 values."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        even = (int(cand.view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return best[1]


def worker_sum(n, workers, seed, s=1.75):
    """acc = sum of `workers` decoded payloads, as the server forms it."""
    rng = np.random.default_rng(seed)
    acc = np.zeros(n, np.float32)
    for w in range(workers):
        x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        st, M, _ = oracle.compress(x, np.zeros(n, np.float32), s)
        oracle.decompress_accumulate(st, M, n, s, acc)
    return acc


def test_one_worker_is_compress():
    rng = np.random.default_rng(1)
    acc = (rng.standard_normal(4099) * 1e-2).astype(np.float32)
    err = (rng.standard_normal(4099) * 1e-3).astype(np.float32)
    for s in (1.0, 1.5, 1.9):
        a = oracle.server_compress(acc, 1, err, s)
        b = oracle.compress(acc, err, s)
        assert np.array_equal(a[0], b[0]) and a[1] == b[1]
        assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


@pytest.mark.parametrize("workers", [2, 8, 64])
def test_power_of_two_workers_is_exact_scaling(workers):
    # acc / 2^k and acc * 2^-k are the same correctly rounded value
    acc = worker_sum(3001, 4, seed=workers)
    acc[::7] *= np.float32(1e-38)  # subnormal quotients included
    err = np.zeros_like(acc)
    a = oracle.server_compress(acc, workers, err, 1.5)
    b = oracle.compress(acc * np.float32(1.0 / workers), err, 1.5)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1]
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


@pytest.mark.parametrize("workers", [3, 5, 7, 10])
def test_mean_rounding_is_exact(workers):
    # one large element takes the max; every other element quantizes to 0, so
    # its new error is the mean itself: compare with exact rational rounding
    rng = np.random.default_rng(workers)
    acc = (rng.standard_normal(400) * 1e-3).astype(np.float32)
    acc[17] = np.float32(1.0)
    _, M, e = oracle.server_compress(acc, workers, np.zeros_like(acc), 1.0)
    want = np.array([f32_round(Fraction(float(a)) / workers) for a in acc.tolist()], np.float32)
    assert M == want[17]
    small = np.arange(acc.size) != 17
    assert np.array_equal(e[small].view(np.uint32), want[small].view(np.uint32))
    # the max element has q = 1: err' = mean - M*s, exact
    assert e[17] == want[17] - M * np.float32(1.0)


def test_error_feedback_invariant_over_rounds():
    # per round: decode(server payload) + err_new == mean + err_old, exactly in fp32
    n, workers, s = 5003, 8, 1.75
    err = np.zeros(n, np.float32)
    for rnd in range(4):
        acc = worker_sum(n, workers, seed=100 + rnd)
        st, M, e_new = oracle.server_compress(acc, workers, err, s)
        y = oracle.decompress(st, M, n, s)
        Ms = M * np.float32(s)
        assert set(np.unique(y).tolist()) <= {0.0, float(Ms), float(-Ms)}
        v = acc * np.float32(1.0 / workers) + err
        assert np.array_equal((y + e_new).view(np.uint32), v.view(np.uint32))
        err = e_new


def test_argument_errors():
    acc = np.ones(10, np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.server_compress(acc, 0, np.zeros(10, np.float32), 1.5)
    with pytest.raises(oracle.OracleError):
        oracle.server_compress(acc, 8, np.zeros(10, np.float32), 2.0)
