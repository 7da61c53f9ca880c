"""Pins of the oracle's quartic encoding (3LC page, "Proposed method", item 2:
five ternary values packed into one byte, 20% smaller than a 2-bit code)."""
import itertools

import numpy as np
import pytest

import oracle


def all_tuples():
    return np.array(list(itertools.product((-1, 0, 1), repeat=5)), dtype=np.int8)


def test_all_243_tuples_round_trip_and_match_base3_parse():
    T = all_tuples()
    b = oracle.quartic_pack(T.ravel())
    assert b.size == 243
    # Independent formulation: the byte is the base-3 number whose digits,
    # most significant first, are q_4+1 ... q_0+1 (Python's int parser).
    for t, byte in zip(T, b):
        digits = "".join(str(int(v) + 1) for v in reversed(t))
        assert int(digits, 3) == int(byte)
    back = oracle.quartic_unpack(b, T.size).reshape(243, 5)
    assert np.array_equal(back, T)


def test_image_is_exactly_0_to_242():
    b = oracle.quartic_pack(all_tuples().ravel())
    assert sorted(b.tolist()) == list(range(243))


def test_golden_anchors(golden):
    for case in golden["quartic"]:
        b = oracle.quartic_pack(np.array(case["q"], dtype=np.int8))
        assert b.tolist() == [case["byte"]], case["id"]


def test_bits_per_value_is_20_percent_below_2bit():
    # ceil(n/5) bytes for n values: 8/5 = 1.6 bits per value when 5 | n.
    for n in (5, 10, 1_000_000):
        bits = 8 * oracle.quartic_len(n) / n
        assert bits == pytest.approx(1.6)
        assert 1 - bits / 2.0 == pytest.approx(0.20)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 9, 11, 1234])
def test_ragged_lengths_pad_with_zero_trits(n):
    rng = np.random.default_rng(n)
    q = rng.integers(-1, 2, n).astype(np.int8)
    b = oracle.quartic_pack(q)
    assert b.size == (n + 4) // 5
    padded = np.zeros(5 * b.size, dtype=np.int8)
    padded[:n] = q
    assert np.array_equal(b, oracle.quartic_pack(padded))
    assert np.array_equal(oracle.quartic_unpack(b, n), q)


def test_digit_order_is_element_order():
    # element i is digit i%5 with weight 3^(i%5)
    for j in range(5):
        q = np.zeros(5, dtype=np.int8)
        q[j] = 1
        assert oracle.quartic_pack(q)[0] == 121 + 3 ** j
        q[j] = -1
        assert oracle.quartic_pack(q)[0] == 121 - 3 ** j


def test_unpack_rejects_bytes_above_242():
    with pytest.raises(oracle.OracleError) as e:
        oracle.quartic_unpack(np.array([243], dtype=np.uint8), 5)
    assert e.value.code == oracle.ERR_CORRUPT


def test_pack_rejects_out_of_range_codes():
    with pytest.raises(oracle.OracleError) as e:
        oracle.quartic_pack(np.array([2, 0, 0, 0, 0], dtype=np.int8))
    assert e.value.code == oracle.ERR_RANGE
