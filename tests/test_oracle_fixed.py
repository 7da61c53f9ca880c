"""Pins of the oracle's fixed-length encodings, the ablations of the 3LC page
("Proposed method", second and third items): the quartic bytes without
zero-run encoding, and the 2-bit encoding the page measures quartic encoding
against (five values per byte instead of four: 20% fewer bytes).

Checked against: the pinned quantizer and quartic pack (quartic-only is
exactly their output), a hand-derived 2-bit example, round trips of every
combination of codes, the closed-form lengths and the 20% saving, the
corrupt-field check, and agreement of the decoded values with the 3LC path."""
import itertools

import numpy as np
import pytest

import oracle

Q, T = oracle.ENC_QUARTIC, oracle.ENC_TWOBIT


def test_two_bit_hand_example():
    # codes [1, 0, -1, 0, 1]: fields hold q + 1, element i in bits 2*(i%4)
    #   byte 0 = 2 | 1<<2 | 0<<4 | 1<<6 = 70
    #   byte 1 = 2 | (three missing fields of code 0) 1<<2 | 1<<4 | 1<<6 = 86
    b = oracle.pack_fixed(np.array([1, 0, -1, 0, 1], np.int8), T)
    assert b.tolist() == [70, 86]
    assert oracle.unpack_fixed(b, 5, T).tolist() == [1, 0, -1, 0, 1]


def test_two_bit_round_trip_every_combination():
    for n in range(1, 10):
        for codes in itertools.islice(itertools.product((-1, 0, 1), repeat=n), 2000):
            q = np.array(codes, np.int8)
            b = oracle.pack_fixed(q, T)
            assert b.size == -(-n // 4)
            assert np.array_equal(oracle.unpack_fixed(b, n, T), q)


def test_two_bit_field_three_is_corrupt():
    for v in (3, 3 << 2, 3 << 4, 3 << 6, 255):
        with pytest.raises(oracle.OracleError):
            oracle.unpack_fixed(np.array([v], np.uint8), 4, T)


@pytest.mark.parametrize("n", [1, 4, 5, 19, 20, 21, 1000, 5120 * 3 + 7])
def test_lengths_and_the_twenty_percent_saving(n):
    assert oracle.fixed_len(n, Q) == -(-n // 5)
    assert oracle.fixed_len(n, T) == -(-n // 4)
    if n % 20 == 0:
        assert oracle.fixed_len(n, Q) * 5 == oracle.fixed_len(n, T) * 4  # 1.6 vs 2 bits per value


@pytest.mark.parametrize("s", [1.0, 1.5, 1.9])
def test_fixed_compress_matches_the_pinned_steps(s):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(5 * 1024 + 13) * 1e-3).astype(np.float32)
    err = (rng.standard_normal(x.size) * 3e-4).astype(np.float32)
    q, M, e = oracle.quantize(x, err, s)
    bq, Mq, eq = oracle.compress_fixed(x, err, s, Q)
    assert Mq == M and np.array_equal(eq.view(np.uint32), e.view(np.uint32))
    assert np.array_equal(bq, oracle.quartic_pack(q))
    bt, Mt, et = oracle.compress_fixed(x, err, s, T)
    assert Mt == M and np.array_equal(et.view(np.uint32), e.view(np.uint32))
    assert np.array_equal(oracle.unpack_fixed(bt, x.size, T), q)
    # the three encodings decode to the same values
    st, M3, _ = oracle.compress(x, err, s)
    y3 = oracle.decompress(st, M3, x.size, s)
    for enc, b in ((Q, bq), (T, bt)):
        y = oracle.decompress_fixed(b, M, x.size, s, enc)
        assert np.array_equal(y.view(np.uint32), y3.view(np.uint32))


def test_quartic_byte_above_242_is_corrupt():
    with pytest.raises(oracle.OracleError):
        oracle.decompress_fixed(np.array([243], np.uint8), np.float32(1), 5, 1.0, Q)
