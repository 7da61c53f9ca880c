"""Pins of the oracle's five-plane layout (byte k holds elements k + j*B,
j = 0..4, as digit j; B = ceil(n/5)), the other reading of which five values
share a quartic byte (3LC page, "Proposed method", second item).  The layout
is a convention the page does not fix; it is pinned here by hand-derived
examples, by an independent formulation (the consecutive packing applied to
the elements reordered by numpy indexing), and by round trips."""
import numpy as np
import pytest

import oracle


def planes_order(n):
    """Index of the element at consecutive position p = 5k + j (or -1 for a pad)."""
    B = -(-n // 5)
    p = np.arange(5 * B)
    i = p // 5 + (p % 5) * B
    return np.where(i < n, i, -1)


def reorder(a, n):
    idx = planes_order(n)
    out = np.zeros(idx.size, dtype=a.dtype)
    out[idx >= 0] = a[idx[idx >= 0]]
    return out


def test_golden_planes(golden):
    for case in golden["planes"]:
        x = np.array(case["x"], np.float32)
        e = np.array(case["err"], np.float32)
        q, M, _ = oracle.quantize(x, e, case["s"])
        assert list(q) == case["q"], case["id"]
        assert float(M) == case["M"], case["id"]
        assert list(oracle.quartic_pack_planes(q)) == case["bytes"], case["id"]
        stream, M2, _ = oracle.compress_planes(x, e, case["s"])
        assert list(stream) == case["stream"], case["id"]
        y = oracle.decompress_planes(stream, M2, x.size, case["s"])
        assert np.array_equal(y, q.astype(np.float32) * np.float32(M2 * np.float32(case["s"]))), case["id"]


@pytest.mark.parametrize("n", list(range(1, 41)) + [997, 1000, 5121, 10_007])
def test_pack_equals_consecutive_packing_of_reordered_codes(n):
    rng = np.random.default_rng(n)
    q = rng.integers(-1, 2, n).astype(np.int8)
    want = oracle.quartic_pack(reorder(q, n))
    assert np.array_equal(oracle.quartic_pack_planes(q), want)
    assert np.array_equal(oracle.quartic_unpack_planes(want, n), q)


def test_every_code_position_round_trips():
    # a single nonzero code at every position of small tensors: the byte and
    # digit it lands in are k = i mod B and j = i div B
    for n in range(1, 31):
        B = -(-n // 5)
        for i in range(n):
            for t in (-1, 1):
                q = np.zeros(n, np.int8)
                q[i] = t
                b = oracle.quartic_pack_planes(q)
                want = np.full(B, 121, np.uint8)
                want[i % B] = 121 + t * 3 ** (i // B)
                assert np.array_equal(b, want), (n, i, t)
                assert np.array_equal(oracle.quartic_unpack_planes(b, n), q)


@pytest.mark.parametrize("n,s", [(5, 1.0), (1234, 1.5), (70_001, 1.9), (131_072, 1.0)])
def test_compress_equals_consecutive_on_reordered_tensor(n, s):
    rng = np.random.default_rng(n + 7)
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    x[rng.random(n) < 0.3] = 0
    e = (rng.standard_normal(n) * 3e-4).astype(np.float32)
    stream, M, e_new = oracle.compress_planes(x, e, s)
    xr, er = reorder(x, n), reorder(e, n)
    stream_r, M_r, e_r = oracle.compress(xr, er, s)
    assert M == M_r
    assert np.array_equal(stream, stream_r)
    idx = planes_order(n)
    back = np.empty(n, np.float32)
    back[idx[idx >= 0]] = e_r[idx >= 0]
    assert np.array_equal(e_new.view(np.uint32), back.view(np.uint32))
    y = oracle.decompress_planes(stream, M, n, s)
    yr = oracle.decompress(stream_r, M_r, xr.size, s)
    back_y = np.empty(n, np.float32)
    back_y[idx[idx >= 0]] = yr[idx >= 0]
    assert np.array_equal(y.view(np.uint32), back_y.view(np.uint32))
