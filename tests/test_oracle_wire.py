"""Pins of the oracle's wire message (the group layout one worker would send
in the exchange): a hand-derived example, the layout read back with numpy's
own little-endian views, round trips, and malformed messages."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "wire_example.json")


def test_hand_derived_example():
    ex = json.load(open(GOLDEN))
    streams, Ms = [], []
    for t in ex["tensors"]:
        x = np.array(t["x"], np.float32)
        st, M, _ = oracle.compress(x, np.zeros_like(x), t["s"])
        assert st.tolist() == t["stream"] and float(M) == t["M"]
        streams.append(st)
        Ms.append(M)
    wire = oracle.wire_pack(streams, np.array(Ms, np.float32))
    assert wire.tolist() == ex["wire"]
    back, M2 = oracle.wire_unpack(np.array(ex["wire"], np.uint8), [len(t["x"]) for t in ex["tensors"]])
    assert [b.tolist() for b in back] == [t["stream"] for t in ex["tensors"]]
    assert M2.tolist() == [t["M"] for t in ex["tensors"]]


@pytest.mark.parametrize("seed", range(6))
def test_layout_read_back_with_numpy_views(seed):
    rng = np.random.default_rng(seed)
    count = int(rng.integers(1, 60))
    sizes = [int(v) for v in rng.integers(1, 5000, count)]
    streams = [rng.integers(0, 256, int(rng.integers(0, -(-n // 5) + 1)), dtype=np.uint8) for n in sizes]
    Ms = (rng.standard_normal(count) * 10 ** rng.uniform(-40, 30, count)).astype(np.float32)
    wire = oracle.wire_pack(streams, Ms)
    lens = np.array([st.size for st in streams])
    assert wire.size == 8 * count + lens.sum()
    hdr = wire[:8 * count].reshape(count, 8)
    assert np.array_equal(hdr[:, :4].copy().view("<u4").ravel(), lens.astype(np.uint32))
    assert np.array_equal(hdr[:, 4:].copy().view("<u4").ravel(), Ms.view(np.uint32))
    assert np.array_equal(wire[8 * count:], np.concatenate(streams + [np.zeros(0, np.uint8)]))
    back, M2 = oracle.wire_unpack(wire, sizes)
    assert all(np.array_equal(a, b) for a, b in zip(back, streams))
    assert np.array_equal(M2.view(np.uint32), Ms.view(np.uint32))
    # bytes after the message are ignored
    back2, _ = oracle.wire_unpack(np.concatenate([wire, np.full(7, 0xAB, np.uint8)]), sizes)
    assert all(np.array_equal(a, b) for a, b in zip(back2, streams))


def test_round_trip_of_compressed_group():
    rng = np.random.default_rng(11)
    sizes = [1, 4, 5, 6, 5120, 5121, 30_001]
    streams, Ms = [], []
    for n in sizes:
        x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        st, M, _ = oracle.compress(x, np.zeros(n, np.float32), 1.5)
        streams.append(st)
        Ms.append(M)
    wire = oracle.wire_pack(streams, np.array(Ms, np.float32))
    back, M2 = oracle.wire_unpack(wire, sizes)
    for n, a, b, m in zip(sizes, back, streams, M2):
        assert np.array_equal(a, b)
        assert np.array_equal(oracle.decompress(a, m, n, 1.5), oracle.decompress(b, m, n, 1.5))


def test_malformed_messages():
    sizes = [10, 3]  # capacities 2 and 1
    wire = np.array(json.load(open(GOLDEN))["wire"], np.uint8)
    for bad in (wire[:17], wire[:15], wire[:0]):  # truncated streams, truncated headers, empty
        with pytest.raises(oracle.OracleError) as e:
            oracle.wire_unpack(bad, sizes)
        assert e.value.code == oracle.ERR_CORRUPT
    too_long = wire.copy()
    too_long[8] = 2  # tensor 1 claims 2 bytes, its capacity is 1
    with pytest.raises(oracle.OracleError) as e:
        oracle.wire_unpack(np.concatenate([too_long, np.zeros(4, np.uint8)]), sizes)
    assert e.value.code == oracle.ERR_CORRUPT
