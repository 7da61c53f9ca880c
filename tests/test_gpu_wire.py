"""GPU parity of the wire message (tlc_wire_pack_group / tlc_wire_unpack_group,
and the range messages of tlc_wire_pack_ranges_group / tlc_wire_unpack_ranges_group):
the message packed from a group's payload must equal, byte for byte, the
oracle's wire message of the oracle's streams and scales; unpacking it into
fresh buffers must give back every stream, length and M, so that it
decompresses to the oracle's values; malformed lengths and short messages
set TLC_ERR_CORRUPT without reading or writing outside the buffers."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, oracle_group_compress, say, to_dev

pytestmark = pytest.mark.gpu


def group_payload(sizes, seed, s=1.5, dense_every=3):
    """A group compressed on the GPU with the oracle's results beside it."""
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(seed)
    g = tlc.Group(sizes)
    x = (rng.standard_normal(g.total) * 1e-3).astype(np.float32)
    err = np.zeros(g.total, np.float32)
    off = 0
    for t, n in enumerate(sizes):  # some tensors with many nonzero codes, long streams
        if t % dense_every == 0:
            err[off:off + n] = (rng.uniform(-1, 1, n) * 3e-3).astype(np.float32)
        off += n
    streams, Ms, _ = oracle_group_compress(x, err, sizes, s)
    out, lens, scales, st = g.compress(to_dev(x), to_dev(err), s)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return g, out, lens, scales, streams, Ms, s


def check_round_trip(g, out, lens, scales, streams, Ms, s, label, trailing=0):
    import torch
    sizes = g.sizes
    want = oracle.wire_pack(streams, Ms)
    wire, wire_len, st = g.wire_pack(out, lens, scales)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, label
    wl = int(wire_len.item())
    assert wl == want.size == 8 * len(sizes) + sum(x.size for x in streams), (label, wl, want.size)
    got = wire[:wl].cpu().numpy()
    if not np.array_equal(got, want):
        i = int(np.flatnonzero(got != want)[0])
        raise AssertionError(f"{label}: message differs first at byte {i} of {wl}")
    # unpack from a buffer holding the message and `trailing` other bytes
    buf = torch.full((wl + trailing,), 0xA5, dtype=torch.uint8, device=wire.device)
    buf[:wl] = wire[:wl]
    o2, l2, s2, st2 = g.wire_unpack(buf, out=torch.full_like(out, 0x5A))
    torch.cuda.synchronize()
    assert int(st2.item()) == 0, label
    assert np.array_equal(l2.cpu().numpy(), np.array([x.size for x in streams])), label
    assert np.array_equal(bits(s2.cpu().numpy()), bits(Ms)), label
    ob = o2.cpu().numpy()
    for t, x in enumerate(streams):
        o = g.offsets[t]
        assert np.array_equal(ob[o:o + x.size], x), (label, t)
        tail = (-(o + x.size)) % 16  # the rest of the stream's last 16-byte word is written as 0
        assert not ob[o + x.size:o + x.size + tail].any(), (label, t)
    y, st_d = g.decompress(o2, l2, s2, s)
    torch.cuda.synchronize()
    assert int(st_d.item()) == 0, label
    want_y = np.concatenate([oracle.decompress(x, Ms[t], n, s) for t, (x, n) in enumerate(zip(streams, sizes))])
    assert np.array_equal(bits(y.cpu().numpy()), bits(want_y)), label


@pytest.mark.parametrize("seed", range(6))
def test_ragged_groups_round_trip(seed):
    rng = np.random.default_rng(seed)
    sizes = [int(v) for v in rng.integers(1, 60_000, 50)] + [1, 2, 5, 6, 5120, 20_481, 100_003]
    say(f"case wire ragged seed={seed}")
    check_round_trip(*group_payload(sizes, seed), label=f"ragged {seed}", trailing=int(rng.integers(0, 40)))


def test_thousands_of_tiny_tensors():
    rng = np.random.default_rng(7)
    sizes = [int(v) for v in rng.integers(1, 8, 3000)] + [4097, 3]
    say("case wire tiny tensors")
    check_round_trip(*group_payload(sizes, 7, s=1.2, dense_every=2), label="tiny")


def test_long_streams_over_many_chunks():
    # streams of several MB: every chunk boundary at every alignment
    sizes = [16_777_216 + 3, 5_000_001, 17]
    say("case wire long streams")
    check_round_trip(*group_payload(sizes, 11, dense_every=1), label="long")


def test_malformed_lengths_and_short_messages():
    import torch
    sizes = [10_000, 3, 25_000]
    g, out, lens, scales, streams, Ms, s = group_payload(sizes, 3, dense_every=1)
    caps = [-(-n // 5) for n in sizes]
    # pack: a length above its tensor's capacity is corrupt and sent empty
    bad = lens.clone()
    bad[1] = caps[1] + 1
    say("case wire pack with a length above its capacity")
    wire, wl, st = g.wire_pack(out, bad, scales)
    torch.cuda.synchronize()
    assert int(st.item()) == oracle.ERR_CORRUPT
    hdr = wire[:24].cpu().numpy().view("<u4")
    assert hdr[2] == 0 and int(wl.item()) == 24 + streams[0].size + streams[2].size
    # unpack: the good message, then cut short, then with a length above its capacity
    wire, wl, st = g.wire_pack(out, lens, scales)
    torch.cuda.synchronize()
    n = int(wl.item())
    for cut in (n - 1, 24 + streams[0].size, 24):
        say(f"case wire unpack of {cut} of {n} bytes")
        _, _, _, st2 = g.wire_unpack(wire, wire_bytes=cut)
        torch.cuda.synchronize()
        assert int(st2.item()) == oracle.ERR_CORRUPT, cut
    w2 = wire.clone()
    w2[8:12] = torch.tensor(list(int(caps[1] + 1).to_bytes(4, "little")), dtype=torch.uint8)
    say("case wire unpack of a header length above its capacity")
    _, l3, _, st3 = g.wire_unpack(w2, wire_bytes=n)
    torch.cuda.synchronize()
    assert int(st3.item()) == oracle.ERR_CORRUPT
    assert int(l3[1].item()) == 0


def test_workers_messages_into_one_sum():
    """Eight workers' payloads packed, each message unpacked on the receiving
    side, and all eight applied with the many-payload accumulate: the sum of
    the oracle's decoded payloads in worker order."""
    import torch
    sizes = [30_000, 7, 5120, 12_345]
    P = 8
    msgs, want_payloads = [], []
    for w in range(P):
        g, out, lens, scales, streams, Ms, s = group_payload(sizes, 100 + w, dense_every=1 + w % 3)
        wire, wl, st = g.wire_pack(out, lens, scales)
        msgs.append((wire, int(wl.item())))
        want_payloads.append((streams, Ms))
    inp = torch.empty((P, g.stream_bytes), dtype=torch.uint8, device="cuda:0")
    in_lens = torch.empty((P, len(sizes)), dtype=torch.int64, device="cuda:0")
    in_sc = torch.empty((P, len(sizes)), dtype=torch.float32, device="cuda:0")
    for w, (wire, wl) in enumerate(msgs):
        _, _, _, st = g.wire_unpack(wire, wire_bytes=wl, out=inp[w], out_lens=in_lens[w], scales=in_sc[w])
        torch.cuda.synchronize()
        assert int(st.item()) == 0, w
    acc0 = (np.random.default_rng(5).standard_normal(g.total) * 1e-3).astype(np.float32)
    want = acc0.copy()
    for streams, Ms in want_payloads:
        off = 0
        for t, n in enumerate(sizes):
            oracle.decompress_accumulate(streams[t], Ms[t], n, s, want[off:off + n])
            off += n
    acc = to_dev(acc0)
    say("case wire: 8 messages into one sum")
    _, st = g.decompress_accumulate_many(inp, in_lens.view(-1), in_sc.view(-1), s, acc)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(bits(acc.cpu().numpy()), bits(want))


@pytest.mark.parametrize("ranges", [1, 3, 8])
def test_range_messages(ranges):
    """tlc_wire_pack_ranges_group: message k is the oracle's message of range k
    alone; each unpacks into the whole group's payload at its range's first
    slot, and the group decompresses to the oracle's values.  One range is the
    group's message."""
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(40 + ranges)
    sizes = [int(v) for v in rng.integers(1, 30_000, 45)] + [5120, 1, 3]
    g, out, lens, scales, streams, Ms, s = group_payload(sizes, 40 + ranges, dense_every=2)
    count = len(sizes)
    cuts = [0] + sorted(int(v) for v in rng.choice(np.arange(1, count), ranges - 1, replace=False)) + [count]
    say(f"case wire ranges={ranges}")
    wire, wlens, st = g.wire_pack_ranges(out, lens, scales, cuts)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    wl = wlens.cpu().numpy()
    got = wire[:int(wl.sum())].cpu().numpy()
    want = np.concatenate([oracle.wire_pack(streams[a:b], Ms[a:b]) for a, b in zip(cuts, cuts[1:])])
    assert np.array_equal(got, want)
    assert [int(v) for v in wl] == [8 * (b - a) + sum(x.size for x in streams[a:b]) for a, b in zip(cuts, cuts[1:])]
    if ranges == 1:
        w1, l1, _ = g.wire_pack(out, lens, scales)
        torch.cuda.synchronize()
        assert int(l1.item()) == int(wl[0]) and torch.equal(w1[:int(wl[0])], wire[:int(wl[0])])
    rx = torch.full_like(out, 0x33)
    rx_lens = torch.empty_like(lens)
    rx_sc = torch.empty_like(scales)
    pos = 0
    for k, (a, b) in enumerate(zip(cuts, cuts[1:])):
        sub = tlc.Group(sizes[a:b])
        so = g.offsets[a]
        msg = wire[pos:pos + int(wl[k])].clone()  # a message of its own, as a receiver holds it
        _, _, _, st = sub.wire_unpack(msg, out=rx[so:so + sub.stream_bytes], out_lens=rx_lens[a:b],
                                      scales=rx_sc[a:b])
        torch.cuda.synchronize()
        assert int(st.item()) == 0, k
        pos += int(wl[k])
    y, st_d = g.decompress(rx, rx_lens, rx_sc, s)
    torch.cuda.synchronize()
    assert int(st_d.item()) == 0
    want_y = np.concatenate([oracle.decompress(x, Ms[t], n, s) for t, (x, n) in enumerate(zip(streams, sizes))])
    assert np.array_equal(bits(y.cpu().numpy()), bits(want_y))
    # all the messages back to back (and a few bytes after them) in one call
    total = int(wl.sum())
    buf = torch.full((total + 5,), 0xA5, dtype=torch.uint8, device=wire.device)
    buf[:total] = wire[:total]
    say(f"case wire ranges={ranges}: one unpack of the {ranges} messages")
    o1, l1, s1, st1 = g.wire_unpack_ranges(buf, cuts, out=torch.full_like(out, 0x5A))
    torch.cuda.synchronize()
    assert int(st1.item()) == 0
    assert np.array_equal(l1.cpu().numpy(), np.array([x.size for x in streams]))
    assert np.array_equal(bits(s1.cpu().numpy()), bits(Ms))
    ob, rb = o1.cpu().numpy(), rx.cpu().numpy()
    for t, x in enumerate(streams):  # each slot: the stream, then zeros to its 16-byte word's end
        o = g.offsets[t]
        e = o + x.size + (-(o + x.size)) % 16
        assert np.array_equal(ob[o:o + x.size], x) and not ob[o + x.size:e].any(), t
        assert np.array_equal(ob[o:e], rb[o:e]), t
    # cut short (inside the last message; inside the second message's
    # headers; at the last message's start; after its headers, before its
    # streams): corrupt, nothing copied, and the ranges whose headers were not
    # all inside the bytes given come out empty
    ends = [int(v) for v in np.cumsum(wl)]
    starts = [0] + ends[:-1]
    cases = {total - 1}
    if ranges > 1:
        cases |= {ends[0] + 4, starts[-1], starts[-1] + 8 * (cuts[-1] - cuts[-2])}
    for nb in sorted(cases):
        if nb < 8 * count:
            continue  # refused on the host (below 8 bytes per tensor)
        say(f"case wire ranges={ranges}: unpack of {nb} of {total} bytes")
        o2, l2, s2, st2 = g.wire_unpack_ranges(buf, cuts, wire_bytes=nb, out=torch.full_like(out, 0x5A))
        torch.cuda.synchronize()
        assert int(st2.item()) == oracle.ERR_CORRUPT, nb
        assert not (o2.cpu().numpy() != 0x5A).any(), nb
        read_to = count
        for q in range(ranges):
            if starts[q] + 8 * (cuts[q + 1] - cuts[q]) > nb:
                read_to = cuts[q]
                break
        l2h, s2h = l2.cpu().numpy(), s2.cpu().numpy()
        assert np.array_equal(l2h[:read_to], [x.size for x in streams[:read_to]]), nb
        assert not l2h[read_to:].any() and not s2h[read_to:].any(), nb
        assert np.array_equal(bits(s2h[:read_to]), bits(Ms[:read_to])), nb
    # a length above its capacity in the last range is corrupt, sent empty, and moves no other message
    bad = lens.clone()
    bad[count - 1] = -(-sizes[-1] // 5) + 1
    w2, l2, st2 = g.wire_pack_ranges(out, bad, scales, cuts)
    torch.cuda.synchronize()
    assert int(st2.item()) == oracle.ERR_CORRUPT
    l2 = l2.cpu().numpy()
    assert np.array_equal(l2[:-1], wl[:-1]) and int(l2[-1]) == int(wl[-1]) - streams[-1].size
    n_ok = int(wl[:-1].sum())
    assert torch.equal(w2[:n_ok], wire[:n_ok])


def test_range_pack_and_unpack_replayed_from_one_graph():
    """The send side's range pack and the receive side's range unpack captured
    once in a HIP graph: every replay, after an eager compress of a new
    payload into the same buffers, gives the messages and the unpacked payload
    that the eager calls give for that payload (the unpack takes the whole
    buffer's size, the messages lying back to back at its start)."""
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(77)
    sizes = [int(v) for v in rng.integers(1, 40_000, 30)] + [5120, 3, 70_001]
    g = tlc.Group(sizes)
    cuts = [0, 4, 19, len(sizes)]
    dev = "cuda:0"
    out = torch.empty(g.stream_bytes, dtype=torch.uint8, device=dev)
    lens = torch.empty(g.count, dtype=torch.int64, device=dev)
    scales = torch.zeros(g.count, dtype=torch.float32, device=dev)
    err = torch.zeros(g.total, dtype=torch.float32, device=dev)
    ws_c = g.workspace()
    st_c = torch.zeros(1, dtype=torch.int32, device=dev)
    wire = torch.zeros(g.wire_bound(), dtype=torch.uint8, device=dev)
    wl = torch.zeros(len(cuts) - 1, dtype=torch.int64, device=dev)
    rx = torch.zeros(g.stream_bytes, dtype=torch.uint8, device=dev)
    rl = torch.zeros(g.count, dtype=torch.int64, device=dev)
    rs = torch.zeros(g.count, dtype=torch.float32, device=dev)
    ws_p, ws_u = g.wire_workspace(), g.wire_workspace()
    st_p = torch.zeros(1, dtype=torch.int32, device=dev)
    st_u = torch.zeros(1, dtype=torch.int32, device=dev)

    def calls():
        g.wire_pack_ranges(out, lens, scales, cuts, wire=wire, wire_lens=wl, workspace=ws_p, status=st_p)
        g.wire_unpack_ranges(wire, cuts, out=rx, out_lens=rl, scales=rs, workspace=ws_u, status=st_u)

    say("case wire calls in one graph: capture")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            calls()
    torch.cuda.synchronize()
    for rep in range(3):
        x = (rng.standard_normal(g.total) * 10 ** -rep).astype(np.float32)
        x[rng.random(g.total) < 0.4] = 0
        g.compress(to_dev(x), err, 1.5, out=out, out_lens=lens, scales=scales, workspace=ws_c, status=st_c)
        torch.cuda.synchronize()
        assert int(st_c.item()) == 0
        say(f"case wire calls in one graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert int(st_p.item()) == 0 and int(st_u.item()) == 0, rep
        w_e, wl_e, st_e = g.wire_pack_ranges(out, lens, scales, cuts)
        torch.cuda.synchronize()
        assert int(st_e.item()) == 0
        n = int(wl_e.sum().item())
        assert torch.equal(wl, wl_e) and torch.equal(wire[:n], w_e[:n]), rep
        assert torch.equal(rl, lens), rep
        assert np.array_equal(bits(rs.cpu().numpy()), bits(scales.cpu().numpy())), rep
        ob, rb, lh = out.cpu().numpy(), rx.cpu().numpy(), lens.cpu().numpy()
        for t in range(g.count):
            o = g.offsets[t]
            assert np.array_equal(rb[o:o + int(lh[t])], ob[o:o + int(lh[t])]), (rep, t)
    del graph


def test_range_messages_over_many_scan_rounds():
    """Ranges of more than 4096 tensors (the scan's round), one of a single
    tensor, and cuts at a round's edge: each message is the oracle's, and the
    messages back to back unpack in one call into the group's payload."""
    import torch
    rng = np.random.default_rng(91)
    sizes = [int(v) for v in rng.integers(1, 12, 9000)] + [6000, 1, 20_000]
    count = len(sizes)
    g, out, lens, scales, streams, Ms, s = group_payload(sizes, 91, s=1.3, dense_every=2)
    cuts = [0, 4096, 4097, 8800, count - 1, count]
    say(f"case wire ranges over scan rounds: {count} tensors, cuts {cuts}")
    wire, wlens, st = g.wire_pack_ranges(out, lens, scales, cuts)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    total = int(wlens.sum().item())
    want = np.concatenate([oracle.wire_pack(streams[a:b], Ms[a:b]) for a, b in zip(cuts, cuts[1:])])
    got = wire[:total].cpu().numpy()
    assert got.size == want.size and np.array_equal(got, want)
    o1, l1, s1, st1 = g.wire_unpack_ranges(wire[:total].clone(), cuts, out=torch.full_like(out, 0x5A))
    torch.cuda.synchronize()
    assert int(st1.item()) == 0
    assert np.array_equal(l1.cpu().numpy(), np.array([x.size for x in streams]))
    assert np.array_equal(bits(s1.cpu().numpy()), bits(Ms))
    ob = o1.cpu().numpy()
    for t, x in enumerate(streams):
        o = g.offsets[t]
        assert np.array_equal(ob[o:o + x.size], x), t
