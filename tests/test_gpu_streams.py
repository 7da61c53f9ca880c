"""Calls on two streams at once: two groups, each with its own workspace and
status word, compress and decompress on their own torch streams over several
error-feedback steps without synchronising in between.  Both must match the
CPU oracle bit for bit (the library's process-wide state, the cached grid
sizes and the decode-path hints, must not couple the two)."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, oracle_group_compress, say, to_dev

pytestmark = pytest.mark.gpu


def test_two_streams_concurrently():
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(2024)
    groups = []
    for gidx, (count, hi, s) in enumerate(((30, 80_000, 1.25), (200, 9_000, 1.9))):
        sizes = [int(v) for v in rng.integers(1, hi, count)]
        g = tlc.Group(sizes)
        N = sum(sizes)
        xs = []
        for k in range(4):
            x = (rng.standard_normal(N) * 1e-3).astype(np.float32)
            x[rng.random(N) < 0.3] = 0
            xs.append(x)
        groups.append(dict(g=g, sizes=sizes, N=N, s=s, xs=xs, stream=torch.cuda.Stream(),
                           err=torch.zeros(N, dtype=torch.float32, device="cuda:0"),
                           ws=g.workspace(), outs=[]))
    torch.cuda.synchronize()
    for d in groups:
        d["xd"] = [to_dev(x) for x in d["xs"]]
    torch.cuda.synchronize()
    # enqueue every step of both groups before any synchronisation
    for k in range(4):
        for d in groups:
            with torch.cuda.stream(d["stream"]):
                out, lens, scales, st = d["g"].compress(d["xd"][k], d["err"], d["s"], workspace=d["ws"])
                y, st_d = d["g"].decompress(out, lens, scales, d["s"], workspace=d["ws"])
                d["outs"].append((out, lens, scales, st, y, st_d, d["err"].clone()))
    torch.cuda.synchronize()
    for gidx, d in enumerate(groups):
        err_h = np.zeros(d["N"], np.float32)
        for k in range(4):
            say(f"case two streams group {gidx} step {k}")
            out, lens, scales, st, y, st_d, err_k = d["outs"][k]
            assert int(st.item()) == 0 and int(st_d.item()) == 0
            streams, Ms, err_h = oracle_group_compress(d["xs"][k], err_h, d["sizes"], d["s"])
            assert np.array_equal(bits(scales.cpu().numpy()), bits(Ms)), (gidx, k)
            assert np.array_equal(bits(err_k.cpu().numpy()), bits(err_h)), (gidx, k)
            got_out, got_lens, got_y = out.cpu().numpy(), lens.cpu().numpy(), y.cpu().numpy()
            off = 0
            for t, n in enumerate(d["sizes"]):
                o = d["g"].offsets[t]
                assert got_lens[t] == streams[t].size and np.array_equal(got_out[o:o + got_lens[t]], streams[t])
                assert np.array_equal(bits(got_y[off:off + n]), bits(oracle.decompress(streams[t], Ms[t], n, d["s"])))
                off += n


def test_one_group_pipelined_over_two_streams():
    # The receive side overlapped with the send side, as a worker runs it:
    # batch k is compressed on one stream while payload k-1 is decompressed on
    # another, with its own workspace; events order each payload buffer's
    # write, read and reuse (two payload buffers in turn).  Every payload and
    # every decoded y must match the oracle, step by step.
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(77)
    sizes = [int(v) for v in rng.integers(1, 120_000, 25)] + [600_001]
    g = tlc.Group(sizes)
    N, s, K = sum(sizes), 1.5, 6
    xs = []
    for k in range(K):
        x = (rng.standard_normal(N) * 1e-3).astype(np.float32)
        x[rng.random(N) < 0.3] = 0
        xs.append(x)
    dev = torch.device("cuda:0")
    xd = [to_dev(x) for x in xs]
    err = torch.zeros(N, dtype=torch.float32, device=dev)
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    ws_c, ws_d = g.workspace(), g.workspace()
    pay = [(torch.empty(g.stream_bytes, dtype=torch.uint8, device=dev),
            torch.empty(len(sizes), dtype=torch.int64, device=dev),
            torch.zeros(len(sizes), dtype=torch.float32, device=dev)) for _ in range(2)]
    st_c = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(K)]
    st_d = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(K)]
    ys = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(K)]
    snaps = [None] * K  # (stream bytes, lengths, scales, err) right after compress k, copied on stream A
    ev_c = [torch.cuda.Event() for _ in range(2)]
    ev_d = [torch.cuda.Event() for _ in range(2)]
    torch.cuda.synchronize()

    def comp(k):
        b = k % 2
        if k >= 2:
            sA.wait_event(ev_d[b])
        g.compress(xd[k], err, s, out=pay[b][0], out_lens=pay[b][1], scales=pay[b][2], workspace=ws_c,
                   status=st_c[k], stream=sA)
        with torch.cuda.stream(sA):
            snaps[k] = tuple(t.clone() for t in pay[b]) + (err.clone(),)
        ev_c[b].record(sA)

    def dec(k):
        b = k % 2
        sB.wait_event(ev_c[b])
        g.decompress(pay[b][0], pay[b][1], pay[b][2], s, y=ys[k], workspace=ws_d, status=st_d[k], stream=sB)
        ev_d[b].record(sB)

    comp(0)
    for k in range(1, K):
        comp(k)
        dec(k - 1)
    dec(K - 1)
    torch.cuda.synchronize()
    err_h = np.zeros(N, np.float32)
    for k in range(K):
        say(f"case pipelined step {k}")
        assert int(st_c[k].item()) == 0 and int(st_d[k].item()) == 0
        streams, Ms, err_h = oracle_group_compress(xs[k], err_h, sizes, s)
        out_k, lens_k, sc_k, err_k = (t.cpu().numpy() for t in snaps[k])
        assert np.array_equal(bits(sc_k), bits(Ms)), k
        assert np.array_equal(bits(err_k), bits(err_h)), k
        y_k = ys[k].cpu().numpy()
        off = 0
        for t, n in enumerate(sizes):
            o = g.offsets[t]
            assert lens_k[t] == streams[t].size and np.array_equal(out_k[o:o + lens_k[t]], streams[t]), (k, t)
            assert np.array_equal(bits(y_k[off:off + n]), bits(oracle.decompress(streams[t], Ms[t], n, s))), (k, t)
            off += n
