"""Both directions of the 3LC page's exchange ("Proposed method": workers send
compressed gradients, the server sends back compressed model deltas),
simulated on one GPU with tensors sharded over owners (the reduce-scatter and
all-gather shape of SparCML's "Proposed method"), for two rounds:

  each worker compresses its gradient set and packs one wire message per
  owner (the owner's tensors are a contiguous range, and their slots in the
  worker's payload are the owner's group layout shifted by a multiple of 16);
  each owner unpacks its messages (one at a time, or all in one call), adds
  the workers' payloads in worker order with one many-payload call,
  compresses the mean with its own error buffer (carried across rounds) and
  packs one message; every worker unpacks
  the owners' messages, back to back, with one range unpack into one payload
  of the whole group and decodes the model delta with one grouped decompress.

Every message must equal the oracle's message of the oracle's streams, and
the decoded model delta the oracle's, bit for bit."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("workers,owners", [(4, 3), (8, 5)])
def test_sharded_exchange_both_directions(workers, owners):
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(100 * workers + owners)
    sizes = [int(v) for v in rng.integers(1, 40_000, 37)] + [5120, 1, 70_001]
    count = len(sizes)
    g = tlc.Group(sizes)
    cuts = [0] + sorted(int(v) for v in rng.choice(np.arange(1, count), owners - 1, replace=False)) + [count]
    shards = [(lo, hi, tlc.Group(sizes[lo:hi])) for lo, hi in zip(cuts[:-1], cuts[1:])]
    for lo, hi, sub in shards:  # the owner's layout is the full one shifted
        assert g.offsets[lo] % 16 == 0
        assert all(g.offsets[lo + k] - g.offsets[lo] == sub.offsets[k] for k in range(hi - lo))
    s = 1.75
    err_w = [np.zeros(g.total, np.float32) for _ in range(workers)]
    err_w_d = [torch.zeros(g.total, dtype=torch.float32, device="cuda:0") for _ in range(workers)]
    err_o = [np.zeros(sub.total, np.float32) for _, _, sub in shards]
    err_o_d = [torch.zeros(sub.total, dtype=torch.float32, device="cuda:0") for _, _, sub in shards]
    for rnd in range(2):
        say(f"case exchange workers={workers} owners={owners} round {rnd}")
        # workers: compress, and the oracle's streams beside them
        pays, want = [], []
        for w in range(workers):
            x = (rng.standard_normal(g.total) * 1e-3).astype(np.float32)
            x[rng.random(g.total) < 0.3] = 0
            out, lens, scales, st = g.compress(to_dev(x), err_w_d[w], s)
            streams, Ms = [], []
            off = 0
            for n in sizes:
                stt, M, e = oracle.compress(x[off:off + n], err_w[w][off:off + n], s)
                err_w[w][off:off + n] = e
                streams.append(stt)
                Ms.append(M)
                off += n
            torch.cuda.synchronize()
            assert int(st.item()) == 0
            pays.append((out, lens, scales))
            want.append((streams, np.array(Ms, np.float32)))
        deltas = []  # per owner: the oracle's model-delta streams and scales
        for k, (lo, hi, sub) in enumerate(shards):
            so = g.offsets[lo]
            inp = torch.empty((workers, sub.stream_bytes), dtype=torch.uint8, device="cuda:0")
            in_lens = torch.empty((workers, hi - lo), dtype=torch.int64, device="cuda:0")
            in_sc = torch.empty((workers, hi - lo), dtype=torch.float32, device="cuda:0")
            msgs = []
            for w, (out, lens, scales) in enumerate(pays):
                wire, wl, st = sub.wire_pack(out[so:so + sub.stream_bytes], lens[lo:hi], scales[lo:hi])
                torch.cuda.synchronize()
                assert int(st.item()) == 0
                msg = wire[:int(wl.item())].cpu().numpy()
                assert np.array_equal(msg, oracle.wire_pack(want[w][0][lo:hi], want[w][1][lo:hi])), (rnd, k, w)
                msgs.append(wire[:int(wl.item())])
            if k % 2 == 0:
                # the workers' messages back to back in one call: they are the
                # range messages of the owner's tensors repeated once per
                # worker, whose slots are the workers' payloads stacked
                rep = tlc.Group(sizes[lo:hi] * workers)
                assert rep.stream_bytes == workers * sub.stream_bytes
                _, _, _, st = rep.wire_unpack_ranges(torch.cat(msgs), [w * (hi - lo) for w in range(workers + 1)],
                                                     out=inp.view(-1), out_lens=in_lens.view(-1),
                                                     scales=in_sc.view(-1))
                torch.cuda.synchronize()
                assert int(st.item()) == 0
            else:  # one message at a time
                for w, msg in enumerate(msgs):
                    _, _, _, st = sub.wire_unpack(msg.clone(), out=inp[w], out_lens=in_lens[w], scales=in_sc[w])
                    torch.cuda.synchronize()
                    assert int(st.item()) == 0
            # the owner: workers' sum in worker order, then its compress of the mean
            acc = torch.zeros(sub.total, dtype=torch.float32, device="cuda:0")
            _, st = sub.decompress_accumulate_many(inp, in_lens.view(-1), in_sc.view(-1), s, acc)
            out_o, lens_o, sc_o, st2 = sub.server_compress(acc, workers, err_o_d[k], s)
            wire_o, wl_o, st3 = sub.wire_pack(out_o, lens_o, sc_o)
            torch.cuda.synchronize()
            assert int(st.item()) == 0 and int(st2.item()) == 0 and int(st3.item()) == 0
            acc_h = np.zeros(sub.total, np.float32)
            for w in range(workers):
                off = 0
                for t in range(lo, hi):
                    n = sizes[t]
                    oracle.decompress_accumulate(want[w][0][t], want[w][1][t], n, s, acc_h[off:off + n])
                    off += n
            st_o, M_o = [], []
            off = 0
            for t in range(lo, hi):
                n = sizes[t]
                stt, M, e = oracle.server_compress(acc_h[off:off + n], workers, err_o[k][off:off + n], s)
                err_o[k][off:off + n] = e
                st_o.append(stt)
                M_o.append(M)
                off += n
            M_o = np.array(M_o, np.float32)
            msg_o = wire_o[:int(wl_o.item())].cpu().numpy()
            assert np.array_equal(msg_o, oracle.wire_pack(st_o, M_o)), (rnd, k)
            assert np.array_equal(bits(err_o_d[k].cpu().numpy()), bits(err_o[k])), (rnd, k)
            deltas.append((wire_o, int(wl_o.item()), st_o, M_o))
        # a worker receives every owner's message, back to back in owner order
        # (as an all-gather leaves them), unpacks them in one call into one
        # payload of the whole group and decodes the model delta at once
        rx = torch.cat([wire_o[:wl_o] for wire_o, wl_o, _, _ in deltas])
        rx_out, rx_lens, rx_sc, st = g.wire_unpack_ranges(rx, cuts)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        want_delta = np.empty(g.total, np.float32)
        for (lo, hi, sub), (wire_o, wl_o, st_o, M_o) in zip(shards, deltas):
            off = g.elem_offsets[lo]
            for t in range(lo, hi):
                n = sizes[t]
                want_delta[off:off + n] = oracle.decompress(st_o[t - lo], M_o[t - lo], n, s)
                off += n
        delta, st_d = g.decompress(rx_out, rx_lens, rx_sc, s)
        torch.cuda.synchronize()
        assert int(st_d.item()) == 0
        assert np.array_equal(bits(delta.cpu().numpy()), bits(want_delta)), rnd
        for w in range(workers):
            assert np.array_equal(bits(err_w_d[w].cpu().numpy()), bits(err_w[w])), (rnd, w)
