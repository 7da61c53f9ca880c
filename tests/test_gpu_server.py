"""GPU parity of the model-delta direction (3LC page, "Proposed method",
fourth item): the server compresses the mean of the workers' decoded payloads
(acc / workers, fp32 IEEE divide) with its own error buffer.  The HIP path
(tlc_server_compress, tlc_server_compress_group through the C ABI) is
compared bit for bit with the CPU oracle: stream bytes and length, M and the
server's error buffer, over several rounds with the error carried."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu

TILE = 5120


def worker_sum(n, workers, seed, s=1.75, zeros=0.3):
    """The server's acc: the fp32 sum of `workers` decoded payloads (oracle)."""
    rng = np.random.default_rng(seed)
    acc = np.zeros(n, np.float32)
    for _ in range(workers):
        x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        x[rng.random(n) < zeros] = 0
        st, M, _ = oracle.compress(x, np.zeros(n, np.float32), s)
        oracle.decompress_accumulate(st, M, n, s, acc)
    return acc


def check_server_single(acc, workers, err, s, label):
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    want_st, want_M, want_err = oracle.server_compress(acc, workers, err, s)
    ed = to_dev(err)
    c = tlc.server_compress(to_dev(acc), workers, ed, s)
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0, label
    assert np.float32(c.scale.item()) == want_M, (label, c.scale.item(), want_M)
    got = c.stream().cpu().numpy()
    assert got.size == want_st.size and np.array_equal(got, want_st), label
    assert np.array_equal(bits(ed.cpu().numpy()), bits(want_err)), label
    return want_err


@pytest.mark.parametrize("n", [1, 7, TILE - 1, 3 * TILE + 2, 262_147])
def test_server_compress_single(n):
    for workers in (1, 2, 3, 7, 8):
        for s in (1.0, 1.75):
            say(f"case server n={n} workers={workers} s={s}")
            acc = worker_sum(n, min(workers, 4), seed=n + workers)
            rng = np.random.default_rng(workers)
            err = (rng.standard_normal(n) * 1e-4).astype(np.float32)
            check_server_single(acc, workers, err, s, f"n={n} w={workers} s={s}")


def test_server_compress_special_values():
    # quotients that are subnormal, -0.0 sums, ties of the mean against M*s/2
    acc = np.array([3e-38, -1e-39, -0.0, 0.0, 6.0, -3.0, 1.5, 2.9999998, 3.0000002] * 5, np.float32)
    for workers in (1, 2, 3, 6, 8, 16, 1024):
        for s in (1.0, 1.5, 1.99):
            say(f"case server special workers={workers} s={s}")
            check_server_single(acc, workers, np.zeros_like(acc), s, f"special w={workers} s={s}")


def test_server_rounds_group():
    # three rounds of: 8 workers' payloads summed by the server, server compress
    # with its error carried; ragged tensors with unaligned starts
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(42)
    sizes = [int(v) for v in rng.integers(1, 40_000, 60)] + [1, 5, TILE, 2 * TILE + 3, 300_001]
    g = tlc.Group(sizes)
    N = sum(sizes)
    workers, s = 8, 1.75
    err_h = np.zeros(N, np.float32)
    err_d = torch.zeros(N, dtype=torch.float32, device="cuda:0")
    for rnd in range(3):
        say(f"case server group round {rnd}")
        acc = worker_sum(N, 3, seed=900 + rnd)
        out, lens, scales, st = g.server_compress(to_dev(acc), workers, err_d, s)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        got_out, got_lens, got_M = out.cpu().numpy(), lens.cpu().numpy(), scales.cpu().numpy()
        off = 0
        for t, n in enumerate(sizes):
            want_st, want_M, e = oracle.server_compress(acc[off:off + n], workers, err_h[off:off + n], s)
            err_h[off:off + n] = e
            o, L = g.offsets[t], int(got_lens[t])
            assert got_M[t] == want_M, (rnd, t)
            assert L == want_st.size and np.array_equal(got_out[o:o + L], want_st), (rnd, t, n)
            off += n
        assert np.array_equal(bits(err_d.cpu().numpy()), bits(err_h)), rnd
