"""GPU parity of both decompress launch sequences (tlc_set_decode_policy):
the sparse one (zero fill, then the nonzero codes written over it) and the
dense one (tile starts recorded while parsing, then every encode tile decoded
in LDS and written once), and of the automatic choice between them.  Streams
and M come from the CPU oracle; y must match the oracle's decompress bit for
bit, on single tensors and ragged groups (tensors starting off a 16-byte
boundary), on sparse and dense streams, and corrupt streams must set the
status under every policy."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu

TILE = 5120
POLICIES = ("sparse", "dense", "auto")


@pytest.fixture(params=POLICIES)
def policy(request):
    from gradient_compression_distributed_lc_amd import tlc
    code = {"sparse": tlc.DECODE_SPARSE, "dense": tlc.DECODE_DENSE, "auto": tlc.DECODE_AUTO}[request.param]
    tlc.set_decode_policy(code)
    yield request.param
    tlc.set_decode_policy(tlc.DECODE_AUTO)


def payload(n, seed, dense, s):
    """An oracle stream: dense ones carry an error buffer near the threshold,
    so that most quartic bytes hold a nonzero code."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    if dense:
        e = (rng.uniform(-1, 1, n) * 3e-3).astype(np.float32)
    else:
        e = np.zeros(n, np.float32)
        x[rng.random(n) < 0.3] = 0
    st, M, _ = oracle.compress(x, e, s)
    return st, M


def gpu_decompress(st, M, n, s, ws=None):
    # the stream sits at the start of a buffer of the compress capacity
    # ceil(n/5) (the binding requires it); the device length says how much of
    # it is the stream
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    buf = np.zeros(max(-(-n // 5), st.size), np.uint8)
    buf[:st.size] = st
    ind = to_dev(buf)
    lend = torch.tensor([st.size], dtype=torch.int64, device=ind.device)
    y, status = tlc.decompress(ind, lend, to_dev(np.array([M], np.float32)), n, s, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("n", [1, 4, 5, 6, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, 262_147, 1_000_003])
def test_single_sparse_and_dense(policy, n):
    for dense in (False, True):
        for s in (1.0, 1.75):
            say(f"case decode path {policy} n={n} dense={dense} s={s}")
            st, M = payload(n, n + 7 * dense, dense, s)
            y, status = gpu_decompress(st, M, n, s)
            assert status == 0, (n, dense, s)
            assert np.array_equal(bits(y), bits(oracle.decompress(st, M, n, s))), (n, dense, s)


def test_group_ragged_unaligned(policy):
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(77)
    sizes = [int(v) for v in rng.integers(1, 25_000, 70)] + [1, 3, TILE - 3, TILE + 2, 4 * TILE + 1, 200_003]
    g = tlc.Group(sizes)
    N = sum(sizes)
    for dense in (False, True, False):
        s = 1.5
        say(f"case decode path {policy} group dense={dense}")
        out = np.zeros(g.stream_bytes, np.uint8)
        lens = np.zeros(len(sizes), np.int64)
        Ms = np.zeros(len(sizes), np.float32)
        want = np.empty(N, np.float32)
        off = 0
        for t, n in enumerate(sizes):
            st, M = payload(n, 1000 * dense + t, dense, s)
            out[g.offsets[t]:g.offsets[t] + st.size] = st
            lens[t], Ms[t] = st.size, M
            want[off:off + n] = oracle.decompress(st, M, n, s)
            off += n
        y, status = g.decompress(to_dev(out), to_dev(lens), to_dev(Ms), s)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(bits(y.cpu().numpy()), bits(want)), dense


def test_corrupt_streams_set_status(policy):
    from gradient_compression_distributed_lc_amd import tlc
    n = 3 * TILE + 7
    for dense in (False, True):
        st, M = payload(n, 5, dense, 1.0)
        B = -(-n // 5)
        good = np.zeros(B, np.uint8)
        good[:st.size] = st
        bad = good.copy()
        bad[0] = 255 if good[0] != 255 else 0
        cases = {"truncated": good[:st.size - 1], "edited": bad[:st.size], "overrun": np.full(B, 255, np.uint8),
                 "empty": good[:0], "too-long": good[:min(B, st.size + 1)] if st.size < B else None}
        for name, buf in cases.items():
            if buf is None:
                continue
            say(f"case decode path {policy} corrupt {name} dense={dense}")
            _, status = gpu_decompress(np.ascontiguousarray(buf), M, n, 1.0)
            assert status == tlc.ERR_CORRUPT, (name, dense)
        y, status = gpu_decompress(st, M, n, 1.0)
        assert status == 0
        assert np.array_equal(bits(y), bits(oracle.decompress(st, M, n, 1.0)))


def test_auto_follows_density_on_one_workspace():
    # alternating sparse and dense streams on one workspace: AUTO switches
    # paths from call to call (one call behind) and every output is exact
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    n = 40 * TILE + 11
    ws = torch.empty(tlc.workspace_size(n), dtype=torch.uint8, device="cuda:0")
    tlc.set_decode_policy(tlc.DECODE_AUTO)
    for k, dense in enumerate((False, True, True, False, False, True)):
        say(f"case decode path auto switch {k} dense={dense}")
        st, M = payload(n, 300 + k, dense, 1.25)
        y, status = gpu_decompress(st, M, n, 1.25, ws=ws)
        assert status == 0
        assert np.array_equal(bits(y), bits(oracle.decompress(st, M, n, 1.25))), k


@pytest.mark.timeout(600)
def test_bert_large_steady_state_streams_both_paths():
    # the full 335M-value set after 150 steps of error feedback on the GPU
    # (inputs cycled through 4 rolled copies): every encode tile holds nonzero
    # codes, so AUTO takes the dense path.  Both paths decode the final streams
    # to the oracle's decode of the same streams, tensor by tensor.
    import torch
    from gradient_compression_distributed_lc_amd import tlc, workloads
    w = workloads.get("bert_large")
    sizes, N, s = w.sizes, w.total, w.s_values[0]
    g = tlc.Group(sizes)
    x0 = to_dev(workloads.generate("bert_large"))
    xs = [x0] + [torch.roll(x0, k * 1_000_003) for k in range(1, 4)]
    err = torch.zeros(N, dtype=torch.float32, device="cuda:0")
    ws = g.workspace()
    out = torch.empty(g.stream_bytes, dtype=torch.uint8, device="cuda:0")
    lens = torch.empty(len(sizes), dtype=torch.int64, device="cuda:0")
    scales = torch.zeros(len(sizes), dtype=torch.float32, device="cuda:0")
    st = torch.empty(1, dtype=torch.int32, device="cuda:0")
    for k in range(150):
        g.compress(xs[k % 4], err, s, out=out, out_lens=lens, scales=scales, workspace=ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got_out, got_lens, got_M = out.cpu().numpy(), lens.cpu().numpy(), scales.cpu().numpy()
    B = sum(-(-n // 5) for n in sizes)
    say(f"case decode path bert_large steady: density {got_lens.sum() / B:.4f}")
    assert got_lens.sum() / B > 0.104  # the dense regime
    want = np.empty(N, np.float32)
    off = 0
    for t, n in enumerate(sizes):
        o = g.offsets[t]
        want[off:off + n] = oracle.decompress(got_out[o:o + got_lens[t]], got_M[t], n, s)
        off += n
    y = torch.empty(N, dtype=torch.float32, device="cuda:0")
    for pol in (tlc.DECODE_DENSE, tlc.DECODE_SPARSE, tlc.DECODE_AUTO, tlc.DECODE_AUTO):
        say(f"case decode path bert_large steady policy {pol}")
        tlc.set_decode_policy(pol)
        try:
            y.fill_(7.0)
            _, st_d = g.decompress(out, lens, scales, s, y=y, workspace=ws)
            torch.cuda.synchronize()
        finally:
            tlc.set_decode_policy(tlc.DECODE_AUTO)
        assert int(st_d.item()) == 0
        assert np.array_equal(bits(y.cpu().numpy()), bits(want)), pol
