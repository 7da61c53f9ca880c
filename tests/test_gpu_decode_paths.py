"""GPU parity of decompress on both launch sequences at every stream density.

Decompress runs one of two launch sequences, chosen on entry by the caller's
path hint word: sparse (zero fill of y, then the stream's nonzero codes
written over it) or dense (the stream decoded chunk by chunk into per-tile
start records, then every 5120-value tile decoded and written once).  The
first kernel rewrites the word with this call's density class.  Streams and M
come from the CPU oracle; y must match the oracle's decompress bit for bit on
both sequences, on single tensors and ragged groups (tensors starting off a
16-byte and off a 4-element boundary, tensors of one to seven values, so that
one code byte spans several tensors), on sparse and dense streams, and on the
full BERT-large set at the error-feedback steady state; the hint word must
hold the density class afterwards; corrupt streams must set the status on
both sequences."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu

TILE = 5120
PATHS = (None, 0, 1)  # no hint word (sparse), a word holding 0, a word holding 1


def density_class(lens, Bs):
    """The class the device writes into the hint word: 1 when the streams
    (each counted up to its quartic length) exceed 0.104 bytes per quartic
    byte."""
    tl = sum(min(int(l), int(b)) for l, b in zip(lens, Bs))
    return 1 if 1000 * tl > 104 * sum(int(b) for b in Bs) else 0


def hint_word(path):
    if path is None:
        return None
    from gradient_compression_distributed_lc_amd import tlc
    h = tlc.path_hint()
    h[0] = path
    return h


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


def gpu_decompress(st, M, n, s, ws=None, path=None):
    # the stream sits at the start of a buffer of the compress capacity
    # ceil(n/5) (the binding requires it); the device length says how much of
    # it is the stream
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    buf = np.zeros(max(-(-n // 5), st.size), np.uint8)
    buf[:st.size] = st
    ind = to_dev(buf)
    lend = torch.tensor([st.size], dtype=torch.int64, device=ind.device)
    h = hint_word(path)
    y = torch.full((n,), 7.0, dtype=torch.float32, device=ind.device)
    y, status = tlc.decompress(ind, lend, to_dev(np.array([M], np.float32)), n, s, y=y, workspace=ws,
                               path_hint=h)
    torch.cuda.synchronize()
    if h is not None and int(status.item()) == 0:
        assert int(h[0]) == density_class([st.size], [-(-n // 5)]), (n, path)
    return y.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("n", [1, 4, 5, 6, 1023, 1024, 1025, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, 262_147,
                               1_000_003])
def test_single_sparse_and_dense(n):
    for dense in (False, True):
        for s in (1.0, 1.75):
            st, M = payload(n, n + 7 * dense, dense, s)
            want = bits(oracle.decompress(st, M, n, s))
            for path in PATHS:
                say(f"case decode n={n} dense={dense} s={s} path={path}")
                y, status = gpu_decompress(st, M, n, s, path=path)
                assert status == 0, (n, dense, s, path)
                assert np.array_equal(bits(y), want), (n, dense, s, path)


def group_case(sizes, dense_of, s, seed, paths=PATHS):
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    g = tlc.Group(sizes)
    N = sum(sizes)
    out = np.zeros(g.stream_bytes, np.uint8)
    lens = np.zeros(len(sizes), np.int64)
    Ms = np.zeros(len(sizes), np.float32)
    want = np.empty(N, np.float32)
    off = 0
    for t, n in enumerate(sizes):
        st, M = payload(n, seed + t, dense_of(t), s)
        out[g.offsets[t]:g.offsets[t] + st.size] = st
        lens[t], Ms[t] = st.size, M
        want[off:off + n] = oracle.decompress(st, M, n, s)
        off += n
    ind, lend, Md = to_dev(out), to_dev(lens), to_dev(Ms)
    for path in paths:
        y = torch.full((N,), 7.0, dtype=torch.float32, device="cuda:0")
        h = hint_word(path)
        y, status = g.decompress(ind, lend, Md, s, y=y, path_hint=h)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, path
        if h is not None:
            assert int(h[0]) == density_class(lens, [-(-n // 5) for n in sizes]), path
        got = bits(y.cpu().numpy())
        if not np.array_equal(got, bits(want)):
            i = int(np.flatnonzero(got != bits(want))[0])
            raise AssertionError(f"path {path}: y differs first at element {i}: {y[i].item()} vs {want[i]}")


def test_group_ragged_unaligned():
    rng = np.random.default_rng(77)
    sizes = [int(v) for v in rng.integers(1, 25_000, 70)] + [1, 3, TILE - 3, TILE + 2, 4 * TILE + 1, 200_003]
    for k, mode in enumerate(("sparse", "dense", "mixed")):
        say(f"case decode group ragged {mode}")
        group_case(sizes, lambda t: mode == "dense" or (mode == "mixed" and t % 3 == 0), 1.5, 1000 * k)


def test_group_of_tiny_tensors_spanning_code_bytes():
    # tensors of 1..7 values: one code byte and one 5120-value tile hold
    # several tensors
    rng = np.random.default_rng(5)
    for k in range(4):
        sizes = [int(v) for v in rng.integers(1, 8, 700)] + [int(v) for v in rng.integers(1, 3000, 5)]
        rng.shuffle(sizes)
        say(f"case decode tiny tensors {k}")
        group_case(sizes, lambda t: (t + k) % 2 == 0, 1.25, 50 + 1000 * k)


def test_group_block_boundaries():
    # tensors ending one element before, at and after multiples of 4 and of
    # 1024, and streams whose chunks end anywhere inside a code byte
    sizes = [1023, 1, 1024, 1025, 3, 4, 5, 2047, 2049, 4 * 4096 * 5 + 3, 4 * 4096 * 5, 17]
    for dense in (False, True):
        say(f"case decode block boundaries dense={dense}")
        group_case(sizes, lambda t: dense, 1.0, 300 + dense)


def test_corrupt_streams_set_status():
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
            for path in PATHS:
                say(f"case decode corrupt {name} dense={dense} path={path}")
                _, status = gpu_decompress(np.ascontiguousarray(buf), M, n, 1.0, path=path)
                assert status == tlc.ERR_CORRUPT, (name, dense, path)
        for path in PATHS:
            y, status = gpu_decompress(st, M, n, 1.0, path=path)
            assert status == 0
            assert np.array_equal(bits(y), bits(oracle.decompress(st, M, n, 1.0))), path


def test_density_changes_on_one_workspace_and_hint_word():
    # alternating sparse and dense streams on one workspace and one hint
    # word, no synchronisation between the calls: each call runs the
    # sequence the previous call's density chose (the first one sparse), the
    # workspace keeps the previous call's records, and every output is exact
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    n = 40 * TILE + 11
    B = -(-n // 5)
    ws = torch.empty(tlc.workspace_size(n), dtype=torch.uint8, device="cuda:0")
    h = tlc.path_hint()
    pattern = (False, True, True, False, False, True, False)
    cases = [payload(n, 300 + k, dense, 1.25) for k, dense in enumerate(pattern)]
    ys = []
    for k, (st, M) in enumerate(cases):
        buf = np.zeros(B, np.uint8)
        buf[:st.size] = st
        y = torch.full((n,), 7.0, dtype=torch.float32, device="cuda:0")
        lend = torch.tensor([st.size], dtype=torch.int64, device="cuda:0")
        ys.append(tlc.decompress(to_dev(buf), lend, to_dev(np.array([M], np.float32)), n, 1.25, y=y, workspace=ws,
                                 path_hint=h))
    torch.cuda.synchronize()
    assert int(h[0]) == density_class([cases[-1][0].size], [B])
    for k, ((st, M), (y, status)) in enumerate(zip(cases, ys)):
        say(f"case decode density switch {k} dense={pattern[k]}")
        assert int(status.item()) == 0, k
        assert np.array_equal(bits(y.cpu().numpy()), bits(oracle.decompress(st, M, n, 1.25))), k


@pytest.mark.timeout(600)
def test_bert_large_steady_state_streams():
    # the full 335M-value set after 150 steps of error feedback on the GPU
    # (inputs cycled through 4 rolled copies): every encode tile holds nonzero
    # codes.  The decompress of the final streams equals the oracle's decode
    # of the same streams, tensor by tensor.
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
    say(f"case decode bert_large steady: density {got_lens.sum() / B:.4f}")
    assert got_lens.sum() / B > 0.104  # the dense regime
    want = np.empty(N, np.float32)
    off = 0
    for t, n in enumerate(sizes):
        o = g.offsets[t]
        want[off:off + n] = oracle.decompress(got_out[o:o + got_lens[t]], got_M[t], n, s)
        off += n
    y = torch.empty(N, dtype=torch.float32, device="cuda:0")
    h = tlc.path_hint()
    for rep in range(3):  # sparse (the word starts at 0), then dense twice
        say(f"case decode bert_large steady, call {rep}, hint {int(h[0])}")
        assert int(h[0]) == (0 if rep == 0 else 1)
        y.fill_(7.0)
        _, st_d = g.decompress(out, lens, scales, s, y=y, workspace=ws, path_hint=h)
        torch.cuda.synchronize()
        assert int(st_d.item()) == 0
        assert int(h[0]) == 1
        assert np.array_equal(bits(y.cpu().numpy()), bits(want)), rep


def test_hint_word_must_be_pinned():
    # a hint word the device cannot reach is an argument error, before any
    # launch (the binding refuses it first; the raw C call returns the code)
    import ctypes
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    n = 1000
    st, M = payload(n, 1, False, 1.0)
    buf = np.zeros(-(-n // 5), np.uint8)
    buf[:st.size] = st
    ind = to_dev(buf)
    lend = torch.tensor([st.size], dtype=torch.int64, device="cuda:0")
    sd = to_dev(np.array([M], np.float32))
    with pytest.raises(ValueError):
        tlc.decompress(ind, lend, sd, n, 1.0, path_hint=torch.zeros(1, dtype=torch.int32))
    y = torch.empty(n, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(tlc.workspace_size(n), dtype=torch.uint8, device="cuda:0")
    status = torch.empty(1, dtype=torch.int32, device="cuda:0")
    word = (ctypes.c_uint32 * 1)(0)  # ordinary host memory
    P = ctypes.c_void_p
    rc = tlc.lib().tlc_decompress(P(ind.data_ptr()), P(lend.data_ptr()), P(sd.data_ptr()), n, 1.0,
                                  P(y.data_ptr()), P(ws.data_ptr()), ws.numel(), P(status.data_ptr()),
                                  ctypes.cast(word, P), None)
    assert rc == tlc.ERR_INVALID_ARG
    # and the library still works afterwards
    yy, status = gpu_decompress(st, M, n, 1.0, path=1)
    assert status == 0 and np.array_equal(bits(yy), bits(oracle.decompress(st, M, n, 1.0)))
