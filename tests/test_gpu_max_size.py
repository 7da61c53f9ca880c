"""GPU parity at the largest tensor the library takes: n = 2^32 - 1 fp32
values (16 GiB): compress (with a zero hint and with the exact M), decompress
on both launch sequences (sparse, and dense through a path hint word of 1),
accumulate, and the many-payload accumulate of the stream twice, through the
C ABI.

The input is a zero tensor with seeded spikes (first and last element
included), so the oracle's results are computed exactly without holding the
whole tensor on the host:
* with err = 0, v = x; M and every spike's code and new error come from the
  oracle's quantizer on a small array holding the spike values (its max is
  the tensor's M, so the threshold is the same);
* the expected stream is the oracle's zero-run encoding of the full quartic
  byte array (121 everywhere except the bytes that hold spike codes);
* everything else is checked by properties on the device: err, y and the
  accumulated sum are zero exactly where no spike has a nonzero code, and
  hold the oracle's values at the spikes."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say

pytestmark = pytest.mark.gpu

N_MAX = 2 ** 32 - 1


@pytest.mark.timeout(900)
def test_max_size_tensor():
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    n, s = N_MAX, 1.5
    rng = np.random.default_rng(2 ** 32 - 1)
    idx = np.unique(np.concatenate([[0, 1, 4, n - 1, n - 2, n - 5, 5 * 858_993_000],
                                    rng.integers(0, n, 300, dtype=np.int64)]))
    val = (rng.standard_normal(idx.size) * 1e-3).astype(np.float32)
    val[idx == n - 1] = np.float32(2.5e-3)  # the max sits on the last element
    say(f"case max size: n={n}, {idx.size} spikes")

    # oracle on the spike values: M, codes, new errors (zeros elsewhere stay 0)
    q_sp, M, e_sp = oracle.quantize(val, np.zeros_like(val), s)
    assert M == np.abs(val).max()
    B = -(-n // 5)
    qbytes = np.full(B, 121, np.uint8)
    for k in np.unique(idx // 5):
        b = 0
        for d in range(5):
            i = 5 * k + d
            j = np.searchsorted(idx, i)
            c = int(q_sp[j]) if j < idx.size and idx[j] == i else 0
            b += (c + 1) * 3 ** d
        qbytes[k] = b
    want_stream = oracle.zre_encode(qbytes)
    del qbytes
    say(f"case max size: oracle stream {want_stream.size} bytes")

    dev = torch.device("cuda:0")
    x = torch.zeros(n, dtype=torch.float32, device=dev)
    ti = torch.from_numpy(idx).to(dev)
    x[ti] = torch.from_numpy(val).to(dev)
    err = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = torch.empty(tlc.workspace_size(n), dtype=torch.uint8, device=dev)
    # twice from err = 0: a zero hint (the second pass reads err again), then
    # the exact M as the hint (the second pass reads the candidate lists)
    for hint in (0.0, float(M)):
        say(f"case max size: compress, hint {hint}")
        err.zero_()
        sc = torch.full((1,), hint, dtype=torch.float32, device=dev)
        c = tlc.compress(x, err, s, scale=sc, workspace=ws)
        torch.cuda.synchronize()
        assert int(c.status.item()) == 0
        assert np.float32(c.scale.item()) == M
        got = c.stream().cpu().numpy()
        assert got.size == want_stream.size and np.array_equal(got, want_stream)
        assert np.array_equal(bits(err[ti].cpu().numpy()), bits(e_sp))
        assert int(torch.count_nonzero(err).item()) == int(np.count_nonzero(e_sp))
    nz = q_sp != 0
    del x
    say("case max size: compress ok, decompress")

    y, st = tlc.decompress(c.out, c.out_len, c.scale, n, s, workspace=ws)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    # the oracle's decode of the spikes alone (their codes re-encoded as a small
    # stream); every other element decodes to +0.0
    small = oracle.zre_encode(oracle.quartic_pack(q_sp))
    want_y = oracle.decompress(small, M, val.size, s)
    assert np.array_equal(bits(y[ti].cpu().numpy()), bits(want_y))
    assert int(torch.count_nonzero(y).item()) == int(nz.sum())
    # the dense sequence on the same stream (its tile records hold 32-bit
    # byte offsets within the tensor, largest here): the same y; the device
    # then writes the stream's class (sparse) into the hint word
    say("case max size: decompress ok, dense sequence")
    y.fill_(1.0)
    h = tlc.path_hint()
    h[0] = 1
    y, st = tlc.decompress(c.out, c.out_len, c.scale, n, s, y=y, workspace=ws, path_hint=h)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert int(h[0]) == 0
    assert np.array_equal(bits(y[ti].cpu().numpy()), bits(want_y))
    assert int(torch.count_nonzero(y).item()) == int(nz.sum())
    del y
    say("case max size: dense decompress ok, accumulate")

    acc = err  # reuse the 16 GiB buffer: acc starts as the new error
    _, st = tlc.decompress_accumulate(c.out, c.out_len, c.scale, n, s, acc)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    # the oracle's accumulate over the spikes alone: elements without a spike
    # hold 0 and get nothing added
    exp = oracle.decompress_accumulate(small, M, val.size, s, e_sp.copy())
    assert np.array_equal(bits(acc[ti].cpu().numpy()), bits(exp))
    assert int(torch.count_nonzero(acc).item()) == int(np.count_nonzero(exp))

    # the many-payload accumulate at the same size: the stream twice, as two
    # payloads (the second one's bytes start ~859 MB into the buffer, and its
    # tile records follow the first one's 838,861)
    say("case max size: accumulate ok")
    B = tlc.compress_bound(n)
    stride = -(-B // 16) * 16
    two = torch.empty(2 * stride, dtype=torch.uint8, device=dev)
    two[:B].copy_(c.out[:B])
    two[stride:stride + B].copy_(c.out[:B])
    g = tlc.Group([n], device=dev)
    lens2 = torch.cat([c.out_len, c.out_len])
    scales2 = torch.cat([c.scale, c.scale])
    for route in (None, 0):  # one pass over acc; one add pass per payload
        say(f"case max size: two payloads in one call, sequence {route}")
        h = None
        if route is not None:
            h = tlc.path_hint()
            h[0] = route
        _, st = g.decompress_accumulate_many(two.view(2, stride), lens2, scales2, s, acc, path_hint=h)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for _ in range(2):
            exp = oracle.decompress_accumulate(small, M, val.size, s, exp)
        assert np.array_equal(bits(acc[ti].cpu().numpy()), bits(exp))
        assert int(torch.count_nonzero(acc).item()) == int(np.count_nonzero(exp))
