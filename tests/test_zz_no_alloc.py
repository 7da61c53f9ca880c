"""GPU test of tlc_compress_static, the compress for callers that cannot
allocate: through the C ABI, two calls in a row (the second on a smaller
tensor, so the fixed scratch array holds the first call's contents), each
compared bit for bit with tlc_compress on a caller workspace and with the CPU
oracle: stream bytes, length, M, the new error buffer and the status."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    x[rng.random(n) < 0.3] = 0.0
    err = (rng.standard_normal(n) * 2e-4).astype(np.float32)
    return x, err


def test_static_compress_matches_workspace_compress():
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    assert tlc.compress_static_max_n() == 1 << 24
    dev = torch.device("cuda:0")
    for k, (n, s) in enumerate(((1 << 24, 1.75), (1_234_567, 1.5), (3 * 5120 + 11, 1.25))):
        say(f"case no-alloc call {k}: n={n} s={s}")
        x, err = _inputs(n, 40 + k)
        want_st, want_M, want_e = oracle.compress(x, err, s)
        xd = to_dev(x)
        # the existing entry point on a caller workspace
        e_ws = to_dev(err)
        ref = tlc.compress(xd, e_ws, s, scale=torch.zeros(1, dtype=torch.float32, device=dev))
        # the fixed-scratch entry point, every buffer passed in
        e_st = to_dev(err)
        out = torch.empty(tlc.compress_bound(n), dtype=torch.uint8, device=dev)
        out_len = torch.empty(1, dtype=torch.int64, device=dev)
        scale = torch.zeros(1, dtype=torch.float32, device=dev)
        status = torch.full((1,), 99, dtype=torch.int32, device=dev)
        got = tlc.compress_static(xd, e_st, s, out=out, out_len=out_len, scale=scale, status=status)
        torch.cuda.synchronize()
        assert int(ref.status.item()) == 0 and int(got.status.item()) == 0
        L = int(got.out_len.item())
        assert L == int(ref.out_len.item()) == want_st.size
        assert np.array_equal(got.out[:L].cpu().numpy(), ref.out[:L].cpu().numpy())
        assert np.array_equal(got.out[:L].cpu().numpy(), want_st)
        assert np.float32(got.scale.item()) == np.float32(ref.scale.item()) == want_M
        assert np.array_equal(bits(e_st.cpu().numpy()), bits(e_ws.cpu().numpy()))
        assert np.array_equal(bits(e_st.cpu().numpy()), bits(want_e))
    # n above the maximum is refused before anything is enqueued
    small = torch.zeros(16, dtype=torch.float32, device=dev)
    rc = tlc.lib().tlc_compress_static(tlc._ptr(small), tlc._ptr(small), (1 << 24) + 1, 1.5, tlc._ptr(small),
                                       1 << 30, tlc._ptr(small), tlc._ptr(small), tlc._ptr(small), None)
    assert rc == tlc.ERR_TOO_LARGE
