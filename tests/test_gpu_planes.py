"""GPU parity of the five-plane byte layout (byte k of a tensor holds elements
k + jB, j = 0..4): tlc_planes_gather, the grouped codec on the plan of sizes
5*ceil(n/5), and tlc_planes_scatter, against the oracle's compress_planes and
decompress_planes, bit for bit (stream bytes and lengths, M, error buffer, y)
over error-feedback steps."""
import numpy as np
import pytest

import oracle

from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu


def test_planes_group_matches_oracle():
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    rng = np.random.default_rng(55)
    sizes = [1, 2, 3, 4, 5, 6, 7, 11, 5119, 5120, 5121, 70_001, 131_072] + \
        [int(v) for v in rng.integers(1, 40_000, 20)]
    padded = [5 * (-(-n // 5)) for n in sizes]
    g, gp = tlc.Group(sizes), tlc.Group(padded)
    N, NP, s = g.total, gp.total, 1.5
    dev = torch.device("cuda:0")
    src_off = torch.tensor(g.elem_offsets[:-1], dtype=torch.int64, device=dev)
    dst_off = torch.tensor(gp.elem_offsets[:-1], dtype=torch.int64, device=dev)
    nv = torch.tensor(sizes, dtype=torch.int64, device=dev)
    err = torch.zeros(N, dtype=torch.float32, device=dev)
    err_h = np.zeros(N, np.float32)
    xp = torch.empty(NP, dtype=torch.float32, device=dev)
    ep = torch.empty(NP, dtype=torch.float32, device=dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    ws = gp.workspace()
    for step in range(3):
        say(f"case planes step {step}")
        x = (rng.standard_normal(N) * 1e-3).astype(np.float32)
        x[rng.random(N) < 0.3] = 0
        xd = to_dev(x)
        tlc.planes_gather(xd, src_off, xp, dst_off, nv, max(sizes))
        tlc.planes_gather(err, src_off, ep, dst_off, nv, max(sizes))
        out, lens, scales, st = gp.compress(xp, ep, s, workspace=ws)
        tlc.planes_scatter(ep, dst_off, err, src_off, nv, max(sizes))
        yp, st_d = gp.decompress(out, lens, scales, s, workspace=ws)
        tlc.planes_scatter(yp, dst_off, y, src_off, nv, max(sizes))
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and int(st_d.item()) == 0
        got_out, got_lens, got_M = out.cpu().numpy(), lens.cpu().numpy(), scales.cpu().numpy()
        got_err, got_y = err.cpu().numpy(), y.cpu().numpy()
        for t, n in enumerate(sizes):
            a, b = g.elem_offsets[t], g.elem_offsets[t + 1]
            stream, M, e_new = oracle.compress_planes(x[a:b], err_h[a:b], s)
            o = gp.offsets[t]
            assert got_lens[t] == stream.size and np.array_equal(got_out[o:o + stream.size], stream), (step, t, n)
            assert bits(np.array([got_M[t]]))[0] == bits(np.array([M]))[0], (step, t)
            assert np.array_equal(bits(got_err[a:b]), bits(e_new)), (step, t)
            assert np.array_equal(bits(got_y[a:b]), bits(oracle.decompress_planes(stream, M, n, s))), (step, t)
            err_h[a:b] = e_new
