"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (grouped calls over the whole gradient set):

* single_1m    one compress + decompress, s = 1.0
* single_16m   10 steps with fresh inputs (seed 200+t) and the error carried, s = 1.5
* resnet110    329 tensors, one grouped compress + decompress, s = 1.9
* resnet50     161 tensors, s in {1.0, 1.5, 1.9}, error reset for each s
* bert_large   391 tensors, workers 0..7 (seed 500+w) each compressed from a
               zero error buffer, then the 8 payloads decompress-accumulated in
               order into one fp32 sum (one call per payload, and all eight in
               one many-payload call), and the server's compress of their mean

Everything is compared bit for bit with the CPU oracle: every tensor's stream
and length, M, the error buffer, the decompressed values and the sum.  The
scale buffer each compress reads as its hint is set on purpose: zeros (the
second pass reads the error buffer again) or the previous M (the second pass
reads the first pass's candidate lists), so both paths run at full size."""
import numpy as np
import pytest

import oracle
from gradient_compression_distributed_lc_amd import workloads

from gpu_util import bits, check_group, check_single, oracle_group_compress, say, to_dev

pytestmark = pytest.mark.gpu


def test_single_1m():
    x = workloads.generate("single_1m")
    say("case single_1m")
    got = check_single(x, np.zeros_like(x), 1.0, acc=np.zeros_like(x), label="single_1m")
    say(f"single_1m bits/value {8 * got['L'] / x.size:.4f}")
    say("case single_1m, previous-M hint")
    check_single(x, np.zeros_like(x), 1.0, acc=np.zeros_like(x), label="single_1m hint", hint=float(got["M"]))


@pytest.mark.timeout(600)
def test_single_16m_ten_steps_with_error_feedback():
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    w = workloads.get("single_16m")
    n, s = w.total, w.s_values[0]
    e_cpu = np.zeros(n, np.float32)
    ed = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    sc = torch.zeros(1, dtype=torch.float32, device="cuda:0")  # carried: step t reads step t-1's M
    for t in range(10):
        x = workloads.generate("single_16m", step=t)
        say(f"case single_16m step {t}")
        st, M, e_cpu = oracle.compress(x, e_cpu, s)
        c = tlc.compress(to_dev(x), ed, s, scale=sc)
        y, st_d = tlc.decompress(c.out, c.out_len, c.scale, n, s)
        torch.cuda.synchronize()
        assert int(c.status.item()) == 0 and int(st_d.item()) == 0
        assert np.float32(c.scale.item()) == M
        assert np.array_equal(c.stream().cpu().numpy(), st), t
        assert np.array_equal(bits(ed.cpu().numpy()), bits(e_cpu)), t
        assert np.array_equal(bits(y.cpu().numpy()), bits(oracle.decompress(st, M, n, s))), t
        say(f"single_16m step {t} bits/value {8 * st.size / n:.4f}")


def test_resnet110_group():
    from gradient_compression_distributed_lc_amd import tlc
    w = workloads.get("resnet110")
    g = tlc.Group(w.sizes)
    x = workloads.generate("resnet110")
    say("case resnet110")
    _, _, scales, _ = check_group(g, x, np.zeros_like(x), w.s_values[0], label="resnet110")
    say("case resnet110, previous-M hint")
    check_group(g, x, np.zeros_like(x), w.s_values[0], label="resnet110 hint", hint=scales.cpu().numpy())


@pytest.mark.timeout(600)
def test_resnet50_group_s_sweep():
    from gradient_compression_distributed_lc_amd import tlc
    w = workloads.get("resnet50")
    g = tlc.Group(w.sizes)
    x = workloads.generate("resnet50")
    hint = None  # zeros for the first s, then the M the previous s found (the same x)
    for s in w.s_values:
        say(f"case resnet50 s={s}")
        _, _, scales, _ = check_group(g, x, np.zeros_like(x), s, label=f"resnet50 s={s}", hint=hint)
        hint = scales.cpu().numpy()


@pytest.mark.timeout(1200)
def test_bert_large_eight_workers_accumulate():
    import torch
    from gradient_compression_distributed_lc_amd import tlc
    w = workloads.get("bert_large")
    s, sizes, N = w.s_values[0], w.sizes, w.total
    g = tlc.Group(sizes)
    acc_d = torch.zeros(N, dtype=torch.float32, device="cuda:0")
    acc_h = np.zeros(N, np.float32)
    x = np.empty(N, np.float32)
    ws = g.workspace()
    pay = torch.empty((8, g.stream_bytes), dtype=torch.uint8, device="cuda:0")  # the 8 workers' payloads
    pay_lens = torch.empty((8, len(sizes)), dtype=torch.int64, device="cuda:0")
    pay_scales = torch.empty((8, len(sizes)), dtype=torch.float32, device="cuda:0")
    hint = None  # worker 0: zeros; worker w > 0: worker w-1's M
    for wk in range(8):
        say(f"case bert_large worker {wk}: generate")
        workloads.generate("bert_large", worker=wk, out=x)
        zero = np.zeros(N, np.float32)
        want = oracle_group_compress(x, zero, sizes, s)
        say(f"case bert_large worker {wk}: compress/decompress parity")
        out, lens, scales, (streams, Ms) = check_group(g, x, zero, s, label=f"bert_large worker {wk}", want=want,
                                                       hint=hint)
        hint = Ms
        pay[wk].copy_(out)
        pay_lens[wk].copy_(lens)
        pay_scales[wk].copy_(scales)
        _, st = g.decompress_accumulate(out, lens, scales, s, acc_d, workspace=ws)
        off = 0
        for t, n in enumerate(sizes):
            oracle.decompress_accumulate(streams[t], Ms[t], n, s, acc_h[off:off + n])
            off += n
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        del out, lens, scales
    say("case bert_large: 8-payload sum")
    assert np.array_equal(bits(acc_d.cpu().numpy()), bits(acc_h))
    # the same eight payloads in one many-payload call from a zero sum, on
    # both launch sequences (one pass over the sum; one add pass per payload)
    acc_m = torch.zeros(N, dtype=torch.float32, device="cuda:0")
    for route in (1, 0):
        say(f"case bert_large: 8 payloads in one call, sequence {route}")
        acc_m.zero_()
        h = tlc.path_hint()
        h[0] = route
        _, st = g.decompress_accumulate_many(pay, pay_lens.view(-1), pay_scales.view(-1), s, acc_m, path_hint=h)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert np.array_equal(bits(acc_m.cpu().numpy()), bits(acc_h)), route
        assert int(h[0]) == 0  # first-step payloads are sparse
    del acc_m, pay
    # model-delta direction: the server compresses the workers' mean with its
    # own (zero) error buffer; every tensor's stream, M and error bit for bit
    say("case bert_large: server compress of the 8-worker mean")
    err_d = torch.zeros(N, dtype=torch.float32, device="cuda:0")
    out, lens, scales, st = g.server_compress(acc_d, 8, err_d, s, workspace=ws,
                                              scales=torch.zeros(len(sizes), dtype=torch.float32, device="cuda:0"))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got_out, got_lens, got_M = out.cpu().numpy(), lens.cpu().numpy(), scales.cpu().numpy()
    got_err = bits(err_d.cpu().numpy())
    off = 0
    for t, n in enumerate(sizes):
        want_st, want_M, want_e = oracle.server_compress(acc_h[off:off + n], 8, np.zeros(n, np.float32), s)
        o, L = g.offsets[t], int(got_lens[t])
        assert got_M[t] == want_M, t
        assert L == want_st.size and np.array_equal(got_out[o:o + L], want_st), t
        assert np.array_equal(got_err[off:off + n], bits(want_e)), t
        off += n
