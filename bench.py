"""Benchmark of the 3LC codec hot path on one MI355X.

One step = one worker's grouped compress of a whole gradient set (error
accumulation, per-tensor scale, ternary quantization, quartic packing,
zero-run encoding) followed by the grouped decompress of that payload
(zero-run decoding, quartic decoding, dequantization).  The error buffer is
carried from step to step, as in training, and every step sees a different
gradient set (the generated set rotated by k * 1,000,003 elements).  Inputs
are generated once on the host (seeded, synthetic) and are resident in HBM
before timing starts.

Default workload: the BERT-large gradient set (391 tensors, 335,141,888
fp32 values, 30% exact zeros, the rest N(0, 1e-4)), s = 1.75.

Printed: one JSON line with the whole-job throughput in GB/s of fp32 input
(4 bytes x values / (compress + decompress time)), the roofline of the
dominant kernel (the 12-byte/element pass over x and err) measured with HIP
events inside the timed region, bits per value, and the CPU oracle timed on
the host over the same workload (single-threaded, and as independent
per-tensor calls over up to 16 host cores).  Also reported, outside the timed steps:
compress and decompress timed apart, the 8-payload accumulate, the same
step after --steady-steps steps of error feedback (the error buffer then
keeps every encode tile active and the streams are about twice as dense),
the model-delta direction's server step (the workers' sum, then the
compress of their mean with the server's error buffer), and the ablations:
the same codes as quartic bytes only and as 2-bit fields (no zero-run
encoding), with the zero-run gain of the first step; and the same steps
pipelined over two streams (the decompress of payload k-1 while batch k is
compressed).

    python bench.py [--steps K] [--warmup W] [--workload bert_large] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
DOMINANT = "tlc_accum_max"      # reads x and err, writes err: 12 B per element
DOMINANT_BYTES_PER_ELEM = 12
METRIC = "3LC compress+decompress GB/s (fp32 in) and % of HBM roofline; bits/value"


def kernel_source_hash(kernel: str = "k_accum_max") -> str:
    """Hash of one kernel's source text (from its signature to the closing
    brace at column 0), of the candidate-bound helper it calls and of every
    file-scope constant (code only, without comments or spacing), so that
    counters taken on it stay valid while other kernels change, and are
    dropped once it or a constant changes."""
    with open(os.path.join(ROOT, "gradient_compression_distributed_lc_amd", "csrc", "tlc.hip")) as f:
        src = f.read()
    parts = []
    for sig in (f"void {kernel}(", "float cand_bound("):
        i = src.index(sig)
        parts.append(src[i:src.index("\n}\n", i)])
    parts += ["".join(ln.split("//")[0].split()) for ln in src.splitlines() if ln.startswith("constexpr ")]
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload, {}).get(DOMINANT)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(x: np.ndarray, sizes, s: float, passes: int):
    """The oracle, untuned, single-threaded, over the whole workload."""
    import oracle
    from gradient_compression_distributed_lc_amd import workloads
    offs = workloads.offsets(sizes)
    streams, Ms = [], []
    tc = td = 0.0
    y = np.empty(max(sizes), dtype=np.float32)
    err0 = None
    for p in range(passes):
        err = np.zeros(x.size, dtype=np.float32)
        cur_streams, cur_M = [], []
        t0 = time.perf_counter()
        for t, n in enumerate(sizes):
            out = np.empty(-(-n // 5), dtype=np.uint8)
            L, M = oracle.compress_inplace(x[offs[t]:offs[t + 1]], err[offs[t]:offs[t + 1]], s, out)
            cur_streams.append(out[:L])
            cur_M.append(M)
        t1 = time.perf_counter()
        for t, n in enumerate(sizes):
            oracle.decompress(cur_streams[t], cur_M[t], n, s, out=y[:n])
        t2 = time.perf_counter()
        tc += t1 - t0
        td += t2 - t1
        if p == 0:
            streams, Ms, err0 = cur_streams, cur_M, err
    elems = passes * x.size
    return {
        "value": round(4.0 * elems / (tc + td) / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"whole workload ({len(sizes)} tensors, {x.size} values), {passes} pass(es) of "
                  f"compress+decompress, single-threaded C oracle",
        "compress_s": round(tc / passes, 3),
        "decompress_s": round(td / passes, 3),
    }, streams, Ms, err0


def cpu_baseline_all_cores(x: np.ndarray, sizes, s: float, passes: int):
    """The same oracle, untouched, as independent per-tensor units spread over
    the host's cores (a thread pool; each call into the C oracle runs outside
    the interpreter lock).  Largest tensors are started first."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from gradient_compression_distributed_lc_amd import workloads
    offs = workloads.offsets(sizes)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(avail, 16))
    order = sorted(range(len(sizes)), key=lambda t: -sizes[t])
    oracle.lib()  # built and loaded before the clock starts
    outs = [np.empty(-(-n // 5), dtype=np.uint8) for n in sizes]
    ys = [np.empty(n, dtype=np.float32) for n in sizes]

    def unit(t, err):
        a, b = offs[t], offs[t + 1]
        L, M = oracle.compress_inplace(x[a:b], err[a:b], s, outs[t])
        oracle.decompress(outs[t][:L], M, sizes[t], s, out=ys[t])

    total = 0.0
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for _ in range(passes):
            err = np.zeros(x.size, dtype=np.float32)
            t0 = time.perf_counter()
            list(pool.map(lambda t: unit(t, err), order))
            total += time.perf_counter() - t0
    return {
        "value": round(4.0 * passes * x.size / total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"whole workload, {passes} pass(es) of compress+decompress, one oracle call per tensor "
                  f"on a pool of {threads} threads ({avail} cores available)",
        "host_cpu": host_cpu_model(),
    }


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bert_large")
    ap.add_argument("--s", type=float, default=None)
    ap.add_argument("--cpu-passes", type=int, default=8, help="oracle passes over the workload (about 10-15 s)")
    ap.add_argument("--pool", type=int, default=32, help="distinct gradient sets cycled through (HBM: 4 B/value each)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--no-copy", action="store_true", help="skip the copy-bandwidth yardstick")
    ap.add_argument("--steady-steps", type=int, default=150,
                    help="error-feedback steps before the steady-state figure (0: skip it)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the codec runs on one device and this build has no "
              "multi-GPU exchange; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from gradient_compression_distributed_lc_amd import tlc, workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.get(args.workload)
    s = args.s if args.s is not None else wl.s_values[0]
    sizes = wl.sizes
    N = wl.total

    t_gen = time.perf_counter()
    x_host = workloads.generate(args.workload)
    print(f"[bench] generated {args.workload}: {len(sizes)} tensors, {N} values in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    group = tlc.Group(sizes, device=dev)
    x0 = torch.from_numpy(x_host).to(dev)
    # A training step sees a fresh gradient: step k compresses the gradient set
    # rotated by k * 1,000,003 elements (same distribution, different values),
    # so the error buffer evolves as it does in training.  Repeating one
    # gradient instead makes the buffer pile up and is not the workload.
    pool = max(1, min(args.steps + args.warmup, args.pool))
    xs = [x0] + [torch.roll(x0, shifts=k * 1_000_003) for k in range(1, pool)]
    ed = torch.zeros(N, dtype=torch.float32, device=dev)
    yd = torch.empty(N, dtype=torch.float32, device=dev)
    out = torch.empty(group.stream_bytes, dtype=torch.uint8, device=dev)
    lens = torch.empty(len(sizes), dtype=torch.int64, device=dev)
    scales = torch.empty(len(sizes), dtype=torch.float32, device=dev)
    st_c = torch.empty(1, dtype=torch.int32, device=dev)
    st_d = torch.empty(1, dtype=torch.int32, device=dev)
    ws = group.workspace()

    counter = [0]

    def step():
        xd = xs[counter[0] % pool]
        counter[0] += 1
        group.compress(xd, ed, s, out=out, out_lens=lens, scales=scales, workspace=ws, status=st_c)
        group.decompress(out, lens, scales, s, y=yd, workspace=ws, status=st_d)

    # first step from a zero error buffer on the unrotated set: kept for the parity check
    step()
    torch.cuda.synchronize()
    first = {"out": out.cpu().numpy(), "lens": lens.cpu().numpy(), "scales": scales.cpu().numpy(),
             "err": ed.cpu().numpy(), "status": (int(st_c.item()), int(st_d.item()))}
    for _ in range(max(args.warmup - 1, 0)):
        step()
    torch.cuda.synchronize()
    # the state the timed steps start from, for the pipelined measurement below
    e_warm, c_warm, sc_warm = ed.clone(), counter[0], scales.clone()

    # timed region: K steps; HIP events bracket the dominant kernel on its stream
    tlc.profile_read()
    tlc.profile_only(DOMINANT)
    tlc.profile_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tlc.profile_enable(False)
    kt = tlc.profile_read()
    last_bits = 8.0 * float(lens.sum().item()) / N

    # phase times: compress calls alone, then decompress calls alone, each
    # bracketed as a whole (the error buffer keeps evolving; inputs rotate)
    kp = min(args.steps, 10)
    p0, p1, p2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    p0.record()
    for _ in range(kp):
        group.compress(xs[counter[0] % pool], ed, s, out=out, out_lens=lens, scales=scales, workspace=ws,
                       status=st_c)
        counter[0] += 1
    p1.record()
    for _ in range(kp):
        group.decompress(out, lens, scales, s, y=yd, workspace=ws, status=st_d)
    p2.record()
    torch.cuda.synchronize()
    comp_ms = p0.elapsed_time(p1) / kp
    dec_ms = p1.elapsed_time(p2) / kp

    # Pipelined: a worker's receive side does not wait for its own compress,
    # so the decompress of payload k-1 runs on a second stream while batch k
    # is compressed (events order each payload's write, read and reuse).  The
    # same inputs and error state as the timed steps; K compress and K
    # decompress calls between the first launch and the last completion.
    e_keep, c_keep = ed.clone(), counter[0]
    ed.copy_(e_warm)
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    ws_d = group.workspace()
    pay = [(torch.empty_like(out), torch.empty_like(lens), sc_warm.clone()) for _ in range(2)]
    st_pc, st_pd = torch.zeros_like(st_c), torch.zeros_like(st_d)
    ev_c = [torch.cuda.Event() for _ in range(2)]
    ev_d = [torch.cuda.Event() for _ in range(2)]
    torch.cuda.synchronize()

    def pcomp(k, base):
        b = k % 2
        if k >= 2:
            sA.wait_event(ev_d[b])  # payload k-2 has been decoded: its buffers are free
        group.compress(xs[(base + k) % pool], ed, s, out=pay[b][0], out_lens=pay[b][1], scales=pay[b][2],
                       workspace=ws, status=st_pc, stream=sA)
        ev_c[b].record(sA)

    def pdec(k):
        b = k % 2
        sB.wait_event(ev_c[b])
        group.decompress(pay[b][0], pay[b][1], pay[b][2], s, y=yd, workspace=ws_d, status=st_pd, stream=sB)
        ev_d[b].record(sB)

    def pipeline(K, base):
        pcomp(0, base)
        for k in range(1, K):
            pcomp(k, base)
            pdec(k - 1)
        pdec(K - 1)

    pipeline(3, c_warm)  # warm-up (the error state is reset below)
    torch.cuda.synchronize()
    ed.copy_(e_warm)
    for b in range(2):
        pay[b][2].copy_(sc_warm)
    torch.cuda.synchronize()
    pa, pb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pa.record(sA)
    pipeline(args.steps, c_warm)
    pb.record(sB)
    torch.cuda.synchronize()
    if (int(st_pc.item()), int(st_pd.item())) != (0, 0):
        raise SystemExit("device status not ok in the pipelined steps")
    pipe_ms = pa.elapsed_time(pb) / args.steps
    ed.copy_(e_keep)
    counter[0] = c_keep
    del e_keep
    torch.cuda.synchronize()

    # per-kernel breakdown: a separate, shorter pass with every kernel bracketed
    # (events add a small gap around each kernel, so short kernels read long)
    tlc.profile_only(None)
    tlc.profile_enable(True)
    for _ in range(min(args.steps, 5)):
        step()
    torch.cuda.synchronize()
    tlc.profile_enable(False)
    kt_all = tlc.profile_read()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    if (int(st_c.item()), int(st_d.item())) != (0, 0) or first["status"] != (0, 0):
        raise SystemExit(f"device status not ok: {first['status']} / {(int(st_c.item()), int(st_d.item()))}")

    def per_launch(name, table):
        n, ms = table.get(name, (0, 0.0))
        return ms / n if n else 0.0

    dom_ms = per_launch(DOMINANT, kt)
    achieved = DOMINANT_BYTES_PER_ELEM * N / (dom_ms * 1e-3) / 1e9 if dom_ms else 0.0

    # accumulate of the same payload, 8 times (the 8-worker receive side)
    acc = torch.zeros(N, dtype=torch.float32, device=dev)
    st_a = torch.empty(1, dtype=torch.int32, device=dev)
    group.decompress_accumulate(out, lens, scales, s, acc, workspace=ws, status=st_a)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(8):
        group.decompress_accumulate(out, lens, scales, s, acc, workspace=ws, status=st_a)
    a1.record()
    torch.cuda.synchronize()
    acc_ms = a0.elapsed_time(a1) / 8

    # model-delta direction, server side: the workers' sum (the payload decoded
    # densely into acc, then accumulated 7 more times), then the server's
    # compress of the 8-worker mean with its own error buffer (carried)
    err_srv = torch.zeros(N, dtype=torch.float32, device=dev)
    out_srv = torch.empty(group.stream_bytes, dtype=torch.uint8, device=dev)
    lens_srv = torch.empty(len(sizes), dtype=torch.int64, device=dev)
    scales_srv = torch.empty(len(sizes), dtype=torch.float32, device=dev)
    st_s = torch.empty(1, dtype=torch.int32, device=dev)

    def server_step():
        group.decompress(out, lens, scales, s, y=acc, workspace=ws, status=st_a)
        for _ in range(7):
            group.decompress_accumulate(out, lens, scales, s, acc, workspace=ws, status=st_a)
        group.server_compress(acc, 8, err_srv, s, out=out_srv, out_lens=lens_srv, scales=scales_srv,
                              workspace=ws, status=st_s)

    server_step()
    torch.cuda.synchronize()
    ks = 5
    s0, s1, s2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    s0.record()
    for _ in range(ks):
        server_step()
    s1.record()
    for _ in range(ks):
        group.server_compress(acc, 8, err_srv, s, out=out_srv, out_lens=lens_srv, scales=scales_srv,
                              workspace=ws, status=st_s)
    s2.record()
    torch.cuda.synchronize()
    if int(st_a.item()) != 0 or int(st_s.item()) != 0:
        raise SystemExit(f"device status not ok in the server step: {int(st_a.item())} / {int(st_s.item())}")
    srv_step_ms = s0.elapsed_time(s1) / ks
    srv_comp_ms = s1.elapsed_time(s2) / ks
    L_srv = int(lens_srv.sum().item())

    # ablations (3LC page, method items two and three): the same quantization
    # with the codes written as quartic bytes only, or as 2-bit fields; each
    # from a zero error buffer, 5 timed compress calls on rotating inputs (the
    # error carried, as in the main steps), then 5 timed decompress calls
    ablations = {}
    err_fx = torch.empty(N, dtype=torch.float32, device=dev)
    for name, enc in (("quartic_only", tlc.ENC_QUARTIC), ("two_bit", tlc.ENC_TWOBIT)):
        offs_h, offs_d, total_b = group.fixed_offsets(enc)
        out_fx = torch.empty(total_b, dtype=torch.uint8, device=dev)
        sc_fx = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
        y_fx = torch.empty(N, dtype=torch.float32, device=dev)
        err_fx.zero_()
        for k in range(3):
            group.compress_fixed(xs[k % pool], err_fx, s, enc, out_fx, offs_d, scales=sc_fx, workspace=ws,
                                 status=st_c)
        group.decompress_fixed(out_fx, offs_d, sc_fx, s, enc, y=y_fx, status=st_d)
        torch.cuda.synchronize()
        f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        f0.record()
        for k in range(3, 8):
            group.compress_fixed(xs[k % pool], err_fx, s, enc, out_fx, offs_d, scales=sc_fx, workspace=ws,
                                 status=st_c)
        f1.record()
        for _ in range(5):
            group.decompress_fixed(out_fx, offs_d, sc_fx, s, enc, y=y_fx, status=st_d)
        f2.record()
        torch.cuda.synchronize()
        if (int(st_c.item()), int(st_d.item())) != (0, 0):
            raise SystemExit(f"device status not ok in the {name} ablation")
        nbytes = sum(tlc.fixed_len(n, enc) for n in sizes)
        c_ms = f0.elapsed_time(f1) / 5
        d_ms = f1.elapsed_time(f2) / 5
        ablations[name] = {"bits_per_value": round(8.0 * nbytes / N, 4), "compress_ms": round(c_ms, 4),
                           "decompress_ms": round(d_ms, 4),
                           "compress_roofline_frac": round((12.0 * N + nbytes) / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                                           4),
                           "decompress_roofline_frac": round((4.0 * N + nbytes) / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                                             4)}
        del out_fx, y_fx
    del err_fx
    B_total = sum(-(-n // 5) for n in sizes)
    ablations["zero_run_gain_first_step"] = round(B_total / int(first["lens"].sum()), 2)

    # the five-plane byte layout (the other reading of which five values share
    # a quartic byte): each tensor gathered into the order p = 5k + j <- k + jB,
    # the grouped codec on the plan of sizes 5*ceil(n/5), the error buffer and
    # y scattered back; the first step from a zero error buffer on the same
    # set as the main first step, then 5 timed compress and decompress calls
    padded = [5 * (-(-n // 5)) for n in sizes]
    gp = tlc.Group(padded, device=dev)
    pl_src = torch.tensor(group.elem_offsets[:-1], dtype=torch.int64, device=dev)
    pl_dst = torch.tensor(gp.elem_offsets[:-1], dtype=torch.int64, device=dev)
    pl_n = torch.tensor(sizes, dtype=torch.int64, device=dev)
    max_n = max(sizes)
    xp = torch.empty(gp.total, dtype=torch.float32, device=dev)
    ep = torch.empty(gp.total, dtype=torch.float32, device=dev)
    err_pl = torch.zeros(N, dtype=torch.float32, device=dev)
    out_pl = torch.empty(gp.stream_bytes, dtype=torch.uint8, device=dev)
    lens_pl = torch.empty(len(sizes), dtype=torch.int64, device=dev)
    sc_pl = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
    ws_pl = gp.workspace()

    def pl_compress(k):
        pl_compress_x(xs[k % pool])

    def pl_compress_x(xk):
        tlc.planes_gather(xk, pl_src, xp, pl_dst, pl_n, max_n)
        tlc.planes_gather(err_pl, pl_src, ep, pl_dst, pl_n, max_n)
        gp.compress(xp, ep, s, out=out_pl, out_lens=lens_pl, scales=sc_pl, workspace=ws_pl, status=st_c)
        tlc.planes_scatter(ep, pl_dst, err_pl, pl_src, pl_n, max_n)

    def pl_decompress():
        gp.decompress(out_pl, lens_pl, sc_pl, s, y=xp, workspace=ws_pl, status=st_d)
        tlc.planes_scatter(xp, pl_dst, yd, pl_src, pl_n, max_n)

    pl_compress(0)
    torch.cuda.synchronize()
    L_pl = int(lens_pl.sum().item())
    for k in range(1, 3):
        pl_compress(k)
    pl_decompress()
    torch.cuda.synchronize()
    f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    f0.record()
    for k in range(3, 8):
        pl_compress(k)
    f1.record()
    for _ in range(5):
        pl_decompress()
    f2.record()
    torch.cuda.synchronize()
    if (int(st_c.item()), int(st_d.item())) != (0, 0):
        raise SystemExit("device status not ok in the five-plane ablation")
    ablations["five_plane"] = {
        "bits_per_value_first_step": round(8.0 * L_pl / N, 4),
        "consecutive_bits_per_value_first_step": round(8.0 * int(first["lens"].sum()) / N, 4),
        "compress_ms": round(f0.elapsed_time(f1) / 5, 4),
        "decompress_ms": round(f1.elapsed_time(f2) / 5, 4),
        "how": "gather into the five-plane order, the grouped codec on the padded plan, scatter back "
               "(times include the gather and scatter)"}

    # steady state of error feedback: the same step continued until the error
    # buffer has filled (every encode tile active, denser streams), then timed
    steady = None
    if args.steady_steps > 0:
        while counter[0] < args.steady_steps:
            step()
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        for _ in range(10):
            step()
        q1.record()
        torch.cuda.synchronize()
        st_ms = q0.elapsed_time(q1) / 10
        if (int(st_c.item()), int(st_d.item())) != (0, 0):
            raise SystemExit("device status not ok in the steady-state steps")
        steady = {"after_steps": counter[0] - 10, "ms_per_step": round(st_ms, 4),
                  "GBps_fp32_in": round(4.0 * N / (st_ms * 1e-3) / 1e9, 1),
                  "bits_per_value": round(8.0 * float(lens.sum().item()) / N, 4)}
        # the same state pipelined over the two streams (10 more steps)
        for b in range(2):
            pay[b][2].copy_(scales)
        torch.cuda.synchronize()
        pa.record(sA)
        pipeline(10, counter[0])
        pb.record(sB)
        torch.cuda.synchronize()
        out_pl_last = pay[(10 - 1) % 2]
        if (int(st_pc.item()), int(st_pd.item())) != (0, 0):
            raise SystemExit("device status not ok in the pipelined steady-state steps")
        steady["pipelined_ms_per_step"] = round(pa.elapsed_time(pb) / 10, 4)
        # the receive side at this density: the last payload accumulated 8 times
        a0.record()
        for _ in range(8):
            group.decompress_accumulate(out_pl_last[0], out_pl_last[1], out_pl_last[2], s, acc, workspace=ws,
                                        status=st_a)
        a1.record()
        torch.cuda.synchronize()
        if int(st_a.item()) != 0:
            raise SystemExit("device status not ok in the steady-state accumulate")
        steady["accumulate_ms_per_payload"] = round(a0.elapsed_time(a1) / 8, 4)
        # the two byte layouts on the same codes: quantization does not depend
        # on the layout, so one more step's input and this error state, taken
        # by each layout on copies of the error buffer
        xk = xs[counter[0] % pool]
        e_a = ed.clone()
        group.compress(xk, e_a, s, out=out, out_lens=lens, scales=scales, workspace=ws, status=st_c)
        err_pl.copy_(ed)
        pl_compress_x(xk)
        torch.cuda.synchronize()
        if int(st_c.item()) != 0:
            raise SystemExit("device status not ok in the steady-state layout comparison")
        ablations["five_plane"]["bits_per_value_steady"] = round(8.0 * int(lens_pl.sum().item()) / N, 4)
        ablations["five_plane"]["consecutive_bits_per_value_steady"] = round(8.0 * int(lens.sum().item()) / N, 4)
        del e_a
    del pay, ws_d, gp, xp, ep, err_pl, out_pl, ws_pl


    # copy yardstick: what a plain streaming copy reaches on this GPU
    copy_gbps = None
    if not args.no_copy:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        for _ in range(2):
            tlc.copy_probe(src, dst, nbytes)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            tlc.copy_probe(src, dst, nbytes)
        c1.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * nbytes * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst

    L_total = int(first["lens"].sum())
    bits = 8.0 * L_total / N
    bits_hdr = 8.0 * (L_total + 4 * len(sizes)) / N
    alg_bytes_comp = 12.0 * N + L_total + 4 * len(sizes)
    alg_bytes_dec = 4.0 * N + L_total
    # server step: dense decode of the first payload (4 B/value + stream), 7
    # sparse accumulates (stream + 8 B per nonzero code), the mean's compress
    nnz_bytes = 0.0  # the nonzero codes are a few thousand here: below rounding
    alg_bytes_srv = (4.0 * N + L_total) + 7 * (L_total + nnz_bytes) + (12.0 * N + L_srv + 4 * len(sizes))
    gbps = 4.0 * N / (ms_per_step * 1e-3) / 1e9

    cpu = cpu_all = None
    parity = "not checked (--no-cpu)"
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu, streams, Ms, err0 = cpu_baseline(x_host, sizes, s, args.cpu_passes)
        ok = np.array_equal(first["scales"].view(np.uint32), np.asarray(Ms, np.float32).view(np.uint32))
        ok &= np.array_equal(first["err"].view(np.uint32), err0.view(np.uint32))
        for t in range(len(sizes)):
            o = group.offsets[t]
            L = int(first["lens"][t])
            ok &= L == streams[t].size and np.array_equal(first["out"][o:o + L], streams[t])
        parity = "bit-exact vs oracle (streams, M, error buffer; first step)" if ok else "MISMATCH"
        if not ok:
            print("[bench] PARITY MISMATCH", file=sys.stderr, flush=True)
        cpu["host_cpu"] = host_cpu_model()
        print("[bench] timing the CPU oracle on all cores", file=sys.stderr, flush=True)
        cpu_all = cpu_baseline_all_cores(x_host, sizes, s, args.cpu_passes)

    traffic = stored_traffic(args.workload)
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "tensors": len(sizes), "values": N, "s": s,
                   "values_dist": wl.description, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": DOMINANT, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_elem": DOMINANT_BYTES_PER_ELEM,
                     "avg_ms": round(dom_ms, 4)},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "parity": parity,
        "bits_per_value": round(bits, 4),
        "bits_per_value_with_scale": round(bits_hdr, 4),
        "compression_ratio_vs_fp32": round(32.0 / bits_hdr, 1),
        "compress_ms": round(comp_ms, 4),
        "decompress_ms": round(dec_ms, 4),
        "compress_GBps_fp32_in": round(4.0 * N / (comp_ms * 1e-3) / 1e9, 1) if comp_ms else None,
        "decompress_GBps_fp32_in": round(4.0 * N / (dec_ms * 1e-3) / 1e9, 1) if dec_ms else None,
        "path_roofline_frac": round((alg_bytes_comp + alg_bytes_dec) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                    4),
        "compress_roofline_frac": round(alg_bytes_comp / (comp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if comp_ms else None,
        "compress_roofline_frac_nominal_12p3B": round(12.3 * N / (comp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if comp_ms else None,
        "decompress_roofline_frac": round(alg_bytes_dec / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if dec_ms else None,
        "accumulate_ms_per_payload": round(acc_ms, 4),
        "server_step_ms": round(srv_step_ms, 4),
        "server_step_roofline_frac": round(alg_bytes_srv / (srv_step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "server_compress_ms": round(srv_comp_ms, 4),
        "server_compress_roofline_frac": round((12.0 * N + L_srv + 4 * len(sizes)) / (srv_comp_ms * 1e-3) / 1e9
                                               / HBM_PEAK_GBPS, 4),
        "server_bits_per_value": round(8.0 * L_srv / N, 4),
        "copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        # the same algorithmic bytes against the measured copy rate instead of the nominal peak
        "path_copy_ceiling_frac": round((alg_bytes_comp + alg_bytes_dec) / (ms_per_step * 1e-3) / 1e9 / copy_gbps, 4)
        if copy_gbps else None,
        "dominant_copy_ceiling_frac": round(achieved / copy_gbps, 4) if copy_gbps else None,
        "bits_per_value_last_step": round(last_bits, 4),
        "steady_state": steady,
        "pipelined": {"ms_per_step": round(pipe_ms, 4), "GBps_fp32_in": round(4.0 * N / (pipe_ms * 1e-3) / 1e9, 1),
                      "path_roofline_frac": round((alg_bytes_comp + alg_bytes_dec) / (pipe_ms * 1e-3) / 1e9
                                                  / HBM_PEAK_GBPS, 4),
                      "how": "compress of batch k on one stream, decompress of payload k-1 on another "
                             "(receive side overlapped with the send side), same inputs and error state "
                             "as the timed steps"},
        "ablations": ablations,
        "kernels_ms_per_launch_events": {k: round(v[1] / v[0], 4) for k, v in kt_all.items() if v[0]},
        "wall_s_timed": round(wall, 3),
        "kernel_source": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
