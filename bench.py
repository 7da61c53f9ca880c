"""Benchmark of the 3LC codec hot path on one MI355X.

One step = one worker's grouped compress of a whole gradient set (error
accumulation, per-tensor scale, ternary quantization, quartic packing,
zero-run encoding) followed by the grouped decompress of that payload
(zero-run decoding, quartic decoding, dequantization).  Inputs are seeded
and synthetic, generated on the host and resident in HBM before any timing.

Headline line (BERT-large gradient set, 391 tensors, 335,141,888 fp32 values,
30% exact zeros, the rest N(0, 1e-4), s = 1.75): K steps with the error
buffer carried from step to step, as in training, each step on a different
gradient set (the generated set rotated by k * 1,000,003 elements, 32 such
sets used in turn).  Each step is bracketed by HIP events: the line gives the
mean (value), median and min step time, the roofline of the dominant kernel
(the 12-byte/element pass over x and err) timed with HIP events on its own
stream inside the timed region, bits per value, and the CPU oracle timed on
the host.  The decompress follows a path hint word carried from step to step.

Per-configuration records (``configs``), each with the median and min over at
least 20 repetitions, GB/s of fp32 input, the fraction of the HBM roofline of
the step's algorithmic bytes and of the measured copy rate, and bits/value:
* single_1m: one compress+decompress from a zero error buffer (restored
  outside the timed window before every repetition);
* single_16m: 10 consecutive steps on fresh inputs (seed 200+t) with the
  error carried, run 3 times, every step timed;
* resnet110: one grouped step (329 tensors), also in us and tensors/s;
* resnet50: one grouped step at each s in {1.0, 1.5, 1.9};
* bert_large_first_step: worker w's set (seed 500+w, w = 0..7) compressed
  from a zero error buffer and decompressed, 3 repetitions per worker; then
  the 8 workers' payloads decompressed and accumulated into one fp32 sum,
  in one many-payload call and as 8 calls in worker order (bit-identical);
* bert_large_steady: the headline's steps continued until the error buffer
  has filled (every encode tile active, streams about twice as dense), 20
  steps timed; then each worker's own 150-step error-feedback run, and the
  8 steady-state payloads accumulated as above.

Also reported: compress and decompress timed apart, the same steps pipelined
over two streams, the model-delta direction's server step, and the ablations
(the codes as quartic bytes only or as 2-bit fields, the five-plane layout).

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--only CONFIG]
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
ROT = 1_000_003                 # rotation between the gradient sets of consecutive steps
WORKERS = 8
# Per-kernel times from a pass where the library brackets every launch with two
# events: the host then submits more slowly than short kernels run, so the GPU
# waits between them and those waits land inside the brackets.
EVENTS_NOTE = ("each launch bracketed by two HIP events in a pass of its own; kernels shorter than a few tens "
               "of microseconds read long there (host submission gaps fall inside the brackets), so kernel "
               "durations of the short kernels come from the rocprofv3 kernel traces")
RECORDS = ("single_1m", "single_16m", "resnet110", "resnet50", "bert_large_first_step", "bert_large_steady")


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


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# timing helpers


def timed(torch, reps: int, body, before=None):
    """Runs body(r, mark) for r < reps on torch's current stream, each
    repetition bracketed by HIP events (mark() records one more in between);
    before(r), if given, runs outside the brackets.  Returns, per repetition,
    the list of segment times in ms (one synchronisation at the end)."""
    marks = []
    for r in range(reps):
        if before is not None:
            before(r)
        m = []

        def mark(m=m):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            m.append(e)

        mark()
        body(r, mark)
        mark()
        marks.append(m)
    torch.cuda.synchronize()
    return [[m[i].elapsed_time(m[i + 1]) for i in range(len(m) - 1)] for m in marks]


def stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "mean": round(float(a.mean()), 4), "reps": int(a.size)}


def frac(nbytes: float, ms: float, peak_gbps: float):
    return round(nbytes / (ms * 1e-3) / 1e9 / peak_gbps, 4) if ms and peak_gbps else None


def quartic_bytes(sizes) -> int:
    """Bytes of the tensors' quartic encoding: five codes per byte."""
    return sum(-(-int(n) // 5) for n in sizes)


def step_record(N: int, tensors: int, s: float, L: int, step_ms, comp_ms, dec_ms, copy_gbps, dom=None, B=None):
    """The measurement table of one configuration: times over the
    repetitions, and the roofline of the step's algorithmic bytes
    (compress 12 B/value + stream + 4 B per M; decompress 4 B/value +
    stream) at the median step time.  B is the tensors' quartic byte count
    (the sum of ceil(n/5)), for the zero-run encoding's ratio B/L."""
    st, sc, sd = stats(step_ms), stats(comp_ms), stats(dec_ms)
    alg_c = 12.0 * N + L + 4 * tensors
    alg_d = 4.0 * N + L
    med = st["median"]
    achieved = (alg_c + alg_d) / (med * 1e-3) / 1e9
    rec = {
        "values": N, "tensors": tensors, "s": s,
        "ms_per_step": st,
        "compress_ms": sc,
        "decompress_ms": sd,
        "GBps_fp32_in": round(4.0 * N / (med * 1e-3) / 1e9, 1),
        "compress_GBps_fp32_in": round(4.0 * N / (sc["median"] * 1e-3) / 1e9, 1),
        "decompress_GBps_fp32_in": round(4.0 * N / (sd["median"] * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "bytes_per_step": int(alg_c + alg_d),
                     "what": "compress+decompress algorithmic bytes over the median step"},
        "compress_roofline_frac": frac(alg_c, sc["median"], HBM_PEAK_GBPS),
        "compress_roofline_frac_nominal_12p3B": frac(12.3 * N, sc["median"], HBM_PEAK_GBPS),
        "decompress_roofline_frac": frac(alg_d, sd["median"], HBM_PEAK_GBPS),
        "copy_ceiling_frac": round(achieved / copy_gbps, 4) if copy_gbps else None,
        "bits_per_value": round(8.0 * L / N, 4),
        "bits_per_value_with_scale": round(8.0 * (L + 4 * tensors) / N, 4),
        "compression_ratio_vs_fp32": round(4.0 * N / L, 1),
    }
    if B is not None:
        rec["zero_run_ratio"] = round(B / L, 2)
    if dom is not None:
        launches, ms = dom
        if launches:
            avg = ms / launches
            ach = DOMINANT_BYTES_PER_ELEM * N / (avg * 1e-3) / 1e9
            rec["dominant_kernel"] = {"kernel": DOMINANT, "avg_ms": round(avg, 4), "achieved": round(ach, 1),
                                      "frac": round(ach / HBM_PEAK_GBPS, 4), "launches": launches}
    return rec


def wire_record(torch, group, out, lens, scales, N: int, reps: int = 20):
    """The payload as one wire message (tlc_wire_pack_group) and back
    (tlc_wire_unpack_group): message bytes against the slots' capacity, and
    the two calls' times.  Each moves the message once in and once out (the
    headers included), so its roofline bytes are twice the message length."""
    wire = torch.empty(group.wire_bound(), dtype=torch.uint8, device=out.device)
    wire_len = torch.empty(1, dtype=torch.int64, device=out.device)
    st_w = torch.empty(1, dtype=torch.int32, device=out.device)
    st_u = torch.empty(1, dtype=torch.int32, device=out.device)
    wws = group.wire_workspace()
    out2, lens2 = torch.empty_like(out), torch.empty_like(lens)
    sc2 = torch.empty_like(scales)

    def pack():
        group.wire_pack(out, lens, scales, wire=wire, wire_len=wire_len, workspace=wws, status=st_w)

    def unpack():
        group.wire_unpack(wire, out=out2, out_lens=lens2, scales=sc2, workspace=wws, status=st_u)

    pack()
    unpack()
    torch.cuda.synchronize()
    if int(st_w.item()) != 0 or int(st_u.item()) != 0:
        raise SystemExit("device status not ok in the wire pack or unpack")
    if not torch.equal(lens2, lens) or not torch.equal(sc2.view(torch.int32), scales.view(torch.int32)):
        raise SystemExit("wire unpack did not give back the payload's lengths and scales")
    wl = int(wire_len.item())
    tp = timed(torch, reps, lambda r, mark: pack())
    tu = timed(torch, reps, lambda r, mark: unpack())
    sp, su = stats([v[0] for v in tp]), stats([v[0] for v in tu])
    return {"message_bytes": wl, "slot_capacity_bytes": int(group.stream_bytes),
            "how": "each call alone between two events, so the host's submission of its two launches is "
                   "included; the kernel traces give the kernels' own time",
            "bits_per_value_on_the_wire": round(8.0 * wl / N, 4),
            "pack_ms": sp, "unpack_ms": su,
            "pack_roofline_frac": frac(2.0 * wl, sp["median"], HBM_PEAK_GBPS),
            "unpack_roofline_frac": frac(2.0 * wl, su["median"], HBM_PEAK_GBPS)}


class Bench:
    """Device state shared by the records."""

    def __init__(self, args):
        import torch

        from gradient_compression_distributed_lc_amd import tlc, workloads
        self.torch, self.tlc, self.workloads, self.args = torch, tlc, workloads, args
        self.dev = torch.device("cuda:0")
        self.copy_gbps = None

    # -- yardstick ------------------------------------------------------------
    def copy_yardstick(self):
        torch, tlc = self.torch, self.tlc
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
        dst = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
        for _ in range(2):
            tlc.copy_probe(src, dst, nbytes)
        t = timed(torch, 10, lambda r, mark: tlc.copy_probe(src, dst, nbytes))
        ms = stats([v[0] for v in t])["median"]
        self.copy_gbps = 2 * nbytes / (ms * 1e-3) / 1e9
        del src, dst
        torch.cuda.empty_cache()

    def status_ok(self, *sts, what=""):
        got = [int(v.item()) for v in sts]
        if any(got):
            raise SystemExit(f"device status not ok ({what}): {got}")

    # -- one compress+decompress step from a zero error buffer ----------------
    def one_step(self, name: str, x_host: np.ndarray, sizes, s: float, reps: int):
        torch, tlc = self.torch, self.tlc
        dev = self.dev
        N = int(x_host.size)
        single = len(sizes) == 1
        x = torch.from_numpy(x_host).to(dev)
        err = torch.zeros(N, dtype=torch.float32, device=dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        st_c = torch.empty(1, dtype=torch.int32, device=dev)
        st_d = torch.empty(1, dtype=torch.int32, device=dev)
        hint = tlc.path_hint()
        if single:
            out = torch.empty(tlc.compress_bound(N), dtype=torch.uint8, device=dev)
            lens = torch.empty(1, dtype=torch.int64, device=dev)
            scales = torch.zeros(1, dtype=torch.float32, device=dev)
            ws = torch.empty(tlc.workspace_size(N), dtype=torch.uint8, device=dev)

            def comp():
                tlc.compress(x, err, s, out=out, out_len=lens, scale=scales, workspace=ws, status=st_c)

            def dec():
                tlc.decompress(out, lens, scales, N, s, y=y, workspace=ws, status=st_d, path_hint=hint)
        else:
            g = tlc.Group(sizes, device=dev)
            out = torch.empty(g.stream_bytes, dtype=torch.uint8, device=dev)
            lens = torch.empty(len(sizes), dtype=torch.int64, device=dev)
            scales = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
            ws = g.workspace()

            def comp():
                g.compress(x, err, s, out=out, out_lens=lens, scales=scales, workspace=ws, status=st_c)

            def dec():
                g.decompress(out, lens, scales, s, y=y, workspace=ws, status=st_d, path_hint=hint)

        def before(r):  # a first step: zero error buffer, no previous M
            err.zero_()
            scales.zero_()

        def body(r, mark):
            comp()
            mark()
            dec()

        timed(torch, 3, body, before)
        t = timed(torch, reps, body, before)
        self.status_ok(st_c, st_d, what=name)
        # the dominant kernel's duration, in repetitions of their own (the
        # events around it cost a small step several microseconds)
        tlc.profile_read()
        tlc.profile_only(DOMINANT)
        tlc.profile_enable(True)
        timed(torch, reps, body, before)
        tlc.profile_enable(False)
        dom = tlc.profile_read().get(DOMINANT, (0, 0.0))
        L = int(lens.sum().item())
        rec = step_record(N, len(sizes), s, L, [a + b for a, b in t], [a for a, _ in t], [b for _, b in t],
                          self.copy_gbps, dom, B=quartic_bytes(sizes))
        rec["decompress_sequence"] = "dense" if int(hint[0]) else "sparse"
        rec["nonzero_code_fraction"] = round(float(torch.count_nonzero(y).item()) / N, 6)
        # the same step captured once in a HIP graph and replayed (the library
        # launches only kernels on the caller's stream, so a training loop can
        # capture its codec calls); the first-step reset stays outside
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        before(0)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                comp()
                dec()
        torch.cuda.synchronize()

        def replay(r, mark):
            graph.replay()

        timed(torch, 3, replay, before)
        tg = timed(torch, reps, replay, before)
        self.status_ok(st_c, st_d, what=f"{name}, graph replays")
        rec["graph_ms_per_step"] = stats([v[0] for v in tg])
        del graph
        return rec

    def record_single_1m(self):
        w = self.workloads.get("single_1m")
        return self.one_step("single_1m", self.workloads.generate("single_1m"), w.sizes, w.s_values[0],
                             self.args.reps)

    def record_resnet110(self):
        w = self.workloads.get("resnet110")
        rec = self.one_step("resnet110", self.workloads.generate("resnet110"), w.sizes, w.s_values[0],
                            max(self.args.reps, 30))
        med = rec["ms_per_step"]["median"]
        rec["us_per_step"] = {k: round(v * 1e3, 1) for k, v in rec["ms_per_step"].items() if k != "reps"}
        rec["tensors_per_s"] = round(len(w.sizes) / (med * 1e-3), 0)
        gmed = rec["graph_ms_per_step"]["median"]
        rec["graph_us_per_step"] = {k: round(v * 1e3, 1) for k, v in rec["graph_ms_per_step"].items() if k != "reps"}
        rec["graph_tensors_per_s"] = round(len(w.sizes) / (gmed * 1e-3), 0)
        rec["note"] = "launch-bound: 1.73M values in 329 tensors; the step is the kernels' fixed latencies"
        return rec

    def record_resnet50(self):
        w = self.workloads.get("resnet50")
        x = self.workloads.generate("resnet50")
        return {f"s={s}": self.one_step(f"resnet50 s={s}", x, w.sizes, s, self.args.reps) for s in w.s_values}

    def record_single_16m(self):
        """10 steps with fresh inputs (seed 200+t) and the error carried,
        the whole sequence run 3 times from a zero error buffer."""
        torch, tlc = self.torch, self.tlc
        dev = self.dev
        w = self.workloads.get("single_16m")
        s, N = w.s_values[0], w.total
        xs = [torch.from_numpy(self.workloads.generate("single_16m", step=t)).to(dev) for t in range(10)]
        err = torch.zeros(N, dtype=torch.float32, device=dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        out = torch.empty(tlc.compress_bound(N), dtype=torch.uint8, device=dev)
        lens = torch.empty(1, dtype=torch.int64, device=dev)
        scales = torch.zeros(1, dtype=torch.float32, device=dev)
        ws = torch.empty(tlc.workspace_size(N), dtype=torch.uint8, device=dev)
        st_c = torch.empty(1, dtype=torch.int32, device=dev)
        st_d = torch.empty(1, dtype=torch.int32, device=dev)
        hint = tlc.path_hint()

        def step(t):
            tlc.compress(xs[t], err, s, out=out, out_len=lens, scale=scales, workspace=ws, status=st_c)

        def dec():
            tlc.decompress(out, lens, scales, N, s, y=y, workspace=ws, status=st_d, path_hint=hint)

        # an untimed run that reads each step's length
        err.zero_()
        scales.zero_()
        step_L = []
        for t in range(10):
            step(t)
            dec()
            step_L.append(int(lens.item()))
        runs = 3
        per_step = [[] for _ in range(10)]
        comp, decm, tot = [], [], []
        for _ in range(runs):
            torch.cuda.synchronize()
            err.zero_()
            scales.zero_()

            def body(t, mark):
                step(t)
                mark()
                dec()

            t_ms = timed(torch, 10, body)
            for t, (a, b) in enumerate(t_ms):
                per_step[t].append(a + b)
                comp.append(a)
                decm.append(b)
            tot.append(sum(a + b for a, b in t_ms))
        self.status_ok(st_c, st_d, what="single_16m")
        # bits over the 10 steps' streams
        L_mean = int(round(np.mean(step_L)))
        rec = step_record(N, 1, s, L_mean, [a for v in per_step for a in v], comp, decm, self.copy_gbps,
                          B=quartic_bytes([N]))
        rec["per_step_ms_median"] = [round(float(np.median(v)), 4) for v in per_step]
        rec["bits_per_value_per_step"] = [round(8.0 * v / N, 4) for v in step_L]
        rec["ten_steps_ms"] = stats(tot)
        rec["how"] = (f"{runs} runs of the 10 carried steps from a zero error buffer; ms_per_step pools "
                      f"all {10 * runs} steps; bits_per_value is the mean over the 10 steps")
        return rec

    # -- BERT-large workers -----------------------------------------------------
    def bert_workers(self, steady_steps: int, cpu: bool):
        """Worker w's set (seed 500+w) for w < 8, resident on the device; each
        worker's first payload (zero error buffer) and, if steady_steps, its
        payload after steady_steps steps of its own error feedback (step k on
        the set rotated by (k mod 32) * 1,000,003)."""
        torch, tlc = self.torch, self.tlc
        dev = self.dev
        wl = self.workloads.get("bert_large")
        sizes, N, s = wl.sizes, wl.total, wl.s_values[0]
        g = tlc.Group(sizes, device=dev)
        self.bert_group = g
        SB = g.stream_bytes
        pay = {k: (torch.empty((WORKERS, SB), dtype=torch.uint8, device=dev),
                   torch.empty((WORKERS, len(sizes)), dtype=torch.int64, device=dev),
                   torch.zeros((WORKERS, len(sizes)), dtype=torch.float32, device=dev))
               for k in (("first", "steady") if steady_steps else ("first",))}
        err = torch.zeros(N, dtype=torch.float32, device=dev)
        stage = torch.empty(N, dtype=torch.float32, device=dev)
        st_c = torch.empty(1, dtype=torch.int32, device=dev)
        ws = g.workspace()
        xs = []
        oracle_first = []
        for w in range(WORKERS):
            t0 = time.perf_counter()
            xh = self.workloads.generate("bert_large", worker=w)
            xd = torch.from_numpy(xh).to(dev)
            xs.append(xd)
            if cpu:
                import oracle
                offs = self.workloads.offsets(sizes)
                e = np.zeros(N, np.float32)
                cur = []
                for t, n in enumerate(sizes):
                    o = np.empty(-(-n // 5), np.uint8)
                    L, M = oracle.compress_inplace(xh[offs[t]:offs[t + 1]], e[offs[t]:offs[t + 1]], s, o)
                    cur.append((o[:L].copy(), np.float32(M)))
                oracle_first.append(cur)
                del e
            del xh
            err.zero_()
            o, ln, sc = pay["first"]
            g.compress(xd, err, s, out=o[w], out_lens=ln[w], scales=sc[w], workspace=ws, status=st_c)
            if steady_steps:
                so, sl, ss = pay["steady"]
                ss[w].copy_(sc[w])
                for k in range(1, steady_steps):
                    sh = (k % 32) * ROT % N
                    stage[sh:].copy_(xd[:N - sh])
                    stage[:sh].copy_(xd[N - sh:])
                    g.compress(stage, err, s, out=so[w], out_lens=sl[w], scales=ss[w], workspace=ws, status=st_c)
            torch.cuda.synchronize()
            self.status_ok(st_c, what=f"bert_large worker {w}")
            log(f"worker {w}: set, first payload{' and steady payload' if steady_steps else ''} "
                f"in {time.perf_counter() - t0:.1f}s")
        del stage, err
        torch.cuda.empty_cache()
        parity = None
        if cpu:
            o, ln, sc = (v.cpu().numpy() for v in pay["first"])
            ok = True
            for w in range(WORKERS):
                for t, (stt, M) in enumerate(oracle_first[w]):
                    off = g.offsets[t]
                    ok &= int(ln[w, t]) == stt.size and np.array_equal(o[w, off:off + stt.size], stt)
                    ok &= np.float32(sc[w, t]).view(np.uint32) == M.view(np.uint32)
            parity = ok
        return xs, pay, oracle_first, parity

    def exchange_record(self, payload, reps: int = 10, marker=None):
        """One GPU's share of the sharded exchange at the BERT-large shape,
        8 workers that are also the 8 owners of contiguous tensor ranges
        (balanced by values), without the transport: GPU 0 packs its payload
        into one wire message per owner (send); as owner of range 0 it
        unpacks the 8 workers' messages for that range, adds them in worker
        order with one many-payload call, compresses the mean with its own
        error buffer and packs the result (owner); it unpacks the 8 owners'
        messages into one payload of the whole group and decodes the model
        delta with one grouped decompress (receive).  The
        messages GPU 0 receives are packed beforehand from the workers'
        payloads and the owners' results, and lie back to back as the
        transport would leave them.  The 8 messages GPU 0 sends come from one
        call (tlc_wire_pack_ranges_group), and each side's 8 received messages
        are unpacked by one call (tlc_wire_unpack_ranges_group)."""
        torch, tlc = self.torch, self.tlc
        g = self.bert_group
        sizes, N = g.sizes, g.total
        s = self.workloads.get("bert_large").s_values[0]
        o, ln, sc = payload
        dev = self.dev
        cuts, acc_n, k = [0], 0, 1
        for t, n in enumerate(sizes):
            acc_n += n
            if k < WORKERS and acc_n >= k * N / WORKERS and t + 1 < len(sizes):
                cuts.append(t + 1)
                k += 1
        cuts.append(len(sizes))
        shards = [(lo, hi, tlc.Group(sizes[lo:hi], device=dev)) for lo, hi in zip(cuts[:-1], cuts[1:])]

        def view(w, lo, hi, sub):  # worker w's payload restricted to tensors lo..hi-1
            so = g.offsets[lo]
            return o[w][so:so + sub.stream_bytes], ln[w][lo:hi], sc[w][lo:hi]

        # messages to owner 0 from every worker, and every owner's result message
        lo0, hi0, sub0 = shards[0]
        ws0 = sub0.wire_workspace()
        to_owner0 = []
        for w in range(WORKERS):
            wire, wl, _ = sub0.wire_pack(*view(w, lo0, hi0, sub0), workspace=ws0)
            to_owner0.append((wire, int(wl.item())))
        owner_msgs = []
        for lo, hi, sub in shards:
            inp = torch.empty((WORKERS, sub.stream_bytes), dtype=torch.uint8, device=dev)
            il = torch.empty((WORKERS, hi - lo), dtype=torch.int64, device=dev)
            isc = torch.empty((WORKERS, hi - lo), dtype=torch.float32, device=dev)
            for w in range(WORKERS):
                a, b, c = view(w, lo, hi, sub)
                inp[w].copy_(a)
                il[w].copy_(b)
                isc[w].copy_(c)
            acc = torch.zeros(sub.total, dtype=torch.float32, device=dev)
            sub.decompress_accumulate_many(inp, il.view(-1), isc.view(-1), s, acc)
            e_srv = torch.zeros(sub.total, dtype=torch.float32, device=dev)
            out_o, lens_o, sc_o, _ = sub.server_compress(acc, WORKERS, e_srv, s)
            wire, wl, _ = sub.wire_pack(out_o, lens_o, sc_o)
            owner_msgs.append((wire, int(wl.item())))
            del inp, il, isc, acc, e_srv
        torch.cuda.synchronize()
        # GPU 0's buffers
        send_buf = torch.empty(g.wire_bound(), dtype=torch.uint8, device=dev)
        send_lens = torch.empty(len(shards), dtype=torch.int64, device=dev)
        send_ws = g.wire_workspace()
        st = torch.zeros(8, dtype=torch.int32, device=dev)
        inp0 = torch.empty((WORKERS, sub0.stream_bytes), dtype=torch.uint8, device=dev)
        il0 = torch.empty((WORKERS, hi0 - lo0), dtype=torch.int64, device=dev)
        isc0 = torch.empty((WORKERS, hi0 - lo0), dtype=torch.float32, device=dev)
        acc0 = torch.empty(sub0.total, dtype=torch.float32, device=dev)
        e0 = torch.zeros(sub0.total, dtype=torch.float32, device=dev)
        wsm = torch.empty(sub0.accumulate_many_workspace_size(WORKERS), dtype=torch.uint8, device=dev)
        wsc = sub0.workspace()
        out0 = torch.empty(sub0.stream_bytes, dtype=torch.uint8, device=dev)
        lens0 = torch.empty(hi0 - lo0, dtype=torch.int64, device=dev)
        sc0 = torch.zeros(hi0 - lo0, dtype=torch.float32, device=dev)
        wire0 = torch.empty(sub0.wire_bound(), dtype=torch.uint8, device=dev)
        wl0 = torch.empty(1, dtype=torch.int64, device=dev)
        hint_m = tlc.path_hint()
        # the owners' messages land in one payload of the whole group (an
        # owner's slots are the group's shifted by a multiple of 16), decoded
        # by one grouped decompress
        rx_out = torch.empty(g.stream_bytes, dtype=torch.uint8, device=dev)
        rx_lens = torch.empty(g.count, dtype=torch.int64, device=dev)
        rx_sc = torch.empty(g.count, dtype=torch.float32, device=dev)
        rx_y = torch.empty(N, dtype=torch.float32, device=dev)
        rx_ws = g.workspace()
        rx_hint = tlc.path_hint()
        # each side's received messages back to back, as the transport leaves
        # them; the workers' messages for range 0 are the range messages of
        # range 0 repeated once per worker, whose slots are the 8 payloads
        # stacked (each copy's slots start at a multiple of 16)
        rx_owner = torch.cat([wire[:wl] for wire, wl in to_owner0])
        rep0 = tlc.Group(list(sub0.sizes) * WORKERS, device=dev)
        cuts0 = [w * (hi0 - lo0) for w in range(WORKERS + 1)]
        assert rep0.stream_bytes == WORKERS * sub0.stream_bytes
        assert all(rep0.offsets[cuts0[w]] == w * sub0.stream_bytes for w in range(WORKERS))
        ws_rep0 = rep0.wire_workspace()
        rx_delta = torch.cat([wire[:wl] for wire, wl in owner_msgs])
        rx_wws = g.wire_workspace()

        def do_send():  # one message per owner, back to back, in one call
            g.wire_pack_ranges(o[0], ln[0], sc[0], cuts, wire=send_buf, wire_lens=send_lens, workspace=send_ws,
                               status=st[0:1])

        def do_owner():  # the 8 workers' messages in one call
            rep0.wire_unpack_ranges(rx_owner, cuts0, out=inp0.view(-1), out_lens=il0.view(-1), scales=isc0.view(-1),
                                    workspace=ws_rep0, status=st[1:2])
            sub0.decompress_accumulate_many(inp0, il0.view(-1), isc0.view(-1), s, acc0, workspace=wsm,
                                            status=st[2:3], path_hint=hint_m)
            sub0.server_compress(acc0, WORKERS, e0, s, out=out0, out_lens=lens0, scales=sc0, workspace=wsc,
                                 status=st[3:4])
            sub0.wire_pack(out0, lens0, sc0, wire=wire0, wire_len=wl0, workspace=ws0, status=st[4:5])

        def do_recv():  # the 8 owners' messages in one call
            g.wire_unpack_ranges(rx_delta, cuts, out=rx_out, out_lens=rx_lens, scales=rx_sc, workspace=rx_wws,
                                 status=st[5:6])
            g.decompress(rx_out, rx_lens, rx_sc, s, y=rx_y, workspace=rx_ws, status=st[6:7], path_hint=rx_hint)

        def before(r):
            acc0.zero_()
            e0.zero_()

        def body(r, mark):
            do_send()
            mark()
            do_owner()
            mark()
            do_recv()

        timed(torch, 2, body, before)
        if marker is not None:  # a profiler's part: the eager repetitions
            torch.cuda.synchronize()
            marker()
        t = timed(torch, reps, body, before)
        if int(st.abs().sum().item()) != 0:
            raise SystemExit(f"device status not ok in the exchange: {st.tolist()}")
        if marker is not None:  # a profiler's part: the capture and the warm-up replays
            marker()
        # the same share captured once in a HIP graph and replayed (every call
        # has its buffers, workspaces and status words given, so nothing is
        # allocated while capturing; the resets stay outside)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        before(0)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                do_send()
                do_owner()
                do_recv()
        torch.cuda.synchronize()

        def replay(r, mark):
            graph.replay()

        timed(torch, 3, replay, before)
        if marker is not None:  # a profiler's part: the graph replays
            torch.cuda.synchronize()
            marker()
        tg = timed(torch, reps, replay, before)
        if int(st.abs().sum().item()) != 0:
            raise SystemExit(f"device status not ok in the exchange's graph replays: {st.tolist()}")
        del graph
        sent = int(send_lens.sum().item())
        recv_owner = sum(wl for _, wl in to_owner0)
        recv_delta = sum(wl for _, wl in owner_msgs)
        return {
            "workers_and_owners": WORKERS,
            "owner0_tensors": hi0 - lo0, "owner0_values": sub0.total,
            "send_ms": stats([v[0] for v in t]), "owner_ms": stats([v[1] for v in t]),
            "receive_ms": stats([v[2] for v in t]), "total_ms": stats([sum(v) for v in t]),
            "graph_total_ms": stats([v[0] for v in tg]),
            "bytes_sent_by_gpu0": sent, "bytes_received_as_owner": recv_owner,
            "bytes_received_model_delta": recv_delta,
            "dense_fp32_bytes_per_gpu": 4 * N,
            "how": ("GPU 0's work in an exchange of first-step payloads without the transport: send = its "
                    "payload as 8 wire messages, one per owner, in one call; owner = unpack the 8 workers' "
                    "messages for its range in one call, one many-payload sum, the compress of the mean with its "
                    "error buffer, one message; receive = unpack the 8 owners' messages in one call into one "
                    "payload of the group and decode the model delta with one grouped decompress.  Its own "
                    "compress of the gradient set is the first-step record's compress_ms."),
        }

    def accumulate_record(self, payload, oracle_payloads=None):
        """The 8 payloads decompressed and accumulated into one fp32 sum in
        worker order: one many-payload call against 8 single-payload calls,
        20 repetitions each, acc cleared outside the timed window.  The many
        call runs with one path hint word carried from call to call (as a
        caller would pass it; the first call takes the sparse sequence), and
        with each launch sequence forced (a fresh word per call)."""
        torch, tlc = self.torch, self.tlc
        g = self.bert_group
        N, count = g.total, g.count
        s = self.workloads.get("bert_large").s_values[0]
        o, ln, sc = payload
        acc = torch.empty(N, dtype=torch.float32, device=self.dev)
        st = torch.empty(1, dtype=torch.int32, device=self.dev)
        ws_many = torch.empty(g.accumulate_many_workspace_size(WORKERS), dtype=torch.uint8, device=self.dev)
        ws = g.workspace()
        lflat, sflat = ln.reshape(-1), sc.reshape(-1)

        carried = tlc.path_hint()
        carried[0] = 0

        def many(r, mark):
            g.decompress_accumulate_many(o, lflat, sflat, s, acc, workspace=ws_many, status=st, path_hint=carried)

        def forced(route):
            words = []
            for _ in range(self.args.reps + 2):
                w = tlc.path_hint()
                w[0] = route
                words.append(w)

            def body(r, mark):
                g.decompress_accumulate_many(o, lflat, sflat, s, acc, workspace=ws_many, status=st,
                                             path_hint=words.pop())
            return body

        def seq(r, mark):
            for w in range(WORKERS):
                g.decompress_accumulate(o[w], ln[w], sc[w], s, acc, workspace=ws, status=st)

        def clear(r):
            acc.zero_()

        reps = self.args.reps
        timed(torch, 2, many, clear)
        t_many = [v[0] for v in timed(torch, reps, many, clear)]
        self.status_ok(st, what="accumulate many")
        # the kernels' share, in repetitions of their own (events around every
        # launch slow the call down)
        tlc.profile_read()
        tlc.profile_only(None)
        tlc.profile_enable(True)
        timed(torch, 5, many, clear)
        tlc.profile_enable(False)
        k_many = tlc.profile_read()
        self.status_ok(st, what="accumulate many, profiled")
        acc_many = acc.clone()
        route_ms = {}
        for route, name in ((0, "sparse"), (1, "dense")):
            body = forced(route)
            timed(torch, 2, body, clear)
            route_ms[name] = stats([v[0] for v in timed(torch, reps, body, clear)])
            self.status_ok(st, what=f"accumulate many, {name} sequence")
            if not torch.equal(acc.view(torch.int32), acc_many.view(torch.int32)):
                raise SystemExit(f"accumulate many: the {name} sequence's sum differs")
        timed(torch, 2, seq, clear)
        t_seq = [v[0] for v in timed(torch, reps, seq, clear)]
        self.status_ok(st, what="accumulate sequential")
        same = bool(torch.equal(acc.view(torch.int32), acc_many.view(torch.int32)))
        L = int(ln.sum().item())
        alg = 8.0 * N + L  # one pass over acc (read and write) plus every stream
        sm = stats(t_many)
        rec = {"payloads": WORKERS, "stream_bytes_total": L,
               "bits_per_value_mean": round(8.0 * L / WORKERS / N, 4),
               "many_call_ms": sm, "many_call_sequence": "dense" if int(carried[0]) else "sparse",
               "many_call_ms_sparse_sequence": route_ms["sparse"], "many_call_ms_dense_sequence": route_ms["dense"],
               "sequential_calls_ms": stats(t_seq),
               "many_call_roofline": {"bound": "hbm", "achieved": round(alg / (sm["median"] * 1e-3) / 1e9, 1),
                                      "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                      "frac": frac(alg, sm["median"], HBM_PEAK_GBPS),
                                      "bytes": int(alg),
                                      "what": "one read and write of all of acc (8 B/value) plus the 8 streams; "
                                              "tiles no payload touches are skipped, and the sparse sequence "
                                              "touches only the elements with a nonzero code, so sparse "
                                              "payloads can exceed 1"},
               "many_call_kernels_ms_per_launch": {k: round(v[1] / v[0], 4) for k, v in k_many.items() if v[0]},
               "many_equals_sequential": same}
        if oracle_payloads is not None:
            import oracle
            want = np.zeros(N, np.float32)
            offs = self.workloads.offsets(g.sizes)
            for w in range(WORKERS):
                for t, (stt, M) in enumerate(oracle_payloads[w]):
                    oracle.decompress_accumulate(stt, M, g.sizes[t], s, want[offs[t]:offs[t + 1]])
            rec["parity"] = ("bit-exact vs the oracle's accumulate of its own 8 payloads in worker order"
                             if np.array_equal(acc_many.cpu().numpy().view(np.uint32), want.view(np.uint32))
                             else "MISMATCH")
        del acc, acc_many, ws_many
        return rec


PROFILE_PHASES = ("early", "steady", "receive", "resnet110", "exchange", "calibrate")


def profile_phase(args):
    """One phase of the workload alone, for a profiler run (rocprofv3 sees
    every kernel of the process): `early` the headline's warm-up and timed
    steps, then the last payload packed into one wire message and unpacked,
    as often; `steady` 150 steps, then the timed steps and the wire message; `receive` the 8
    BERT-large workers' payloads (150 steps each), then the many-payload call
    on each launch sequence and the single-payload accumulates, for the
    steady-state and for the first-step payloads; `resnet110` one-step repetitions of the ResNet-110 group;
    `exchange` one GPU's share of the sharded exchange of the 8 first-step
    payloads, as eager calls and as graph replays;
    `calibrate` the copy and gather yardsticks of the traffic counters.  A
    64 KiB tlc_copy_probe marks the start of every part that a summary
    reads (parts in the order listed in the printed line)."""
    import torch

    from gradient_compression_distributed_lc_amd import tlc, workloads
    dev = torch.device("cuda:0")
    mark_a = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    mark_b = torch.empty_like(mark_a)

    def marker():
        tlc.copy_probe(mark_a, mark_b, 1 << 16)

    out = {"profile": args.profile, "steps": args.steps}
    if args.profile in ("early", "steady"):
        wl = workloads.get("bert_large")
        sizes, N, s = wl.sizes, wl.total, wl.s_values[0]
        g = tlc.Group(sizes, device=dev)
        x0 = torch.from_numpy(workloads.generate("bert_large")).to(dev)
        xs = [x0] + [torch.roll(x0, shifts=k * ROT) for k in range(1, 32)]
        err = torch.zeros(N, dtype=torch.float32, device=dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        o = torch.empty(g.stream_bytes, dtype=torch.uint8, device=dev)
        ln = torch.empty(len(sizes), dtype=torch.int64, device=dev)
        sc = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
        ws = g.workspace()
        st = torch.empty(2, dtype=torch.int32, device=dev)
        hint = tlc.path_hint()
        k = 0
        before = args.warmup if args.profile == "early" else args.steady_steps
        out["parts"] = ["timed steps", "the last payload as one wire message and back"]
        for phase in ("before", "timed"):
            if phase == "timed":
                torch.cuda.synchronize()
                marker()
            for _ in range(before if phase == "before" else args.steps):
                g.compress(xs[k % 32], err, s, out=o, out_lens=ln, scales=sc, workspace=ws, status=st[:1])
                g.decompress(o, ln, sc, s, y=y, workspace=ws, status=st[1:], path_hint=hint)
                k += 1
        wire = torch.empty(g.wire_bound(), dtype=torch.uint8, device=dev)
        wlen = torch.empty(1, dtype=torch.int64, device=dev)
        wws = g.wire_workspace()
        o2, ln2, sc2 = torch.empty_like(o), torch.empty_like(ln), torch.empty_like(sc)
        st_w = torch.empty(2, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        marker()
        for _ in range(args.steps):
            g.wire_pack(o, ln, sc, wire=wire, wire_len=wlen, workspace=wws, status=st_w[:1])
            g.wire_unpack(wire, out=o2, out_lens=ln2, scales=sc2, workspace=wws, status=st_w[1:])
        torch.cuda.synchronize()
        out["status"] = st.cpu().tolist()
        out["wire_status"] = st_w.cpu().tolist()
        out["wire_bytes"] = int(wlen.item())
        out["bits_per_value"] = round(8.0 * int(ln.sum().item()) / N, 4)
        out["decompress_sequence"] = "dense" if int(hint[0]) else "sparse"
    elif args.profile == "receive":
        bench = Bench(args)
        xs, pay, _, _ = bench.bert_workers(args.steady_steps, False)
        del xs
        torch.cuda.empty_cache()
        g = bench.bert_group
        s = workloads.get("bert_large").s_values[0]
        acc = torch.zeros(g.total, dtype=torch.float32, device=dev)
        wsm = torch.empty(g.accumulate_many_workspace_size(WORKERS), dtype=torch.uint8, device=dev)
        ws = g.workspace()
        st = torch.empty(1, dtype=torch.int32, device=dev)
        out["parts"] = []
        for kind in ("steady", "first"):
            o, ln, sc = pay[kind]
            out["parts"] += [f"{kind}: one call for 8 payloads, dense sequence",
                             f"{kind}: one call for 8 payloads, sparse sequence", f"{kind}: 8 single-payload calls"]
            for route in (1, 0):
                words = [tlc.path_hint() for _ in range(args.steps)]
                for w in words:
                    w[0] = route
                torch.cuda.synchronize()
                marker()
                for k in range(args.steps):
                    g.decompress_accumulate_many(o, ln.reshape(-1), sc.reshape(-1), s, acc, workspace=wsm, status=st,
                                                 path_hint=words[k])
            torch.cuda.synchronize()
            marker()
            for _ in range(args.steps):
                for w in range(WORKERS):
                    g.decompress_accumulate(o[w], ln[w], sc[w], s, acc, workspace=ws, status=st)
        torch.cuda.synchronize()
        out["status"] = int(st.item())
    elif args.profile == "exchange":
        bench = Bench(args)
        xs, pay, _, _ = bench.bert_workers(0, False)
        del xs
        torch.cuda.empty_cache()
        out["parts"] = ["eager calls", "graph capture and warm-up replays", "graph replays"]
        rec = bench.exchange_record(pay["first"], reps=args.steps, marker=marker)
        out["total_ms"] = rec["total_ms"]["median"]
        out["graph_total_ms"] = rec["graph_total_ms"]["median"]
    elif args.profile == "resnet110":
        wl = workloads.get("resnet110")
        sizes, N, s = wl.sizes, wl.total, wl.s_values[0]
        g = tlc.Group(sizes, device=dev)
        x = torch.from_numpy(workloads.generate("resnet110")).to(dev)
        err = torch.zeros(N, dtype=torch.float32, device=dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        o = torch.empty(g.stream_bytes, dtype=torch.uint8, device=dev)
        ln = torch.empty(len(sizes), dtype=torch.int64, device=dev)
        sc = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
        ws = g.workspace()
        st = torch.empty(2, dtype=torch.int32, device=dev)
        hint = tlc.path_hint()
        out["parts"] = ["timed steps"]
        for phase in ("before", "timed"):
            if phase == "timed":
                torch.cuda.synchronize()
                marker()
            for _ in range(args.warmup if phase == "before" else args.steps):
                err.zero_()
                sc.zero_()
                g.compress(x, err, s, out=o, out_lens=ln, scales=sc, workspace=ws, status=st[:1])
                g.decompress(o, ln, sc, s, y=y, workspace=ws, status=st[1:], path_hint=hint)
        torch.cuda.synchronize()
        out["status"] = st.cpu().tolist()
    else:  # calibrate: 1 GiB streaming copy; 4M one-value reads from distinct 128-byte lines
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        n = 1 << 22
        lines = torch.randperm(nbytes // 128, device=dev)[:n].to(torch.int64)
        idx = (lines * 32 + torch.randint(0, 32, (n,), device=dev)).to(torch.int32)
        gdst = torch.empty(n, dtype=torch.float32, device=dev)
        out["parts"] = [f"copy of {nbytes} bytes", f"gather of {n} values from distinct 128-byte lines"]
        torch.cuda.synchronize()
        marker()
        for _ in range(args.steps):
            tlc.copy_probe(src, dst, nbytes)
        torch.cuda.synchronize()
        marker()
        for _ in range(args.steps):
            tlc.gather_probe(src.view(torch.float32), idx, gdst)
        torch.cuda.synchronize()
        out["copy_bytes"] = 2 * nbytes
        out["gather_values"] = n
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20, help="repetitions per configuration record (>= 20)")
    ap.add_argument("--workload", default="bert_large")
    ap.add_argument("--s", type=float, default=None)
    ap.add_argument("--cpu-passes", type=int, default=8, help="oracle passes over the workload (about 10-15 s)")
    ap.add_argument("--pool", type=int, default=32, help="distinct gradient sets cycled through (HBM: 4 B/value each)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle legs (profiling runs)")
    ap.add_argument("--no-records", action="store_true", help="headline only")
    ap.add_argument("--only", choices=RECORDS, default=None,
                    help="run one configuration record and print it (profiling runs)")
    ap.add_argument("--steady-steps", type=int, default=150,
                    help="error-feedback steps before the steady-state figures (0: skip them)")
    ap.add_argument("--profile", choices=PROFILE_PHASES, default=None,
                    help="run one phase alone for a profiler and print a short line (not the benchmark line)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the codec runs on one device and the library has no "
              "transport between GPUs; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from gradient_compression_distributed_lc_amd import tlc, workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile:
        profile_phase(args)
        return
    bench = Bench(args)
    bench.copy_yardstick()
    copy_gbps = bench.copy_gbps

    if args.only:
        log(f"record {args.only}")
        if args.only.startswith("bert_large"):
            steady = args.only == "bert_large_steady"
            xs, pay, _, _ = bench.bert_workers(args.steady_steps if steady else 0, False)
            rec = bench.accumulate_record(pay["steady" if steady else "first"])
        else:
            rec = getattr(bench, f"record_{args.only}")()
        print(json.dumps({"record": args.only, **rec}), flush=True)
        return

    records = {}
    if not args.no_records:
        for name in ("single_1m", "single_16m", "resnet110", "resnet50"):
            log(f"record {name}")
            records[name] = getattr(bench, f"record_{name}")()
            torch.cuda.empty_cache()

    wl = workloads.get(args.workload)
    s = args.s if args.s is not None else wl.s_values[0]
    sizes = wl.sizes
    N = wl.total

    t_gen = time.perf_counter()
    x_host = workloads.generate(args.workload)
    log(f"generated {args.workload}: {len(sizes)} tensors, {N} values in {time.perf_counter() - t_gen:.1f}s")

    group = tlc.Group(sizes, device=dev)
    x0 = torch.from_numpy(x_host).to(dev)
    # A training step sees a fresh gradient: step k compresses the gradient set
    # rotated by k * 1,000,003 elements (same distribution, different values),
    # so the error buffer evolves as it does in training.  Repeating one
    # gradient instead makes the buffer pile up and is not the workload.
    pool = max(1, min(max(args.steps + args.warmup, args.steady_steps), args.pool))
    xs = [x0] + [torch.roll(x0, shifts=k * ROT) for k in range(1, pool)]
    ed = torch.zeros(N, dtype=torch.float32, device=dev)
    yd = torch.empty(N, dtype=torch.float32, device=dev)
    out = torch.empty(group.stream_bytes, dtype=torch.uint8, device=dev)
    lens = torch.empty(len(sizes), dtype=torch.int64, device=dev)
    scales = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
    st_c = torch.empty(1, dtype=torch.int32, device=dev)
    st_d = torch.empty(1, dtype=torch.int32, device=dev)
    ws = group.workspace()
    hint = tlc.path_hint()

    counter = [0]

    def compress_next():
        xd = xs[counter[0] % pool]
        counter[0] += 1
        group.compress(xd, ed, s, out=out, out_lens=lens, scales=scales, workspace=ws, status=st_c)

    def decompress():
        group.decompress(out, lens, scales, s, y=yd, workspace=ws, status=st_d, path_hint=hint)

    def step():
        compress_next()
        decompress()

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

    # timed region: K steps, an event between consecutive steps; the library
    # brackets the dominant kernel with HIP events on its own stream
    tlc.profile_read()
    tlc.profile_only(DOMINANT)
    tlc.profile_enable(True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record()
    for k in range(args.steps):
        step()
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tlc.profile_enable(False)
    kt = tlc.profile_read()
    step_ms = [evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)]
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_per_step = ms_total / args.steps
    last_bits = 8.0 * float(lens.sum().item()) / N
    nonzero_last = float(torch.count_nonzero(yd).item()) / N  # the last step's decoded values: q != 0
    hint_after = "dense" if int(hint[0]) else "sparse"
    # the last timed step's payload as one wire message (outside the timed region)
    wire_rec = wire_record(torch, group, out, lens, scales, N)

    # phase times: compress calls alone, then decompress calls alone, each
    # call bracketed (the error buffer keeps evolving; inputs rotate)
    kp = max(args.steps, 20)
    tc = timed(torch, kp, lambda r, mark: compress_next())
    td = timed(torch, kp, lambda r, mark: decompress())
    comp_st, dec_st = stats([v[0] for v in tc]), stats([v[0] for v in td])
    comp_ms, dec_ms = comp_st["mean"], dec_st["mean"]

    # Pipelined: a worker's receive side does not wait for its own compress,
    # so the decompress of payload k-1 runs on a second stream while batch k
    # is compressed (events order each payload's write, read and reuse).  The
    # same inputs and error state as the timed steps; K compress and K
    # decompress calls between the first launch and the last completion.
    e_keep, c_keep = ed.clone(), counter[0]
    ed.copy_(e_warm)
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    ws_d = group.workspace()
    hint_d = tlc.path_hint()
    hint_d[0] = int(hint[0])
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
        group.decompress(pay[b][0], pay[b][1], pay[b][2], s, y=yd, workspace=ws_d, status=st_pd,
                         path_hint=hint_d, stream=sB)
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
    if (int(st_c.item()), int(st_d.item())) != (0, 0) or first["status"] != (0, 0):
        raise SystemExit(f"device status not ok: {first['status']} / {(int(st_c.item()), int(st_d.item()))}")

    def per_launch(name, table):
        n, ms = table.get(name, (0, 0.0))
        return ms / n if n else 0.0

    dom_ms = per_launch(DOMINANT, kt)
    achieved = DOMINANT_BYTES_PER_ELEM * N / (dom_ms * 1e-3) / 1e9 if dom_ms else 0.0

    # model-delta direction, server side: the workers' sum (the payload decoded
    # into acc, then 7 more copies of it accumulated by one many-payload call),
    # then the server's compress of the 8-worker mean with its own error
    # buffer (carried)
    acc = torch.zeros(N, dtype=torch.float32, device=dev)
    st_a = torch.empty(1, dtype=torch.int32, device=dev)
    st_m = torch.empty(1, dtype=torch.int32, device=dev)
    pay7 = out.unsqueeze(0).expand(7, -1).contiguous()
    lens7, scales7 = lens.repeat(7), scales.repeat(7)
    ws7 = torch.empty(group.accumulate_many_workspace_size(7), dtype=torch.uint8, device=dev)
    hint7 = tlc.path_hint()
    err_srv = torch.zeros(N, dtype=torch.float32, device=dev)
    out_srv = torch.empty(group.stream_bytes, dtype=torch.uint8, device=dev)
    lens_srv = torch.empty(len(sizes), dtype=torch.int64, device=dev)
    scales_srv = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
    st_s = torch.empty(1, dtype=torch.int32, device=dev)

    def server_step():
        group.decompress(out, lens, scales, s, y=acc, workspace=ws, status=st_a)
        group.decompress_accumulate_many(pay7, lens7, scales7, s, acc, workspace=ws7, status=st_m, path_hint=hint7)
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
    if int(st_a.item()) != 0 or int(st_m.item()) != 0 or int(st_s.item()) != 0:
        raise SystemExit(f"device status not ok in the server step: {int(st_a.item())} / {int(st_m.item())} / "
                         f"{int(st_s.item())}")
    srv_step_ms = s0.elapsed_time(s1) / ks
    srv_comp_ms = s1.elapsed_time(s2) / ks
    L_srv = int(lens_srv.sum().item())
    del acc, err_srv, out_srv, pay7, ws7

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
                           "compress_roofline_frac": frac(12.0 * N + nbytes, c_ms, HBM_PEAK_GBPS),
                           "decompress_roofline_frac": frac(4.0 * N + nbytes, d_ms, HBM_PEAK_GBPS)}
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

    # steady state of error feedback: the same steps continued until the error
    # buffer has filled (every encode tile active, denser streams), then 20
    # steps timed one by one
    steady = None
    if args.steady_steps > 0:
        while counter[0] < args.steady_steps:
            step()
        torch.cuda.synchronize()
        after = counter[0]
        tlc.profile_read()
        tlc.profile_only(DOMINANT)
        tlc.profile_enable(True)
        t = timed(torch, max(args.reps, 20), lambda r, mark: (compress_next(), mark(), decompress()))
        tlc.profile_enable(False)
        dom_steady = tlc.profile_read().get(DOMINANT, (0, 0.0))
        if (int(st_c.item()), int(st_d.item())) != (0, 0):
            raise SystemExit("device status not ok in the steady-state steps")
        L_steady = int(lens.sum().item())
        steady = step_record(N, len(sizes), s, L_steady, [a + b for a, b in t], [a for a, _ in t],
                             [b for _, b in t], copy_gbps, dom_steady, B=quartic_bytes(sizes))
        steady["after_steps"] = after
        steady["decompress_sequence"] = "dense" if int(hint[0]) else "sparse"
        # the per-kernel breakdown at this state (every kernel bracketed)
        tlc.profile_only(None)
        tlc.profile_enable(True)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        tlc.profile_enable(False)
        steady["kernels_ms_per_launch_events"] = {k: round(v[1] / v[0], 4) for k, v in tlc.profile_read().items()
                                                  if v[0]}
        steady["kernels_events_note"] = EVENTS_NOTE
        # the same state pipelined over the two streams (10 more steps)
        for b in range(2):
            pay[b][2].copy_(scales)
        hint_d[0] = int(hint[0])
        torch.cuda.synchronize()
        pa.record(sA)
        pipeline(10, counter[0])
        pb.record(sB)
        torch.cuda.synchronize()
        if (int(st_pc.item()), int(st_pd.item())) != (0, 0):
            raise SystemExit("device status not ok in the pipelined steady-state steps")
        steady["pipelined_ms_per_step"] = round(pa.elapsed_time(pb) / 10, 4)
        steady["wire"] = wire_record(torch, group, out, lens, scales, N)
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
    del pay, ws_d, gp, xp, ep, err_pl, out_pl, ws_pl, xs, x0
    torch.cuda.empty_cache()

    L_total = int(first["lens"].sum())
    bits = 8.0 * L_total / N
    bits_hdr = 8.0 * (L_total + 4 * len(sizes)) / N
    alg_bytes_comp = 12.0 * N + L_total + 4 * len(sizes)
    alg_bytes_dec = 4.0 * N + L_total
    # server step: the first payload decoded into acc (4 B/value + stream), 7
    # accumulated in one many-payload call (stream + 8 B per nonzero code
    # each), the mean's compress
    nnz_bytes = 0.0  # the nonzero codes are a few thousand here: below rounding
    alg_bytes_srv = (4.0 * N + L_total) + 7 * (L_total + nnz_bytes) + (12.0 * N + L_srv + 4 * len(sizes))
    gbps = 4.0 * N / (ms_per_step * 1e-3) / 1e9

    cpu = cpu_all = None
    parity = "not checked (--no-cpu)"
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu, streams, Ms, err0 = cpu_baseline(x_host, sizes, s, args.cpu_passes)
        ok = np.array_equal(first["scales"].view(np.uint32), np.asarray(Ms, np.float32).view(np.uint32))
        ok &= np.array_equal(first["err"].view(np.uint32), err0.view(np.uint32))
        for t in range(len(sizes)):
            o = group.offsets[t]
            L = int(first["lens"][t])
            ok &= L == streams[t].size and np.array_equal(first["out"][o:o + L], streams[t])
        parity = "bit-exact vs oracle (streams, M, error buffer; first step)" if ok else "MISMATCH"
        if not ok:
            log("PARITY MISMATCH")
        cpu["host_cpu"] = host_cpu_model()
        log("timing the CPU oracle on all cores")
        cpu_all = cpu_baseline_all_cores(x_host, sizes, s, args.cpu_passes)
    del x_host

    # the 8 workers of the BERT-large configuration: each worker's first step
    # from a zero error buffer (timed), and the receive side's accumulate of
    # the 8 seed-distinct payloads, first-step and steady-state
    if not args.no_records and args.workload == "bert_large":
        log("bert_large workers")
        wxs, wpay, oracle_first, wparity = bench.bert_workers(args.steady_steps, not args.no_cpu)
        # first step per worker: 3 repetitions each, error buffer and M cleared outside the window
        err_w = torch.zeros(N, dtype=torch.float32, device=dev)
        sc_w = torch.zeros(len(sizes), dtype=torch.float32, device=dev)
        hint_w = tlc.path_hint()

        def w_before(r):
            err_w.zero_()
            sc_w.zero_()

        def w_body(r, mark):
            group.compress(wxs[r % WORKERS], err_w, s, out=out, out_lens=lens, scales=sc_w, workspace=ws,
                           status=st_c)
            mark()
            group.decompress(out, lens, sc_w, s, y=yd, workspace=ws, status=st_d, path_hint=hint_w)

        timed(torch, 3, w_body, w_before)
        tlc.profile_read()
        tlc.profile_only(DOMINANT)
        tlc.profile_enable(True)
        tw = timed(torch, 3 * WORKERS, w_body, w_before)
        tlc.profile_enable(False)
        dom_w = tlc.profile_read().get(DOMINANT, (0, 0.0))
        if (int(st_c.item()), int(st_d.item())) != (0, 0):
            raise SystemExit("device status not ok in the workers' first steps")
        L_first = int(wpay["first"][1].sum().item()) // WORKERS
        rec = step_record(N, len(sizes), s, L_first, [a + b for a, b in tw], [a for a, _ in tw],
                          [b for _, b in tw], copy_gbps, dom_w, B=quartic_bytes(sizes))
        rec["how"] = ("worker w's set (seed 500+w), compress from a zero error buffer and no previous M, "
                      "then decompress; 3 repetitions per worker, w = 0..7")
        rec["decompress_sequence"] = "dense" if int(hint_w[0]) else "sparse"
        if wparity is not None:
            rec["parity"] = ("bit-exact vs oracle (8 workers' streams and M)" if wparity else "MISMATCH")
        del err_w, sc_w, wxs
        torch.cuda.empty_cache()
        log("accumulate of the 8 first-step payloads")
        rec["accumulate_8"] = bench.accumulate_record(wpay["first"], oracle_first if not args.no_cpu else None)
        log("exchange of the 8 first-step payloads, one GPU's share")
        rec["exchange_8"] = bench.exchange_record(wpay["first"])
        records["bert_large_first_step"] = rec
        if steady is not None:
            log("accumulate of the 8 steady-state payloads")
            steady["accumulate_8"] = bench.accumulate_record(wpay["steady"])
            steady["accumulate_8"]["how"] = (f"worker w's payload after {args.steady_steps} steps of its own "
                                             f"error feedback (step k on its set rotated by "
                                             f"(k mod 32) * {ROT})")
        del wpay
    if steady is not None:
        records["bert_large_steady"] = steady

    traffic = stored_traffic(args.workload)
    sm = stats(step_ms)
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": sm["median"],
        "ms_per_step_min": sm["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "tensors": len(sizes), "values": N, "s": s,
                   "values_dist": wl.description, "parallelism": "single GPU",
                   "steps_timed": f"steps {c_warm + 1}..{c_warm + args.steps} of a carried error buffer, "
                                  f"inputs cycled through {pool} rotated copies of the set"},
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
        "compress_ms_median": comp_st["median"],
        "decompress_ms_median": dec_st["median"],
        "decompress_sequence_after_timed_steps": hint_after,
        "compress_GBps_fp32_in": round(4.0 * N / (comp_ms * 1e-3) / 1e9, 1) if comp_ms else None,
        "decompress_GBps_fp32_in": round(4.0 * N / (dec_ms * 1e-3) / 1e9, 1) if dec_ms else None,
        "path_roofline_frac": frac(alg_bytes_comp + alg_bytes_dec, ms_per_step, HBM_PEAK_GBPS),
        "compress_roofline_frac": frac(alg_bytes_comp, comp_ms, HBM_PEAK_GBPS),
        "compress_roofline_frac_nominal_12p3B": frac(12.3 * N, comp_ms, HBM_PEAK_GBPS),
        "decompress_roofline_frac": frac(alg_bytes_dec, dec_ms, HBM_PEAK_GBPS),
        "server_step_ms": round(srv_step_ms, 4),
        "server_step_roofline_frac": frac(alg_bytes_srv, srv_step_ms, HBM_PEAK_GBPS),
        "server_compress_ms": round(srv_comp_ms, 4),
        "server_compress_roofline_frac": frac(12.0 * N + L_srv + 4 * len(sizes), srv_comp_ms, HBM_PEAK_GBPS),
        "server_bits_per_value": round(8.0 * L_srv / N, 4),
        "copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        # the same algorithmic bytes against the measured copy rate instead of the nominal peak
        "path_copy_ceiling_frac": frac(alg_bytes_comp + alg_bytes_dec, ms_per_step, copy_gbps),
        "dominant_copy_ceiling_frac": round(achieved / copy_gbps, 4) if copy_gbps else None,
        "bits_per_value_last_step": round(last_bits, 4),
        "nonzero_code_fraction_last_step": round(nonzero_last, 6),
        "pipelined": {"ms_per_step": round(pipe_ms, 4), "GBps_fp32_in": round(4.0 * N / (pipe_ms * 1e-3) / 1e9, 1),
                      "path_roofline_frac": frac(alg_bytes_comp + alg_bytes_dec, pipe_ms, HBM_PEAK_GBPS),
                      "how": "compress of batch k on one stream, decompress of payload k-1 on another "
                             "(receive side overlapped with the send side), same inputs and error state "
                             "as the timed steps"},
        "configs": records,
        "ablations": ablations,
        "wire": wire_rec,
        "kernels_ms_per_launch_events": {k: round(v[1] / v[0], 4) for k, v in kt_all.items() if v[0]},
        "kernels_events_note": EVENTS_NOTE,
        "wall_s_timed": round(wall, 3),
        "kernel_source": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
