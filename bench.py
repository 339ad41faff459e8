"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--cold] [--pass fwd|bwd|decode] [--fp8] [--mod [--mod-cached]]

A step is one attn_fwd call over one batch of seeded synthetic input already resident in HBM:
the V transpose-pack kernel, the block-table kernel (masked kinds) and the forward kernel.
W untimed steps, then exactly K timed steps bracketed by a device synchronisation on both
sides, timed with HIP events on the stream the kernels run on.  Prints one JSON line.

Default workload: causal attention, B=1, H=32, N=16384, d=128 (the configuration the
throughput target is quoted on).  The metric counts only unmasked FLOPs: 4*d per allowed
(query, key) pair (2d for Q K^T, 2d for P V).

The "roofline" object is for the forward kernel alone: algorithmic FLOPs per launch divided by
its average duration, measured with a HIP event pair the library records around that kernel on
the same stream, against the published dense bf16 MFMA peak of MI355X.

--cold writes a 512 MiB buffer before every step (more than L2 and the Infinity Cache hold) and
times each call alone with its own event pair: the cold-cache figure for the short, HBM-bound
workloads.  The default is warm: back-to-back calls.

--fp8 times the FP8 forward pass (ATTN_PREC_FP8: Q K^T from E4M3 codes of Q and K with one
scale per 256-row Q tile and per 64-key K tile, P V in fp16).  A step then also holds the K
quantization kernel.  Half of the counted FLOPs (Q K^T) run at the fp8 MFMA rate and half (P V)
at the fp16 rate, so the kernel's peak is the harmonic mix of the two published peaks:
1 / (0.5 / 5000 + 0.5 / 2500) = 3333 TFLOP/s.

--mod runs the same workload through a runtime-compiled modification (attn_mod_create /
attn_fwd_mod): the workload's score variant and mask written as HIP C++ functions, compiled by
hipRTC when the benchmark starts.  A step then also holds the two mask-table kernels, unless
--mod-cached is given: then the warmup's first call builds the table and every timed step calls
attn_fwd_mod_cached, which reuses it (the table depends only on the mask, B, N and parameters).

The "cpu_baseline" object times the fp64 CPU oracle (a plain, untuned reference) on the host
cores on a bounded sample of the same workload, in the same unit.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
PEAK_FP8_TFLOPS = 5000.0   # MI355X published dense fp8 MFMA peak
# FP8 forward: Q K^T (half the FLOPs) on fp8 MFMAs, P V (the other half) on fp16 MFMAs
PEAK_FP8_FWD_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0      # MI355X published HBM3E bandwidth
MAX_SCLK_MHZ = 2400.0      # MI355X peak engine clock, the one the MFMA peak is quoted at
METRIC = "attention fwd TFLOP/s (unmasked FLOPs) and % of MFMA peak, 1 MI355X"
DEFAULT_WORKLOAD = "causal_h32_n16384_d128"
KERNEL_SOURCES = ["exact_io_aware_21_amd/csrc/fwd.hip", "exact_io_aware_21_amd/csrc/fwd_kernel.h",
                  "exact_io_aware_21_amd/csrc/kcommon.h", "exact_io_aware_21_amd/csrc/tiles.h",
                  "exact_io_aware_21_amd/csrc/launch.h", "exact_io_aware_21_amd/csrc/hipdefs.h"]


def allowed_pairs(w, doc_offsets=None):
    """Allowed (query, key) pairs over all batch entries and heads, in closed form."""
    N = w.N
    if w.mask == "none":
        per = [N * N] * w.B
    elif w.mask == "causal":
        per = [N * (N + 1) // 2] * w.B
    elif w.mask == "window":
        W = w.window
        m = min(W, N)
        per = [m * (m + 1) // 2 + (N - m) * W] * w.B
    else:
        per = []
        for row in doc_offsets:
            o = [int(x) for x in row]
            per.append(sum((o[r + 1] - o[r]) * (o[r + 1] - o[r] + 1) // 2 for r in range(len(o) - 1)))
    return sum(per) * w.H


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(workload):
    """HBM bytes per launch of the forward kernel from committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_fwd_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_avg(path, counter, kernel_prefix):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and r["Kernel_Name"].startswith(kernel_prefix)]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel {kernel_prefix!r} in {path}")
    return sum(vals) / len(vals)


def write_traffic(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """Turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) into HBM bytes per
    launch of the forward kernel.  Each counter is scaled by the factor that makes it read the
    known byte count of the microbenchmark's plain copy kernel (copy_bytes read and written)."""
    fwd = "void attn::(anonymous namespace)::fwd_kernel"
    copy = "copy_kernel"
    f_scale = copy_bytes / (_pmc_avg(copy_fetch_csv, "FETCH_SIZE", copy) * 1024)
    w_scale = copy_bytes / (_pmc_avg(copy_write_csv, "WRITE_SIZE", copy) * 1024)
    rd = _pmc_avg(fetch_csv, "FETCH_SIZE", fwd) * 1024 * f_scale
    wr = _pmc_avg(write_csv, "WRITE_SIZE", fwd) * 1024 * w_scale
    rec = {"workload": workload, "kernel": "fwd_kernel", "source_sha256": kernel_source_hash(),
           "fetch_scale": f_scale, "write_scale": w_scale, "read_bytes_per_launch": rd,
           "write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr}
    path = os.path.join(ROOT, "profiles", f"traffic_fwd_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


class SclkSampler:
    """Samples the GPU core clock in a background thread while a timed region runs: the current
    level of the driver's `pp_dpm_sclk` file in sysfs (the line marked '*'), every `period_s`.
    The published MFMA peak assumes the 2.4 GHz maximum clock; under sustained matrix-core load the
    clock settles lower, and this records where."""

    # Steps shorter than this are not sampled: on short workloads, whose loop is bound by
    # launch overhead, the sysfs reads (each a query of the power-management firmware by the
    # driver) slowed the timed loop several-fold (plain_n256_d64: 97 us per step with sampling,
    # 18 us without), so the sample would change what it measures.
    MIN_STEP_MS = 0.2

    def __init__(self, period_s=0.005, started=None, step_ms=None):
        """started: optional callable; samples are kept only once it returns True (the bench
        passes the completion query of the first timed step's end event, so that the readings
        taken while the driver's value still lags the idle clock are dropped).  step_ms: the
        step time seen in the warm-up; below MIN_STEP_MS nothing is sampled."""
        import glob
        import threading
        self.period_s = period_s
        self.started = started
        self.dropped = 0
        self.samples = []
        self.path = None
        self.skipped = step_ms is not None and step_ms < self.MIN_STEP_MS
        for path in ([] if self.skipped else
                     sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))):
            if self._read(path) is not None:
                self.path = path
                break
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            mhz = self._read(self.path)
            if mhz is not None:
                if self.started is None or self.started():
                    self.samples.append(mhz)
                else:
                    self.dropped += 1
            self._stop.wait(self.period_s)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if self.skipped:
            return {"skipped": f"steps under {self.MIN_STEP_MS} ms: sysfs clock reads slow the "
                               "launch loop of such short steps"}
        if not self.samples:
            return None
        x = sorted(self.samples)
        return {"median": x[len(x) // 2], "min": x[0], "max": x[-1], "samples": len(x),
                "dropped_before_first_step": self.dropped, "source": self.path}


def clock_scaled_peak(rec, peak, achieved):
    """Adds to the clock record the MFMA peak scaled to the median sampled clock and the fraction
    of it reached.  The sysfs clock is read by the driver on its own schedule and can lag the
    hardware, so a fraction above 1 (physically impossible) marks the reading as stale: the
    fraction is then left out and the record says why."""
    if not rec or "skipped" in rec:
        return rec
    scaled = peak * rec["median"] / MAX_SCLK_MHZ
    rec["mfma_peak_at_median_tflops"] = round(scaled, 1)
    frac = achieved / scaled
    if frac <= 1.0:
        rec["frac_of_that_peak"] = round(frac, 4)
    else:
        rec["frac_of_that_peak"] = None
        rec["note"] = ("sampled clock lags the hardware (the kernel ran faster than the peak at "
                       "that clock allows); not used")
    return rec


KEV_EVERY = 16    # kernel event pairs on every 16th step of a short workload (see the loop)
GRAPH_CALLS = 20  # calls captured per graph in --graph mode (a replay's own launch cost is shared)


def bench_graph(args, w, inp, call):
    """--graph: GRAPH_CALLS calls captured in one HIP graph (the calls allocate nothing and
    issue no memset, so they can be captured), replayed until at least K calls have run, timed
    with a HIP event pair on the replaying stream.  The per-call time is the device's; the
    kernel-only event pair is not recorded inside the graph, so the roofline is taken on the
    whole call."""
    import torch
    G = max(1, min(args.steps, GRAPH_CALLS))
    reps = -(-args.steps // G)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(G):
            call()
    for _ in range(max(1, -(-args.warmup // G))):
        g.replay()
    torch.cuda.synchronize()
    K = reps * G
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    flops = 4.0 * w.d * allowed_pairs(w, inp["doc_offsets"])
    hbm_bytes = w.B * w.H * w.N * (4 * w.d * 2 + 4)
    peak = PEAK_FP8_FWD_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    value = flops / (step_ms * 1e-3) / 1e12
    if flops / hbm_bytes > peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(value, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(value / peak, 4), "traffic": None}
    else:
        gbs = hbm_bytes / (step_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "us_per_call": round(1e3 * step_ms, 2),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8_e4m3+fp16" if args.fp8 else "bf16+fp16",
           "data": "synthetic (seeded N(0, sigma^2) Q/K/V rounded to bf16)",
           "config": {"workload": ("graph_fp8_" if args.fp8 else "graph_") + w.name, "B": w.B,
                      "H": w.H, "N": w.N, "d": w.d, "mask": w.mask,
                      "timing": f"HIP graph of {G} calls, replayed {reps} times; device time per call"},
           "roofline": roof}
    print(json.dumps(out), flush=True)


def mod_source(w):
    """The workload's variant as a runtime-compiled modification: (source, flags, params), params
    an fp32 array (ALiBi slopes; nothing else is needed by these variants)."""
    import numpy as np
    from exact_io_aware_21_amd import inputs
    score, mask = [], None
    if w.softcap:
        score.append(f"s = {float(w.softcap)!r}f * tanhf(s / {float(w.softcap)!r}f);")
    if w.alibi:
        score.append("s -= p[h] * (float)(i - j);")
    if w.mask == "causal":
        mask = "return j <= i;"
    elif w.mask == "window":
        mask = f"return j <= i && i - j < {int(w.window)};"
    elif w.mask != "none":
        raise SystemExit(f"--mod: no runtime-compiled form of the {w.mask} mask in this benchmark")
    src, flags = "", 0
    if score:
        src += ("__device__ float attn_score_mod(float s, int b, int h, int i, int j, "
                "const float *p) { " + " ".join(score) + " return s; }\n")
        flags |= 1
    if mask:
        src += "__device__ bool attn_mask_mod(int b, int i, int j, const float *p) { " + mask + " }\n"
        flags |= 2
    if w.softcap:
        flags |= 4  # ATTN_MODF_MAX_FIRST: a soft-cap moves row maxima often
    if not flags:
        raise SystemExit("--mod: the workload has no score modification or mask")
    params = inputs.alibi_slopes(w.H) if w.alibi else np.zeros(1, dtype=np.float32)
    return src, flags, params


def cpu_baseline(w, inp, budget_s=20.0, chunk=2048, fp8=False):
    """The fp64 oracle on host cores, over whole heads in order (query rows in chunks of `chunk`)
    until `budget_s` has elapsed.  Throughput in the metric's unit (unmasked TFLOP/s).  fp8: Q and
    K of each head are block-quantized and dequantized by the oracle first (timed as well)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i["num_threads"] for i in threadpool_info() if i["user_api"] == "blas"]
                      or [1])
    except Exception:
        threads = 1
    cols = np.arange(w.N)
    t0 = time.perf_counter()
    pairs = 0
    rows_done = 0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        q = oracle.decode_bf16(inp["q"][b:b + 1, h:h + 1])
        k = oracle.decode_bf16(inp["k"][b:b + 1, h:h + 1])
        v = oracle.decode_bf16(inp["v"][b:b + 1, h:h + 1])
        if fp8:
            q = oracle.dequantize_blocks(*oracle.quantize_blocks(q, 256), 256)
            k = oracle.dequantize_blocks(*oracle.quantize_blocks(k, 64), 64)
        offs = None if inp["doc_offsets"] is None else inp["doc_offsets"][b:b + 1]
        slopes = None if inp["slopes"] is None else inp["slopes"][h:h + 1]
        for r0 in range(0, w.N, chunk):
            rows = np.arange(r0, min(r0 + chunk, w.N))
            oracle.attention(q, k, v, float(inp["scale"]), mask=w.mask, window=w.window,
                             softcap=float(w.softcap), slopes=slopes, doc_offsets=offs,
                             rows=rows)
            pairs += int(oracle.allowed(rows, cols, w.N, w.mask, w.window,
                                        None if offs is None else offs[0]).sum())
            rows_done += rows.size
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": 4.0 * w.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 {'FP8 ' if fp8 else ''}oracle on {rows_done // w.N} whole head(s) "
                      f"of {w.name} "
                      f"({rows_done} query rows x {w.N} keys, {pairs} allowed pairs), "
                      f"{dt:.1f} s wall"}


def bench_bwd(args, w, inp, q, k, v, o, lse, var, slopes, offs, dev):
    """Times attn_bwd on the workload (after one attn_fwd for O and L): K timed steps, with the
    library's event pair around the two main backward kernels."""
    import numpy as np
    import torch

    from exact_io_aware_21_amd import attn, inputs

    g = torch.from_numpy(inputs.draw_dout(w.B, w.H, w.N, w.d, w.seed).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    attn.attn_fwd(q, k, v, o, lse, inp["scale"], var, window=w.window, softcap=w.softcap,
                  alibi_slopes=slopes, doc_offsets=offs)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = attn.alloc_bwd_workspace(w.B, w.H, w.N, w.d, var, dev)
    kw = dict(window=w.window, softcap=w.softcap, alibi_slopes=slopes, doc_offsets=offs,
              workspace=ws)
    for _ in range(args.warmup):
        attn.attn_bwd(q, k, v, o, lse, g, dq, dk, dv, inp["scale"], var, **kw)
    K = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in kev:
        a.record()
        b.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sclk = SclkSampler(started=kev[0][1].query)
    with sclk:
        start.record()
        for i in range(K):
            attn.attn_bwd(q, k, v, o, lse, g, dq, dk, dv, inp["scale"], var,
                          timing_events=kev[i], **kw)
        end.record()
        torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    kern_ms = sum(a.elapsed_time(b) for a, b in kev) / K
    flops = 10.0 * w.d * allowed_pairs(w, inp["doc_offsets"])
    achieved = flops / (kern_ms * 1e-3) / 1e12
    out = {
        "metric": "attention bwd TFLOP/s (unmasked FLOPs, 10 d per allowed pair) and % of MFMA "
                  "peak, 1 MI355X",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, sigma^2) Q/K/V and N(0, 1) dO rounded to bf16)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": w.mask,
                   "window": w.window, "alibi": w.alibi, "softcap": w.softcap,
                   "unmasked_gflop": round(flops / 1e9, 3), "bwd_kernels_ms": round(kern_ms, 4),
                   "sclk_mhz": sclk.summary()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(out), flush=True)


DECODE_DEFAULT = "decode_b8h32_len2k_14k_d128_p64"


def bench_decode(args):
    """Times attn_decode (split and merge kernels, the library's event pair around them) on a
    paged-cache workload; the metric is GB/s of compulsory traffic: every cached K and V row of
    every sequence read once, Q read, O (bf16) and L written."""
    import numpy as np
    import torch

    from exact_io_aware_21_amd import attn, inputs

    name = DECODE_DEFAULT if args.workload == DEFAULT_WORKLOAD else args.workload
    w = inputs.DECODE_WORKLOADS[name]
    x = inputs.make_paged_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, kc, vc = to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"])
    table = torch.from_numpy(x["page_table"]).to(dev)
    lens = torch.from_numpy(x["seq_lens"]).to(dev)
    o = torch.empty(w.B, w.H, w.Lq, w.d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.H, w.Lq, dtype=torch.float32, device=dev)
    ws = attn.alloc_decode_workspace(w.B, w.H, w.Lq, w.d, w.page, table.shape[1], dev)
    kw = dict(causal=w.causal, workspace=ws)
    for _ in range(args.warmup):
        attn.attn_decode(q, kc, vc, table, lens, o, lse, float(x["scale"]), **kw)
    K = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in kev:
        a.record()
        b.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sclk = SclkSampler(started=kev[0][1].query)
    with sclk:
        start.record()
        for i in range(K):
            attn.attn_decode(q, kc, vc, table, lens, o, lse, float(x["scale"]),
                             timing_events=kev[i], **kw)
        end.record()
        torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    kern = sorted(a.elapsed_time(b) for a, b in kev)
    kern_ms = sum(kern) / K
    positions = int(x["seq_lens"].astype(np.int64).sum())
    hbm_bytes = positions * w.H * w.d * 2 * 2 + w.B * w.H * w.Lq * (w.d * 2 * 2 + 4)
    gbs = hbm_bytes / (kern_ms * 1e-3) / 1e9
    out = {
        "metric": "attention decode GB/s (compulsory bytes: every cached K and V row once, q, "
                  "O, L), 1 MI355X",
        "value": round(hbm_bytes / (step_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, 1) q and paged K/V cache rounded to bf16; "
                "uniform sequence lengths; scattered pages)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "d": w.d,
                   "page": w.page, "causal": w.causal,
                   "seq_lens": [int(v) for v in x["seq_lens"]],
                   "compulsory_hbm_bytes": hbm_bytes, "decode_kernels_ms": round(kern_ms, 4),
                   "decode_kernels_ms_median": round(kern[K // 2], 4),
                   "decode_kernels_ms_min": round(kern[0], 4), "sclk_mhz": sclk.summary()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, x)
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(w, x, budget_s=20.0):
    """The fp64 decoding oracle on host cores, one sequence at a time until `budget_s` has
    elapsed; GB/s of the same compulsory bytes."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i["num_threads"] for i in threadpool_info() if i["user_api"] == "blas"]
                      or [1])
    except Exception:
        threads = 1
    kc, vc = oracle.decode_bf16(x["k_cache"]), oracle.decode_bf16(x["v_cache"])  # inputs, once
    t0 = time.perf_counter()
    done, nbytes = 0, 0
    for b in range(w.B):
        q = oracle.decode_bf16(x["q"][b:b + 1])
        oracle.decode_attention(q, kc, vc, x["page_table"][b:b + 1], x["seq_lens"][b:b + 1],
                                float(x["scale"]), w.causal)
        done += 1
        nbytes += int(x["seq_lens"][b]) * w.H * w.d * 4 + w.H * w.Lq * (w.d * 4 + 4)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 decoding oracle on {done} of {w.B} sequences of {w.name} "
                      f"(all {w.H} heads), {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)  # also lets the clock settle
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB buffer before every step (evicts L2 and the 256 MB "
                         "Infinity Cache) and time each call alone: the cold-cache HBM figure")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "decode"), default="fwd",
                    help="bwd: time attn_bwd instead (10 d FLOPs per allowed pair; no CPU leg); "
                         "decode: time attn_decode on a paged-cache workload (GB/s)")
    ap.add_argument("--mod", action="store_true",
                    help="run the workload's variant as a runtime-compiled modification")
    ap.add_argument("--mod-cached", action="store_true",
                    help="with --mod: build the mask table once, time attn_fwd_mod_cached")
    ap.add_argument("--graph", action="store_true",
                    help="capture one call in a HIP graph and time K replays: the device-side "
                         "time per call, without the host's per-call overhead")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward pass (ATTN_PREC_FP8; no score modifications)")
    ap.add_argument("--traffic", nargs=4, metavar=("FWD_FETCH", "FWD_WRITE", "COPY_FETCH",
                                                    "COPY_WRITE"),
                    help="write profiles/traffic_fwd_<workload>.json from rocprofv3 counter CSVs")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(args.workload, *args.traffic, copy_bytes=float(1 << 30))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the forward pass here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from exact_io_aware_21_amd import attn, inputs

    if args.which == "decode":
        bench_decode(args)
        return
    w = inputs.WORKLOADS[args.workload]
    inp = inputs.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o = torch.empty(w.B, w.H, w.N, w.d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    slopes = None if inp["slopes"] is None else torch.from_numpy(inp["slopes"]).to(dev)
    offs = None if inp["doc_offsets"] is None else torch.from_numpy(inp["doc_offsets"]).to(dev)
    var = attn.variant_bits(w.mask, w.alibi, w.softcap > 0, fp8=args.fp8)
    if args.fp8 and args.which != "fwd":
        raise SystemExit("--fp8 applies to the forward pass only")
    ws = attn.alloc_workspace(w.B, w.H, w.N, w.d, var, dev)
    kw = dict(window=w.window, softcap=w.softcap, alibi_slopes=slopes, doc_offsets=offs,
              workspace=ws)

    if args.which == "bwd":
        bench_bwd(args, w, inp, q, k, v, o, lse, var, slopes, offs, dev)
        return

    compile_s = None
    if args.mod_cached and not args.mod:
        raise SystemExit("--mod-cached needs --mod")
    if args.mod:
        if args.fp8:
            raise SystemExit("--mod and --fp8 are separate paths")
        src, flags, params = mod_source(w)
        t0 = time.perf_counter()
        mod = attn.AttnMod(src, flags, w.d)
        compile_s = time.perf_counter() - t0
        mparams = torch.from_numpy(params).to(dev)
        mws = mod.alloc_workspace(w.B, w.H, w.N, dev)
        built = []

        def call(timing_events=None):
            mod.fwd(q, k, v, o, lse, inp["scale"], mparams, workspace=mws,
                    timing_events=timing_events, cached_table=args.mod_cached and bool(built))
            built.append(True)
    else:
        # checked and marshalled once: each step is one C call (a serving loop's calling
        # pattern); under --graph the calls go to the capturing stream, else to this one
        call = attn.FwdPlan(q, k, v, o, lse, inp["scale"], var,
                            stream=None if args.graph else torch.cuda.current_stream(), **kw)

    t0 = time.perf_counter()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / args.warmup if args.warmup else None

    if args.graph:
        bench_graph(args, w, inp, call)
        return

    K = args.steps
    # Kernel event pairs on every step, or on every KEV_EVERY-th step when a step takes under
    # SclkSampler.MIN_STEP_MS: two event records cost about as much as such a step's kernel
    # (plain_n256_d64: 13.3 us per step with a pair on every step, the kernel itself ~6 us).
    ev_every = KEV_EVERY if warm_ms is not None and warm_ms < SclkSampler.MIN_STEP_MS else 1
    kev_steps = list(range(0, K, ev_every))
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in kev_steps]
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K if args.cold else 0)]
    for a, b in kev + cev:  # torch creates the underlying hipEvent on the first record
        a.record()
        b.record()
    # the kernel event pairs, marshalled before the timed loop where the call takes them so
    tev = [call.events(e) for e in kev] if isinstance(call, attn.FwdPlan) else kev
    step_ev = [None] * K
    for j, i in enumerate(kev_steps):
        step_ev[i] = tev[j]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sclk = SclkSampler(started=kev[0][1].query, step_ms=warm_ms)
    with sclk:  # sampled from the end of the first timed step until the device has finished
        start.record()
        for i in range(K):
            if args.cold:
                flush.fill_(i & 255)
                cev[i][0].record()
            call(step_ev[i])
            if args.cold:
                cev[i][1].record()
        end.record()
        torch.cuda.synchronize()
    if args.cold:  # the flush is not part of a step: time the calls alone
        step_ms = sum(a.elapsed_time(b) for a, b in cev) / K
    else:
        step_ms = start.elapsed_time(end) / K
    kern = sorted(a.elapsed_time(b) for a, b in kev)
    kern_ms = sum(kern) / len(kern)

    flops = 4.0 * w.d * allowed_pairs(w, inp["doc_offsets"])
    hbm_bytes = w.B * w.H * w.N * (4 * w.d * 2 + 4)  # Q, K, V read; O (bf16) and L written
    value = flops / (step_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(w.name)
    peak = PEAK_FP8_FWD_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    sclk_rec = clock_scaled_peak(sclk.summary(), peak, achieved)
    mfma_bound = flops / hbm_bytes > peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if args.fp8 else traffic}
        if args.fp8:
            roof["peak_note"] = ("Q K^T on fp8 MFMAs (5000 TFLOP/s), P V on fp16 MFMAs "
                                 "(2500 TFLOP/s), half the FLOPs each")
    else:
        gbs = hbm_bytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # Q K^T runs on bf16 (FP8: E4M3) MFMA operands and P V on fp16 ones (P <= 2^8 by the
        # lazy rescale; V converted exactly from bf16), both accumulating in fp32
        "dtype": "fp8_e4m3+fp16" if args.fp8 else "bf16+fp16",
        "data": "synthetic (seeded N(0, sigma^2) Q/K/V rounded to bf16)",
        "config": {"workload": ("fp8_" if args.fp8 else "mod_" if args.mod else "") + w.name,
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": w.mask,
                   "window": w.window, "alibi": w.alibi, "softcap": w.softcap,
                   "unmasked_gflop": round(flops / 1e9, 3),
                   "fwd_kernel_ms": round(kern_ms, 4),
                   "fwd_kernel_ms_median": round(kern[len(kern) // 2], 4),
                   "fwd_kernel_ms_min": round(kern[0], 4),
                   "kernel_events": "every step" if ev_every == 1 else
                                    f"every {ev_every}th step ({len(kern)} of {K})",
                   "cache": "cold: 512 MiB written before each call" if args.cold else "warm",
                   "compulsory_hbm_bytes": hbm_bytes,
                   "sclk_mhz": sclk_rec,
                   **({"runtime_compiled_modification": {
                       "compile_s": round(compile_s, 2),
                       "mask_table": "built once" if args.mod_cached else "built every step"}}
                      if args.mod else {})},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, fp8=args.fp8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
