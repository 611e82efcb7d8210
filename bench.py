"""Benchmark of the KDA forward pass on one MI355X.

One step = one pass of the whole hot path on resident synthetic inputs:
  * a chunked prefill of 1 x 1,048,576 tokens, H = 32, d_k = d_v = 128, bf16
    (log_alpha = -0.05 softplus(N(0,1)), beta = sigmoid(N(0,1)), zero state);
  * 64 decode steps of 256 sequences x 32 heads, d = 128, on a resident fp32
    state (512 MiB) updated in place.
``value`` is the prefill throughput in tokens/s (B*T per second, each token
counted once across its 32 heads), from HIP events around the prefill call
on the library's stream.  The decode figures (sequence-steps/s and state
GB/s) are reported beside it.  ``roofline`` is the prefill against MI355X
HBM (8 TB/s): algorithmic bytes per call = 1540 B per head-token (bf16 q, k,
v, o; fp32 log_alpha; fp32 beta) plus the final states, over the measured
call time; d2d_copy_GBps is a 2 GiB device-to-device copy (the runtime's
copy kernel) measured in the same process, a reference point rather than an
upper bound (the decode kernel streams faster), and mfma_busy_pct the
rocprofv3 MfmaUtil of each kernel from the committed counter summary.  For this workload (32 (sequence,
head) pairs) the library takes
its two-pass path: one call enqueues, per block of chunks, a prep kernel
(chunk-parallel) and a carry kernel (the serial state walk); the roofline
covers the whole call, and the rocprofv3 summary splits it per kernel.

serving: the prefill recording a state snapshot every 4096 tokens (prefix
caching), the 64 decode steps on states held in scattered slots of a
512-state pool (continuous batching), and speculative decoding of 4 draft
tokens per sequence: one call verifies them (outputs, states only read),
one commits an accepted prefix of 0..4 tokens (states advanced), each
reading a state once, beside the time of 4 single decode steps.

other_prefill_workloads: the tiny fp32 batch, the 4 x 4096-token batch and
the 64-sequence varlen batch, each timed alone against its algorithmic
bytes (the library picks the path); the varlen batch also from raw inputs
(front_end: the fused input front-end on the fused path).

front_end: the same prefill from raw inputs (the fused input front-end:
q, k normalised in the kernel, bf16 gate and beta pre-activations, 1282
algorithmic bytes per head-token).

backward: the gradients of that prefill (kda_bwd; a random dO, zero dhT),
which recompute the forward, against 2824 algorithmic bytes per head-token
(q, k, v, dO and gates read, dq, dk, dv and gate gradients written), with
the time relative to the forward call.

gate_variants: the same prefill as Gated DeltaNet (one gate per (token,
head), 1032 B per head-token) and DeltaNet (no gate, 1028 B), timed the
same way, each against the HBM peak.

cpu_baseline: the fp64 oracle on a bounded sample of the same workload (a
few heads over the first tokens), on the host's cores, scaled to tokens/s of
the full 32-head layer.  It doubles as a parity spot check of those outputs.

counters: ``python bench.py --counters`` prints no JSON; it runs, once
each, the launches the committed rocprofv3 counter summaries (profiles/)
are taken on -- the long-context prefill over its first 512 chunks (8
blocks of 64), the 4 x 4096 batch, the 64-sequence varlen batch, one decode
step of 256 x 32 states, the backward of the 512-chunk prefill, and a 512
MiB device copy whose counter readings calibrate the rest -- under
``rocprofv3 --pmc <counter> -- python3 bench.py --counters``.

digest: ``python bench.py --digest DIR`` reads the rocprofv3 output of
those runs (DIR/ks: --kernel-trace; DIR/pmc_<counter>: one --pmc counter
each, FETCH_SIZE, WRITE_SIZE, MfmaUtil), splits the dispatches into the
workloads above (each is a run of this library's kernels between the torch
kernels that generate the next inputs), scales FETCH_SIZE and WRITE_SIZE by
the copy's readings, and writes profiles/traffic.json (with a digest of the
kernel sources: the bench reports the figures only while it matches) and a
markdown summary; with DIR/bench_ks (a --kernel-trace --stats run of the
bench itself) also the bench's kernel statistics.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only-backward] [--counters] [--digest DIR]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_BYTES_PER_HT = 1540          # q,k,v,o bf16 (4 x 256) + log_alpha fp32 (512) + beta (4)
DECODE_BYTES_PER_HS = 2 * 128 * 128 * 4 + 1540   # state read + write, token inputs, output
PREFILL_KERNELS = "prefill_wy_prep_kernel<0, false> + prefill_wy_carry_kernel<16, false>"
DECODE_KERNEL = "decode_step_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--cpu-tokens", type=int, default=1048576)
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the prefill gradients (for profiling)")
    ap.add_argument("--digest", default=None,
                    help="summarise the rocprofv3 output of the --counters runs in this folder")
    ap.add_argument("--counters", action="store_true",
                    help="run the launches the rocprofv3 counter summaries cover, once each")
    ap.add_argument("--chunks", type=int, default=512,
                    help="--counters: 64-token chunks of the long-context prefill")
    return ap.parse_args()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_counter_workloads(torch, kda, gen, chunks):
    """One launch of each workload the counter summaries cover, in a fixed
    order (rocprofv3 lists dispatches in order): long-context prefill of
    `chunks` chunks (32 heads, two-pass: 2 kernels per block of 64 chunks),
    batch4_t4096 (two-pass), varlen_n64 (fused), one decode step, the
    backward of the long-context prefill, then a 512 MiB device copy."""
    dev = "cuda"
    T, H, d = 64 * chunks, 32, 128
    inp = gen.prefill_inputs([T], H, d, d, "bf16", "softplus", state_std=0.0, seed=2, device=dev)
    print("counters: long prefill T=%d H=%d" % (T, H), flush=True)
    kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    torch.cuda.synchronize()
    for wname in ("batch4_t4096", "varlen_n64"):
        wo = gen.WORKLOADS[wname]
        io = gen.workload_prefill_inputs(wo, seed=11, device=dev)
        print("counters: %s prefill" % wname, flush=True)
        kda.prefill(io["q"], io["k"], io["v"], io["log_alpha"], io["beta"], h0=io["h0"],
                    cu_seqlens=io["cu_seqlens"], max_seqlen=max(io["lengths"]))
        torch.cuda.synchronize()
        del io
    S = gen.decode_state(256, H, d, d, std=0.02, seed=3, device=dev)
    t = gen.decode_token_inputs(256, H, d, d, "bf16", "uniform", seed=3, step=0, device=dev)
    print("counters: decode step", flush=True)
    kda.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], S)
    torch.cuda.synchronize()
    do = gen.normal((T, H, d), 2, gen.DO, dev, torch.bfloat16)
    print("counters: backward T=%d" % T, flush=True)
    kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do)
    torch.cuda.synchronize()
    del inp, do
    torch.cuda.empty_cache()
    a = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    print("counters: 512 MiB copy", flush=True)
    b.copy_(a)                       # 512 MiB read + 512 MiB written
    torch.cuda.synchronize()
    print("counters done", flush=True)


KDA_KERNELS = ("prefill_wy_prep_kernel", "prefill_wy_carry_kernel", "prefill_mfma_kernel",
               "prefill_valu_kernel", "plan_order_kernel", "decode_step_kernel",
               "decode_multi_kernel", "bwd_init_kernel", "bwd_prep_kernel", "bwd_carry_kernel",
               "bwd_grad_kernel", "front_act_kernel", "front_chain_kernel")
# the --counters workloads in launch order, and the factor from what each
# measures to the figure reported (the long-context runs cover 512 of the
# 16,384 chunks of the 1M-token call)
COUNTER_WORKLOADS = (("long_t1m_prefill", 16384 / 512.0), ("batch4_t4096", 1.0),
                     ("varlen_n64", 1.0), ("decode_n256_step", 1.0),
                     ("long_t1m_backward", 16384 / 512.0))
COPY_BYTES = 512 << 20


def kernel_short(name):
    """'prefill_wy_prep_kernel<0, false>' from a full kernel name, or None
    for a kernel that is not this library's."""
    for k in KDA_KERNELS:
        i = name.find(k)
        if i >= 0:
            j = name.find("(", i)
            return name[i:j if j > 0 else len(name)]
    return None


def source_digest():
    """Digest of every kernel and host source of the library."""
    h = hashlib.sha256()
    src = os.path.join(ROOT, "gated_delta_rule_05_amd", "csrc")
    for n in sorted(os.listdir(src)):
        if n.endswith((".hip", ".h", ".cpp")):
            h.update(n.encode())
            with open(os.path.join(src, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def load_counters():
    """The per-workload figures of the committed rocprofv3 counter summary
    (profiles/traffic.json) if it was taken on the current sources, else
    None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("workloads")


def _dispatches(path, value_col=None):
    """[(dispatch id, full kernel name, value or (start, end))] in dispatch
    order from a rocprofv3 csv."""
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            v = (float(r[value_col]) if value_col else
                 (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
            out.append((did, r["Kernel_Name"], v))
    out.sort(key=lambda x: x[0])
    return out


def _split_workloads(disp):
    """Runs of this library's dispatches, in order; returns a list of lists
    of (short name, value)."""
    runs, cur = [], []
    for _, name, v in disp:
        s = kernel_short(name)
        if s is None:
            if cur:
                runs.append(cur)
                cur = []
        else:
            cur.append((s, v))
    if cur:
        runs.append(cur)
    return runs


def digest_counters(folder):
    import glob

    def one(pattern):
        hits = sorted(glob.glob(os.path.join(folder, pattern), recursive=True))
        if not hits:
            sys.exit("no %s under %s" % (pattern, folder))
        return hits[0]

    trace = _dispatches(one("ks/**/*kernel_trace.csv"))
    pmc = {c: _dispatches(one("pmc_%s/**/*counter_collection.csv" % c), "Counter_Value")
           for c in ("FETCH_SIZE", "WRITE_SIZE", "MfmaUtil")}
    copies = [v for _, n, v in pmc["FETCH_SIZE"] if "copyBuffer" in n]
    wcopies = [v for _, n, v in pmc["WRITE_SIZE"] if "copyBuffer" in n]
    fetch_factor = COPY_BYTES / 1024.0 / copies[-1]
    write_factor = COPY_BYTES / 1024.0 / wcopies[-1]
    runs = {key: _split_workloads(d) for key, d in
            (("time", trace), ("fetch", pmc["FETCH_SIZE"]), ("write", pmc["WRITE_SIZE"]),
             ("mfma", pmc["MfmaUtil"]))}
    for key, r in runs.items():
        if len(r) != len(COUNTER_WORKLOADS):
            sys.exit("%s: %d runs of library kernels, expected %d" %
                     (key, len(r), len(COUNTER_WORKLOADS)))
    workloads = {}
    for i, (wname, scale) in enumerate(COUNTER_WORKLOADS):
        kern = {}
        for key in ("time", "fetch", "write", "mfma"):
            for s, v in runs[key][i]:
                k = kern.setdefault(s, {"dispatches": 0, "us": 0.0, "read_bytes": 0.0,
                                        "written_bytes": 0.0, "mfma_sum": 0.0, "n_mfma": 0})
                if key == "time":
                    k["dispatches"] += 1
                    k["us"] += (v[1] - v[0]) * 1e-3
                elif key == "fetch":
                    k["read_bytes"] += v * 1024.0 * fetch_factor
                elif key == "write":
                    k["written_bytes"] += v * 1024.0 * write_factor
                else:
                    k["mfma_sum"] += v
                    k["n_mfma"] += 1
        total = 0.0
        for s, k in kern.items():
            k["avg_us"] = k["us"] / max(k["dispatches"], 1)
            k["mfma_busy_pct"] = k.pop("mfma_sum") / max(k.pop("n_mfma"), 1)
            total += k["read_bytes"] + k["written_bytes"]
        workloads[wname] = {"measured_bytes": total, "scale_to_reported": scale,
                            "bytes_per_call": total * scale,
                            "us_per_call": sum(k["us"] for k in kern.values()) * scale,
                            "kernels": kern}
    rec = {"source_digest": source_digest(),
           "what": "rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB between L2 and the fabric, scaled by "
                   "a 512 MiB device copy's readings), MfmaUtil and kernel-trace durations of "
                   "`python3 bench.py --counters`, per workload: long_t1m figures cover 512 of "
                   "the call's 16,384 chunks and are scaled to the whole call",
           "calibration": {"kernel": "__amd_rocclr_copyBuffer (512 MiB device copy)",
                           "fetch_kib": copies[-1], "write_kib": wcopies[-1],
                           "fetch_factor": fetch_factor, "write_factor": write_factor},
           "workloads": workloads,
           "commands": COUNTER_COMMANDS}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# rocprofv3 HBM traffic, MFMA use and kernel times, per workload of `bench.py --counters`", "",
             "Commands (one MI355X; `R` = the repository root; each counter in a run of its own):",
             "", "```"] + COUNTER_COMMANDS + ["```", "",
             "Calibration: a 512 MiB device copy reads FETCH_SIZE %.0f KiB (factor %.3f) and "
             "WRITE_SIZE %.0f KiB (factor %.3f); the byte figures below are scaled by those "
             "factors. Source digest `%s`." % (copies[-1], fetch_factor, wcopies[-1],
                                              write_factor, rec["source_digest"]), ""]
    for wname, scale in COUNTER_WORKLOADS:
        w = workloads[wname]
        lines += ["## %s" % wname, "",
                  "| kernel | dispatches | avg µs | read MB | written MB | MfmaUtil % |",
                  "|---|---:|---:|---:|---:|---:|"]
        for s, k in w["kernels"].items():
            lines.append("| `%s` | %d | %.2f | %.1f | %.1f | %.2f |" % (
                s, k["dispatches"], k["avg_us"], k["read_bytes"] / 1e6, k["written_bytes"] / 1e6,
                k["mfma_busy_pct"]))
        lines += ["", "Measured: %.3f GB in %.1f µs of kernel time%s." % (
            w["measured_bytes"] / 1e9, w["us_per_call"] / scale,
            "" if scale == 1.0 else "; scaled ×%g to the whole call: %.2f GB, %.2f ms" % (
                scale, w["bytes_per_call"] / 1e9, w["us_per_call"] / 1e3)), ""]
    with open(os.path.join(ROOT, "profiles", COUNTERS_MD), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/traffic.json and profiles/%s" % COUNTERS_MD)
    stats = sorted(glob.glob(os.path.join(folder, "bench_ks/**/*kernel_stats.csv"), recursive=True))
    if stats:
        digest_bench_stats(stats[0], rec["source_digest"])


def digest_bench_stats(path, digest):
    """Summary of the kernel statistics of a rocprofv3 run of the bench
    itself: every kernel's calls and average, and the per-call figures the
    bench's roofline uses."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            s = kernel_short(r["Name"]) or r["Name"]
            if s.startswith("void ") or "at::native" in s:
                s = "torch: " + s.split("<")[0].split("(")[0].replace("void ", "")[:60]
            rows.append((s, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[3])
    avg = {s: a for s, _, a, _, _ in rows}
    prep, carry = avg.get("prefill_wy_prep_kernel<0, false>"), avg.get("prefill_wy_carry_kernel<16, false>")
    dec = avg.get("decode_step_kernel<unsigned short, 128, 128, 0, false, false>")
    lines = ["# rocprofv3 kernel statistics of bench.py (all legs; long_t1m prefill, decode_n256, ...)",
             "", "Command (one MI355X; `R` = the repository root):", "", "```",
             BENCH_STATS_COMMAND, "python3 $R/bench.py --digest $R/gpurun_out", "```", "",
             "Source digest `%s`. The run makes 1 warm-up and 5 timed calls of every bench leg "
             "(KDA, Gated DeltaNet and DeltaNet prefills, the front-end prefill, the prefill "
             "with snapshots, decode on dense and pooled states, several-token decode, the "
             "backward), plus the other prefill workloads; torch kernels generate inputs." % digest,
             "", "| kernel | calls | average (µs) | total (ms) | share |", "|---|---:|---:|---:|---:|"]
    for s, n, a, t, pct in rows[:24]:
        lines.append("| `%s` | %d | %.1f | %.2f | %.1f%% |" % (s, n, a, t, pct))
    lines.append("")
    if prep and carry:
        call_ms = 256 * (prep + carry) / 1e3
        nbytes = PREFILL_BYTES_PER_HT * 1048576 * 32 + 32 * 128 * 128 * 4
        lines += ["Derived (long_t1m prefill call = 256 blocks of 64 chunks x 32 heads, one "
                  "prep and one carry launch each):",
                  "- prep %.1f µs + carry %.1f µs per block (carry: %.2f µs per chunk step)" % (
                      prep, carry, carry / 64),
                  "- call = %.2f ms from these averages: %.1f GB/s algorithmic, %.3f of 8 TB/s" % (
                      call_ms, nbytes / (call_ms * 1e-3) / 1e9, nbytes / (call_ms * 1e-3) / 8e12)]
    if dec:
        lines.append("- decode step %.1f µs: %.2f TB/s of algorithmic state traffic (%.3f of 8 TB/s)"
                     % (dec, 256 * 32 * DECODE_BYTES_PER_HS / (dec * 1e-6) / 1e12,
                        256 * 32 * DECODE_BYTES_PER_HS / (dec * 1e-6) / 8e12))
    with open(os.path.join(ROOT, "profiles", BENCH_STATS_MD), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/%s" % BENCH_STATS_MD)


COUNTERS_MD = "hbm_traffic_mfma_kernel_times_by_workload.md"
BENCH_STATS_MD = "kernel_stats_bench_long_t1m_decode_n256_all_legs.md"
BENCH_STATS_COMMAND = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d "
                       "$R/gpurun_out/bench_ks -o bench --output-format csv -- python3 $R/bench.py "
                       "--steps 5 --warmup 1 --no-cpu-baseline")


COUNTER_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $R/gpurun_out/ks "
    "-o ks --output-format csv -- python3 $R/bench.py --counters",
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $R/gpurun_out/pmc_FETCH_SIZE "
    "-o pmc --output-format csv -- python3 $R/bench.py --counters",
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $R/gpurun_out/pmc_WRITE_SIZE "
    "-o pmc --output-format csv -- python3 $R/bench.py --counters",
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc MfmaUtil -d $R/gpurun_out/pmc_MfmaUtil "
    "-o pmc --output-format csv -- python3 $R/bench.py --counters",
    "python3 $R/bench.py --digest $R/gpurun_out",
]


def copy_rate_gbps(torch, nbytes=2 << 30, reps=5):
    """GB/s of a device-to-device copy of nbytes (read + write counted; the
    runtime's copy kernel), best of reps, timed with HIP events."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (best * 1e-3) / 1e9


# algorithmic bytes of the prefill gradients per head-token: reads q, k, v,
# dO (bf16) and log_alpha, beta (fp32); writes dq, dk, dv (bf16), dlog_alpha
# and dbeta (fp32)
# the fused input front-end reads bf16 gate and beta pre-activations:
# q, k, v, o (4 x 256) + gate_pre (256) + beta_pre (2)
FRONT_BYTES_PER_HT = 4 * 256 + 256 + 2
BACKWARD_BYTES_PER_HT = 4 * 256 + 512 + 4 + 3 * 256 + 512 + 4
BACKWARD_KERNELS = ("prefill_wy_prep_kernel<0, false> + prefill_wy_carry_kernel<16, true> (forward "
                    "recompute) + bwd_prep_kernel<0> + bwd_carry_kernel + "
                    "bwd_grad_kernel<unsigned short, 0>")


def bench_backward(torch, kda, gen, inp, steps, warmup):
    """Gradients of the 1M-token prefill (zero h0 and dhT adjoint, random
    dO), timed with HIP events on the launch stream."""
    T, H = inp["q"].shape[:2]
    N = inp["cu_seqlens"].shape[0] - 1
    do = gen.normal((T, H, inp["v"].shape[-1]), 9, gen.DO, "cuda", torch.bfloat16)
    need = kda.backward_workspace_bytes(T, N, H, 128, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    grads = {}

    # each call frees the previous call's gradients first, so the caching
    # allocator hands the same memory back (no device allocation is timed)
    def run():
        grads.clear()
        grads.update(kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do,
                                  cu_seqlens=inp["cu_seqlens"], workspace=ws, want_dh0=False))

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a0, a1 in evs:
        a0.record(stream)
        run()
        a1.record(stream)
    torch.cuda.synchronize()
    ms = sum(a0.elapsed_time(a1) for a0, a1 in evs) / len(evs)
    nbytes = BACKWARD_BYTES_PER_HT * T * H
    out = {"workload": "long_t1m", "ms": ms, "tokens_per_s": T / (ms * 1e-3),
           "vs_forward": None, "workspace_bytes": need,
           "algorithmic_bytes_per_head_token": BACKWARD_BYTES_PER_HT,
           "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
           "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "kernels": BACKWARD_KERNELS}
    del ws
    grads.clear()
    torch.cuda.empty_cache()

    # the same gradients through the fused input front-end: q and k taken
    # as raw (normalised in the call), bf16 gate and beta pre-activations;
    # the gradients come out with respect to those
    gp = gen.normal(tuple(inp["log_alpha"].shape), 9, gen.LOG_ALPHA, "cuda", torch.bfloat16)
    bp = gen.normal((T, H), 9, gen.BETA, "cuda", torch.bfloat16)
    need_f = kda.backward_workspace_bytes(T, N, H, 128, 128, l2norm_qk=True, gate_pre=True,
                                          beta_pre=True)
    ws = torch.empty(need_f, dtype=torch.uint8, device="cuda")

    def run_front():
        grads.clear()
        grads.update(kda.backward(inp["q"], inp["k"], inp["v"], None, None, do,
                                  cu_seqlens=inp["cu_seqlens"], workspace=ws, want_dh0=False,
                                  l2norm_qk=True, gate_pre=gp, gate_scale=0.05, beta_pre=bp))

    run_front()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(2)]
    for a0, a1 in evs:
        a0.record(stream)
        run_front()
        a1.record(stream)
    torch.cuda.synchronize()
    ms_f = sum(a0.elapsed_time(a1) for a0, a1 in evs) / len(evs)
    out["front_end"] = {"ms": ms_f, "tokens_per_s": T / (ms_f * 1e-3), "workspace_bytes": need_f,
                        "vs_plain_pct": 100.0 * (ms_f / ms - 1.0),
                        "kernels": "front_act_kernel + the backward above + front_chain_kernel"}
    del ws, gp, bp
    grads.clear()
    torch.cuda.empty_cache()

    # training-style: the forward also writes the per-chunk state record and
    # the backward reads it instead of recomputing the forward pass
    rec_bytes = kda.chunk_states_bytes(T, N, H)
    rec = torch.empty(rec_bytes, dtype=torch.uint8, device="cuda")
    need_s = kda.backward_workspace_bytes(T, N, H, 128, 128, chunk_states=True)
    ws = torch.empty(need_s, dtype=torch.uint8, device="cuda")
    fwd_out = []

    def run_fwd():
        fwd_out.clear()
        fwd_out.extend(kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                   cu_seqlens=inp["cu_seqlens"], final_state=False,
                                   chunk_states=rec))

    def run_saved():
        grads.clear()
        grads.update(kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do,
                                  cu_seqlens=inp["cu_seqlens"], workspace=ws, want_dh0=False,
                                  chunk_states=rec))

    run_fwd()
    run_saved()
    times = {}
    for name, fn in (("forward", run_fwd), ("backward", run_saved)):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(3)]
        for a0, a1 in evs:
            a0.record(stream)
            fn()
            a1.record(stream)
        torch.cuda.synchronize()
        times[name] = sum(a0.elapsed_time(a1) for a0, a1 in evs) / len(evs)
    out["saved_states"] = {"forward_ms": times["forward"], "backward_ms": times["backward"],
                           "forward_plus_backward_ms": times["forward"] + times["backward"],
                           "record_bytes": rec_bytes, "workspace_bytes": need_s,
                           "backward_vs_plain_pct": 100.0 * (times["backward"] / ms - 1.0)}
    del ws, rec, do
    fwd_out.clear()
    grads.clear()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.digest:
        digest_counters(args.digest)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU; the library has no multi-GPU path "
              "(heads and sequences shard across GPUs without communication).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import gated_delta_rule_05_amd as kda
    import kda_inputs as gen

    dev = "cuda"
    kda.load_library()
    stream = torch.cuda.current_stream()
    if args.counters:
        run_counter_workloads(torch, kda, gen, args.chunks)
        return
    if args.only_backward:
        wb = gen.WORKLOADS["long_t1m"]
        inb = gen.workload_prefill_inputs(wb, seed=2, device=dev)
        print(json.dumps(bench_backward(torch, kda, gen, inb, args.steps, args.warmup)), flush=True)
        return

    # ---------------- inputs (resident before timing) ----------------------
    wp = gen.WORKLOADS["long_t1m"]
    inp = gen.workload_prefill_inputs(wp, seed=2, device=dev)
    T, H = sum(inp["lengths"]), wp.H
    o = torch.empty((T, H, wp.dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((1, H, wp.dk, wp.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.prefill_workspace_bytes(T, 1, H, wp.dk, wp.dv), dtype=torch.uint8,
                     device=dev)
    wd = gen.WORKLOADS["decode_n256"]
    S = gen.decode_state(wd.N, wd.H, wd.dk, wd.dv, std=wd.state_std, seed=3, device=dev)
    S0 = S.clone()
    toks = [gen.decode_token_inputs(wd.N, wd.H, wd.dk, wd.dv, wd.dtype, wd.gate, seed=3,
                                    step=s, device=dev) for s in range(wd.steps)]
    o_dec = torch.empty((wd.N, wd.H, wd.dv), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def prefill():
        kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                    cu_seqlens=inp["cu_seqlens"], out=o, final_state=hT, workspace=ws)

    def decode_all():
        for t in toks:
            kda.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], S, out=o_dec)

    for _ in range(args.warmup):
        prefill()
        decode_all()
    S.copy_(S0)
    torch.cuda.synchronize()

    # ---------------- timed steps -------------------------------------------
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        prefill()
        e1.record(stream)
        decode_all()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [a.elapsed_time(b) for a, b, _ in ev]
    dec_ms = [b.elapsed_time(c) for _, b, c in ev]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    ms_per_step = wall * 1e3 / args.steps

    tokens_per_s = T / (pre_avg * 1e-3)
    alg_bytes = PREFILL_BYTES_PER_HT * T * H + hT.numel() * 4
    achieved = alg_bytes / (pre_avg * 1e-3) / 1e9
    flops_c64 = (10 * 64 * 128 + 6 * 128 * 128) * T * H
    dec_step_us = dec_avg * 1e3 / wd.steps
    dec_bytes = DECODE_BYTES_PER_HS * wd.N * wd.H
    dec_gbps = dec_bytes / (dec_step_us * 1e-6) / 1e9

    # ---------------- gate variants on the same workload ------------------
    # Gated DeltaNet (one gate per (token, head)) and DeltaNet (no gate):
    # the prefill without the fp32 per-channel gate, timed the same way
    variants = {}
    head_gate = gen.gates((T, H), 7, dev, wp.gate).contiguous()
    for name, la, gate, bpht in (("gated_deltanet", head_gate, "head", PREFILL_BYTES_PER_HT - 512 + 4),
                                 ("deltanet", None, "none", PREFILL_BYTES_PER_HT - 512)):
        def run_v():
            kda.prefill(inp["q"], inp["k"], inp["v"], la, inp["beta"], cu_seqlens=inp["cu_seqlens"],
                        out=o, final_state=hT, workspace=ws, gate=gate)
        for _ in range(args.warmup):
            run_v()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a0, a1 in evs:
            a0.record(stream)
            run_v()
            a1.record(stream)
        torch.cuda.synchronize()
        v_ms = sum(a0.elapsed_time(a1) for a0, a1 in evs) / len(evs)
        v_bytes = bpht * T * H + hT.numel() * 4
        variants[name] = {"gate": gate, "prefill_ms": v_ms, "tokens_per_s": T / (v_ms * 1e-3),
                          "algorithmic_bytes_per_head_token": bpht,
                          "achieved_GBps": v_bytes / (v_ms * 1e-3) / 1e9,
                          "frac_of_hbm_peak": v_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del head_gate

    # ---------------- fused input front-end on the same workload ----------
    # the raw form of this workload's inputs: q, k normalised in the kernel,
    # bf16 gate pre-activations x ~ N(0,1) with log_alpha = -0.05 softplus(x)
    # (the workload's own gate law), bf16 beta pre-activations
    gate_pre = gen.normal((T, H, wp.dk), 7, gen.LOG_ALPHA, dev, torch.bfloat16)
    beta_pre = gen.normal((T, H), 7, gen.BETA, dev, torch.bfloat16)
    ws_fe = torch.empty(kda.prefill_workspace_bytes(T, 1, H, wp.dk, wp.dv, front=True),
                        dtype=torch.uint8, device=dev)

    def run_fe():
        kda.prefill(inp["q"], inp["k"], inp["v"], None, None, cu_seqlens=inp["cu_seqlens"],
                    out=o, final_state=hT, workspace=ws_fe, l2norm_qk=True, gate_pre=gate_pre,
                    gate_scale=0.05, beta_pre=beta_pre)
    for _ in range(args.warmup):
        run_fe()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a0, a1 in evs:
        a0.record(stream)
        run_fe()
        a1.record(stream)
    torch.cuda.synchronize()
    fe_ms = sum(a0.elapsed_time(a1) for a0, a1 in evs) / len(evs)
    fe_bytes = FRONT_BYTES_PER_HT * T * H + hT.numel() * 4
    front = {"prefill_ms": fe_ms, "tokens_per_s": T / (fe_ms * 1e-3),
             "algorithmic_bytes_per_head_token": FRONT_BYTES_PER_HT,
             "achieved_GBps": fe_bytes / (fe_ms * 1e-3) / 1e9,
             "frac_of_hbm_peak": fe_bytes / (fe_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
             "vs_plain_pct": 100.0 * (fe_ms / pre_avg - 1.0),
             "kernel": "prefill_wy_prep_kernel<0, true> + prefill_wy_carry_kernel<16, false>"}
    del gate_pre, beta_pre, ws_fe

    # ---------------- serving features ----------------------------------
    # prefill that also records the state every 4096 tokens (prefix
    # caching), and the decode steps on states held in a pool of 512 slots
    # (continuous batching: the 256 sequences own scattered slots)
    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a0, a1 in evs:
            a0.record(stream)
            fn()
            a1.record(stream)
        torch.cuda.synchronize()
        return sum(a0.elapsed_time(a1) for a0, a1 in evs) / len(evs)

    snap_tokens = 4096
    snaps = torch.empty((1, T // snap_tokens, H, wp.dk, wp.dv), dtype=torch.float32, device=dev)
    snap_ms = timed(lambda: kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                        cu_seqlens=inp["cu_seqlens"], out=o, final_state=hT,
                                        workspace=ws, snapshot_tokens=snap_tokens,
                                        snapshots=snaps), args.steps)
    snap_bytes = snaps.numel() * 4
    del snaps
    pool_n = 2 * wd.N
    pool = gen.decode_state(pool_n, wd.H, wd.dk, wd.dv, std=wd.state_std, seed=4, device=dev)
    slots = torch.randperm(pool_n, generator=torch.Generator().manual_seed(5))[:wd.N]
    slots = slots.to(torch.int32).to(dev)

    def decode_pool():
        for t in toks:
            kda.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], pool, out=o_dec,
                            state_index=slots)
    pool_us = timed(decode_pool, args.steps) * 1e3 / wd.steps
    # speculative decoding: verify 4 draft tokens per sequence (outputs of
    # all 4, states only read), then commit an accepted prefix of 0..4
    # tokens (states advanced, no outputs); each call reads a state once
    m_spec = 4
    spec = {key: torch.stack([t[key] for t in toks[:m_spec]], dim=1).contiguous()
            for key in ("q", "k", "v", "log_alpha", "beta")}
    o_spec = torch.empty((wd.N, m_spec, wd.H, wd.dv), dtype=torch.bfloat16, device=dev)
    accepted = torch.randint(0, m_spec + 1, (wd.N,), generator=torch.Generator().manual_seed(6))
    accepted = accepted.to(torch.int32).to(dev)
    verify_us = timed(lambda: kda.decode_multi(spec["q"], spec["k"], spec["v"], spec["log_alpha"],
                                               spec["beta"], S, out=o_spec, write_state=False),
                      args.steps) * 1e3
    commit_us = timed(lambda: kda.decode_multi(spec["q"], spec["k"], spec["v"], spec["log_alpha"],
                                               spec["beta"], S, outputs=False, lengths=accepted),
                      args.steps) * 1e3
    state_bytes = wd.N * wd.H * wd.dk * wd.dv * 4
    live = int((accepted > 0).sum().item())
    del spec, o_spec
    serving = {
        "prefill_snapshots": {"snapshot_tokens": snap_tokens, "snapshot_bytes": snap_bytes,
                              "prefill_ms": snap_ms,
                              "overhead_vs_plain_pct": 100.0 * (snap_ms / pre_avg - 1.0)},
        "decode_state_pool": {"pool_states": pool_n, "sequences": wd.N, "us_per_step": pool_us,
                              "state_GBps": dec_bytes / (pool_us * 1e-6) / 1e9,
                              "frac_of_hbm_peak": dec_bytes / (pool_us * 1e-6) / 1e9 / HBM_PEAK_GBPS},
        "speculative_decode": {
            "draft_tokens": m_spec, "sequences": wd.N,
            "verify_us": verify_us,
            "verify_state_read_GBps": state_bytes / (verify_us * 1e-6) / 1e9,
            "commit_us": commit_us, "committing_sequences": live,
            "commit_state_GBps": (state_bytes + live * wd.H * wd.dk * wd.dv * 4) /
                                 (commit_us * 1e-6) / 1e9,
            "single_steps_us": m_spec * dec_step_us},
    }
    del pool
    torch.cuda.empty_cache()

    # ---------------- the other prefill workloads (the library's automatic path)
    others = {}
    for wname in ("tiny_f32", "batch4_t4096", "varlen_n64"):
        wo = gen.WORKLOADS[wname]
        io = gen.workload_prefill_inputs(wo, seed=11, device=dev)
        To, No = io["q"].shape[0], io["cu_seqlens"].shape[0] - 1
        esz = 4 if wo.dtype == "f32" else 2
        oo = torch.empty((To, wo.H, wo.dv), dtype=io["q"].dtype, device=dev)
        ho = torch.empty((No, wo.H, wo.dk, wo.dv), dtype=torch.float32, device=dev)
        wso = torch.empty(max(1, kda.prefill_workspace_bytes(To, No, wo.H, wo.dk, wo.dv,
                                                             kda.DTYPE_F32 if esz == 4 else kda.DTYPE_BF16,
                                                             max_seqlen=max(io["lengths"]))),
                          dtype=torch.uint8, device=dev)

        msl = max(io["lengths"])

        def run_o():
            kda.prefill(io["q"], io["k"], io["v"], io["log_alpha"], io["beta"], h0=io["h0"],
                        cu_seqlens=io["cu_seqlens"], out=oo, final_state=ho, workspace=wso,
                        max_seqlen=msl)
        o_ms = timed(run_o, max(args.steps, 20))
        fe_o = None
        if wname == "varlen_n64":
            # the same batch from raw inputs (the fused input front-end on the
            # path the library picks for it): q, k normalised in the kernel,
            # bf16 gate and beta pre-activations with this workload's gate law
            gpo = gen.normal((To, wo.H, wo.dk), 11, gen.LOG_ALPHA, dev, torch.bfloat16)
            bpo = gen.normal((To, wo.H), 11, gen.BETA, dev, torch.bfloat16)
            wsf = torch.empty(max(1, kda.prefill_workspace_bytes(To, No, wo.H, wo.dk, wo.dv,
                                                                 kda.DTYPE_BF16, front=True,
                                                                 max_seqlen=msl)),
                              dtype=torch.uint8, device=dev)

            def run_of():
                kda.prefill(io["q"], io["k"], io["v"], None, None, h0=io["h0"],
                            cu_seqlens=io["cu_seqlens"], out=oo, final_state=ho, workspace=wsf,
                            max_seqlen=msl, l2norm_qk=True, gate_pre=gpo, gate_scale=0.05,
                            beta_pre=bpo)
            f_ms = timed(run_of, max(args.steps, 20))
            fb = FRONT_BYTES_PER_HT * To * wo.H + ho.numel() * 4 * 2
            fe_o = {"ms": f_ms, "tokens_per_s": To / (f_ms * 1e-3),
                    "algorithmic_bytes_per_head_token": FRONT_BYTES_PER_HT,
                    "achieved_GBps": fb / (f_ms * 1e-3) / 1e9,
                    "frac_of_hbm_peak": fb / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "vs_plain_pct": 100.0 * (f_ms / o_ms - 1.0),
                    "kernel": "prefill_mfma_kernel<128, 0, true>"}
            del gpo, bpo, wsf
        # q, k, v, o in the input dtype, fp32 gates and beta; states in and out
        per_ht = (2 * wo.dk + 2 * wo.dv) * esz + 4 * wo.dk + 4
        nb = per_ht * To * wo.H + ho.numel() * 4 * (2 if io["h0"] is not None else 1)
        # the chunked form's matrix work, 10 C d + 6 d^2 flops per head-token
        # (C = 64 on the matrix paths, 32 on the fp32 vector path)
        cc = 32 if esz == 4 else 64
        flops = (10 * cc * wo.dk + 6 * wo.dk * wo.dv) * To * wo.H
        others[wname] = {"tokens": To, "sequences": No, "heads": wo.H, "dtype": wo.dtype,
                         "ms": o_ms, "tokens_per_s": To / (o_ms * 1e-3),
                         "head_tokens_per_s": To * wo.H / (o_ms * 1e-3),
                         "algorithmic_bytes": nb, "achieved_GBps": nb / (o_ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": nb / (o_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "useful_TFLOPs": flops / (o_ms * 1e-3) / 1e12,
                         "mfma_useful_frac": (flops / (o_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
                                              if esz == 2 else None)}
        if fe_o is not None:
            others[wname]["front_end"] = fe_o
        del io, oo, ho, wso
    torch.cuda.empty_cache()

    # ---------------- prefill gradients on the same workload ----------------
    backward = bench_backward(torch, kda, gen, inp, args.steps, args.warmup)
    backward["vs_forward"] = backward["ms"] / pre_avg

    counters = load_counters() or {}

    def counted(wname, field="bytes_per_call"):
        w = counters.get(wname)
        return None if w is None else w[field]
    traffic = counted("long_t1m_prefill")
    mfma = None
    if "long_t1m_prefill" in counters:
        mfma = {k: v["mfma_busy_pct"] for k, v in counters["long_t1m_prefill"]["kernels"].items()}
    dec_traffic = counted("decode_n256_step")
    for wname in ("batch4_t4096", "varlen_n64"):
        others[wname]["traffic"] = counted(wname)
        if wname in counters:
            others[wname]["kernels_avg_us"] = {k: v["avg_us"] for k, v in
                                               counters[wname]["kernels"].items()}
            others[wname]["mfma_busy_pct"] = {k: v["mfma_busy_pct"] for k, v in
                                              counters[wname]["kernels"].items()}
    others["tiny_f32"]["traffic"] = None
    backward["traffic"] = counted("long_t1m_backward")
    copy_gbps = copy_rate_gbps(torch)

    result = {
        "metric": "KDA prefill tokens/s (H=32,d=128) + decode state GB/s, % of MI355X roofline",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long_t1m: prefill B=1 T=1048576 H=32 d_k=d_v=128 bf16, "
                               "fp32 state; plus decode_n256: 64 steps x 256 seqs x 32 heads",
                   "global_batch": 1, "seq_len": T, "heads": H, "d_k": 128, "d_v": 128,
                   "parallelism": "none (1 GPU)"},
        "prefill_ms": pre_avg,
        "head_tokens_per_s": tokens_per_s * H,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": PREFILL_KERNELS, "unit_of_launch": "one kda_fwd_prefill call",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "d2d_copy_GBps": copy_gbps,
                     "frac_of_d2d_copy": achieved / copy_gbps,
                     "useful_TFLOPs_c64": flops_c64 / (pre_avg * 1e-3) / 1e12,
                     "mfma_useful_frac_c64": flops_c64 / (pre_avg * 1e-3) / 1e12
                     / MFMA_BF16_PEAK_TFLOPS,
                     "mfma_busy_pct": mfma},
        "decode": {"workload": "decode_n256", "us_per_step": dec_step_us,
                   "seq_steps_per_s": wd.N / (dec_step_us * 1e-6),
                   "state_GBps": dec_gbps, "frac_of_hbm_peak": dec_gbps / HBM_PEAK_GBPS,
                   "frac_of_d2d_copy": dec_gbps / copy_gbps,
                   "algorithmic_bytes_per_step": dec_bytes, "traffic_per_step": dec_traffic,
                   "kernel": DECODE_KERNEL},
        "gate_variants": variants,
        "front_end": front,
        "serving": serving,
        "other_prefill_workloads": others,
        "backward": backward,
        "cpu_baseline": None,
    }

    # ---------------- CPU baseline: the oracle on a bounded sample ---------
    if not args.no_cpu_baseline:
        import oracle
        nh, nt = min(args.cpu_heads, H), min(args.cpu_tokens, T)
        heads = list(range(0, H, max(1, H // nh)))[:nh]

        def hostsel(t):
            return t[:nt, heads].to(torch.float32).cpu().numpy()

        sub = {kk: hostsel(inp[kk]) for kk in ("q", "k", "v", "log_alpha")}
        sub_beta = inp["beta"][:nt, heads].cpu().numpy()
        threads = min(len(heads), os.cpu_count() or 1)
        t_c = time.perf_counter()
        o_ref, _ = oracle.prefill(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub_beta,
                                  scale=1.0 / math.sqrt(wp.dk), threads=threads)
        cpu_s = time.perf_counter() - t_c
        got = o[:nt, heads].to(torch.float64).cpu().numpy()
        err = float(np.max(np.abs(got - o_ref)) / max(np.max(np.abs(o_ref)), 1e-30))
        head_tokens_per_s = nt * len(heads) / cpu_s
        result["cpu_baseline"] = {
            "value": head_tokens_per_s / H, "unit": "tokens/s", "cores": threads,
            "host_cores": os.cpu_count(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "%d of %d heads x first %d tokens of the prefill workload (fp64 "
                      "token loop, one thread per head), %.1f s; tokens/s scaled to all "
                      "%d heads" % (len(heads), H, nt, cpu_s, H),
            "parity_max_rel_err_o": err}

    print(json.dumps(result))


if __name__ == "__main__":
    main()
