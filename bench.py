"""Benchmark of the paged GQA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-extras] [--counters]

A step is one attn_paged_decode call (split planner, paged split-KV kernel
and log-sum-exp combine) over one batch of the workload, with every input
already resident in HBM.  To keep reads cold, R independent input sets are
rotated so that more than 1.5 GB is touched between two uses of a set (more
than the 256 MB Infinity Cache plus the L2s).

Prints ONE JSON line: value = algorithmic HBM bytes per call / measured time
per call (GB/s); us_per_call beside it.  "roofline" covers the split kernel
(timed alone with HIP events on the launch stream, same split count as the
timed calls), against the 8 TB/s specification and against a measured
pure-read streaming probe of the same byte count (attn_hbm_read_probe);
"traffic" comes from the committed rocprofv3 counter summary of the same
rotated input sets when its recorded kernel-source hash matches the current
source, else null.  "cpu_baseline" times the CPU oracle on a bounded sample
of the same workload.
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

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "paged_kv_gqa_03_amd", "csrc", "decode.hip")

# Paged decode workloads: batch, query heads, KV heads, page size, lengths
# (None = U[512, 4096], else that length for every sequence), seed.  D = 128.
DECODE_WORKLOADS = {
    "paged_b128": dict(B=128, Hq=32, Hkv=8, ps=16, fixed=None, seed=1004),
    "paged_b32": dict(B=32, Hq=32, Hkv=8, ps=16, fixed=None, seed=1003),
    "paged_b128_kv4096": dict(B=128, Hq=32, Hkv=8, ps=16, fixed=4096, seed=1004),
    "paged_b32_kv4096": dict(B=32, Hq=32, Hkv=8, ps=16, fixed=4096, seed=1003),
    "paged_b32_ps1": dict(B=32, Hq=32, Hkv=8, ps=1, fixed=None, seed=1011),
    "paged_b128_g8": dict(B=128, Hq=64, Hkv=8, ps=16, fixed=None, seed=1012),
    "paged_b128_g32": dict(B=128, Hq=32, Hkv=1, ps=16, fixed=None, seed=1013),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="paged_b128",
                    choices=list(DECODE_WORKLOADS) + ["contig_b16", "ragged_prefill", "ragged_prefill_masked",
                                                      "swa_fp8"])
    ap.add_argument("--num-splits", type=int, default=0, help="0 = planner")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="untimed: one decode split-kernel launch per rotated input set (paged workloads; the "
                         "whole call for contig_b16 and swa_fp8) and 3 copies of 1 GiB, for rocprofv3 --pmc")
    return ap.parse_args()


def decode_bytes(case):
    """Algorithmic bytes of one paged decode call: every K and V row once,
    the block-table entries used, kv_lens, Q read and O written."""
    lens = case["kv_lens"].tolist()
    ps, Hkv, D, B, Hq = case["page_size"], case["Hkv"], case["D"], case["B"], case["Hq"]
    kv = sum(n * Hkv * D * 2 * 2 for n in lens)
    bt = sum((n + ps - 1) // ps * 4 for n in lens)
    return kv + bt + 4 * B + 2 * B * Hq * D * 2


def contig_bytes():
    """Contiguous decode B=16 Hq=32 Hkv=8 D=128 kv=2048: K, V, Q and O."""
    return 16 * 8 * 2048 * 128 * 4 + 2 * 16 * 32 * 128 * 2


def make_sets(name, device, n_sets):
    import workloads
    w = DECODE_WORKLOADS[name]
    lens = [w["fixed"]] * w["B"] if w["fixed"] else (512, 4096)
    return [workloads.paged_decode_case(w["seed"] + 7919 * r, w["B"], w["Hq"], w["Hkv"], 128, lens, w["ps"],
                                        device=device)
            for r in range(n_sets)]


def workload_desc(name):
    w = DECODE_WORKLOADS[name]
    kv = str(w["fixed"]) if w["fixed"] else "U[512,4096]"
    return ("paged GQA decode B=%d Hq=%d Hkv=%d D=128 page_size=%d kv_lens %s"
            % (w["B"], w["Hq"], w["Hkv"], w["ps"], kv))


def decode_kernel_label(w, slices):
    """Name of the split kernel a paged D = 128 workload runs (the library's
    row layout rule): group sizes 1, 2, 4 on the VALU kernel, others on MFMA
    rows."""
    G, Hkv = w["Hq"] // w["Hkv"], w["Hkv"]
    if G in (1, 2, 4):
        return "decode_split_kernel<128,%d,%d,paged,4> (balanced partition, %d slices)" % (
            G, 8 if Hkv % 8 == 0 else 1, slices)
    gm = min(G, 32)
    while G % gm:
        gm -= 1
    hg = 1 if G // gm > 1 else 4 if Hkv % 4 == 0 else 2 if Hkv % 2 == 0 else 1
    return "decode_mfma_kernel<128,%d,%d,%d> (balanced partition, %d slices)" % (
        (gm + 15) // 16, 2 if w["ps"] % 4 == 0 else 1, hg, slices)


def rotation_count(bytes_per_call):
    """Input sets to rotate so >= 1.5 GB is read between two uses of a set."""
    return max(2, math.ceil(1.5e9 / bytes_per_call))


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counters_path(workload):
    return os.path.join(PROFILES, "decode_%s_counters.json" % workload)


def load_traffic(workload):
    """HBM bytes (read + write) per split-kernel launch of this workload, mean
    over the rotated input sets, from the committed rocprofv3 counter summary
    (calibrated FETCH_SIZE + WRITE_SIZE), with the algorithmic bytes of the
    same launches and the read / algorithmic ratio; None when the summary is
    absent or was taken on another kernel source."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("decode_src_sha256") != source_hash(DECODE_SRC):
        return None
    return c


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def time_calls(torch, fn, sets, steps, warmup):
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(sets[i % len(sets)])
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def time_graph(torch, fn, sets, steps, warmup, replays=3):
    """ms per call when `steps` calls are captured once in a HIP graph and the
    graph is replayed: the GPU's own time per call, without the host's cost
    of issuing each call from Python (as a serving loop that replays graphs
    would see it)."""
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for i in range(warmup):
            fn(sets[i % len(sets)])
    st.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for i in range(steps):
            fn(sets[i % len(sets)])
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * steps)


def probe_ceiling(torch, pa, dev, nbytes, steps=20):
    """Pure-read streaming ceiling at nbytes per launch: attn_hbm_read_probe
    over rotated buffers of nbytes (cold, as the decode inputs), one, two and
    three workgroups per CU; the fastest is reported."""
    nbytes = (int(nbytes) + 15) // 16 * 16
    R = rotation_count(nbytes)
    bufs = [torch.full((nbytes // 4,), r + 1, dtype=torch.int32, device=dev) for r in range(R)]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = None
    for k in (1, 2, 3):
        wg = k * cus
        sink = torch.empty(wg * 16, dtype=torch.int32, device=dev)
        ms = time_calls(torch, lambda b: pa.attn_hbm_read_probe(b, sink, wg), bufs, steps, 4)
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["GB/s"]:
            best = {"GB/s": round(gbs, 1), "us": round(ms * 1e3, 2), "workgroups": wg, "bytes": nbytes,
                    "rotation_sets": R}
    del bufs
    torch.cuda.empty_cache()
    return best


def bench_decode(torch, pa, dev, name, steps, warmup, num_splits=0, breakdown=True, probe=True):
    """One paged decode workload: whole calls (value), then the split kernel
    and the combine each timed alone with HIP events on the launch stream,
    and the streaming ceiling at the same byte count."""
    probe_set = make_sets(name, dev, 1)
    R = rotation_count(decode_bytes(probe_set[0]))
    sets = probe_set + make_sets(name, dev, R)[1:]
    for s in sets:
        s["out"] = torch.empty_like(s["q"])
        s["bytes"] = decode_bytes(s)
    c0 = sets[0]
    max_len = max(s["max_kv_len"] for s in sets)
    S = num_splits or pa.attn_plan_splits(c0["B"], c0["Hkv"], c0["Hq"] // c0["Hkv"], c0["D"], max_len,
                                          c0["page_size"], c0["k_pool"].stride(2))
    ws = torch.empty(max(pa.attn_decode_workspace_bytes(c0["B"], c0["Hq"], c0["D"], S), 256), dtype=torch.uint8,
                     device=dev)

    def call(s):
        pa.attn_paged_decode(s["q"], s["k_pool"], s["v_pool"], s["block_table"], s["kv_lens"], max_len,
                             s["out"], s["page_size"], s["scale"], num_splits=S, workspace=ws)

    torch.cuda.synchronize()
    ms = time_calls(torch, call, sets, steps, warmup)
    mean_bytes = sum(sets[i % R]["bytes"] for i in range(steps)) / steps
    gbs = mean_bytes / (ms * 1e-3) / 1e9
    res = {"us_per_call": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
           "num_splits": S, "rotation_sets": R, "algorithmic_bytes_per_call": int(mean_bytes)}
    if breakdown:
        # The split kernel alone (attn_paged_decode_split: same launch, every
        # piece written as a partial) and the combine, each bracketed by
        # events on the stream they are launched on.
        stream = torch.cuda.current_stream()
        n_k = max(20, steps)
        marks = []
        for i in range(warmup + n_k):
            s = sets[i % R]
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
            pa.attn_paged_decode_split(s["q"], s["k_pool"], s["v_pool"], s["block_table"], s["kv_lens"],
                                       max_len, s["page_size"], s["scale"], S, ws)
            e1.record(stream)
            pa.attn_decode_combine(ws, s["B"], s["Hq"], s["Hkv"], s["D"], S, s["k_pool"].stride(2), s["kv_lens"],
                                   max_len, s["out"])
            e2.record(stream)
            if i >= warmup:
                marks.append((e0, e1, e2, s["bytes"]))
        torch.cuda.synchronize()
        ks = [(a.elapsed_time(b), b.elapsed_time(c), nb) for a, b, c, nb in marks]
        per_call = sorted((k[0] + k[1]) * 1e3 for k in ks)

        def pct(q):
            return round(per_call[min(len(per_call) - 1, int(q * (len(per_call) - 1) + 0.5))], 2)

        k_ms = sum(k[0] for k in ks) / len(ks)
        res["kernel_us"] = round(k_ms * 1e3, 2)
        res["combine_us"] = round(sum(k[1] for k in ks) / len(ks) * 1e3, 2)
        res["kernel_bytes"] = int(sum(k[2] for k in ks) / len(ks))
        res["kernel_GB/s"] = round(res["kernel_bytes"] / (k_ms * 1e-3) / 1e9, 1)
        res["per_call_us"] = {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "calls": len(per_call),
                              "timing": "HIP events around each call's split and combine launches"}
    del sets
    torch.cuda.empty_cache()
    if probe:
        pr = probe_ceiling(torch, pa, dev, mean_bytes)
        res["probe"] = pr
        res["frac_of_probe"] = round(gbs / pr["GB/s"], 4)
        if breakdown:
            res["kernel_frac_of_probe"] = round(res["kernel_GB/s"] / pr["GB/s"], 4)
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(every configuration fits one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_gqa_03_amd as pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.counters:
        run_counters(torch, pa, dev, args.workload, args.num_splits)
        return
    if args.workload == "contig_b16":
        r = bench_contiguous(torch, pa, dev, args.steps, args.warmup, args.num_splits)
        print(json.dumps({"workload": "contiguous decode B=16 Hq=32 Hkv=8 D=128 kv=2048 bhld", **r}), flush=True)
        return
    if args.workload in ("ragged_prefill", "ragged_prefill_masked"):
        r = bench_prefill(torch, pa, dev, args.steps, args.warmup, masked=args.workload.endswith("masked"))
        print(json.dumps({"workload": "ragged paged prefill 8 seqs ctx U[0,2048] new U[1,512] Hq=32 Hkv=8 D=128"
                                      + (" 3-D mask" if args.workload.endswith("masked") else ""), **r}), flush=True)
        return
    if args.workload == "swa_fp8":
        r = bench_swa(torch, pa, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "fp8 sliding-window decode T=64 NH=128 HD=512 W=128", **r}), flush=True)
        return

    # --- timed region: K whole calls, then the per-kernel breakdown ---------
    r = bench_decode(torch, pa, dev, args.workload, args.steps, args.warmup, args.num_splits)
    w = DECODE_WORKLOADS[args.workload]
    kernel = decode_kernel_label(w, r["num_splits"])
    tr = load_traffic(args.workload)
    roofline = {"bound": "hbm", "achieved": r["kernel_GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(r["kernel_GB/s"] / HBM_PEAK_GBS, 4),
                "traffic": tr["hbm_bytes_per_launch"] if tr else None,
                "traffic_algorithmic_bytes_per_launch": tr["algorithmic_bytes_per_launch"] if tr else None,
                "traffic_read_over_algorithmic": tr["read_over_algorithmic"] if tr else None,
                "kernel": kernel, "kernel_us": r["kernel_us"], "combine_us": r["combine_us"],
                "algorithmic_bytes_per_launch": r["kernel_bytes"],
                "probe_ceiling_GBs": r["probe"]["GB/s"], "frac_of_probe": r["kernel_frac_of_probe"]}

    # --- CPU oracle on a bounded sample -------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, args.workload)

    # --- other workloads of the path (context lines, not the headline) -----
    extras = {}
    if not args.no_extras:
        extras = run_extras(torch, pa, dev, args)

    line = {
        "metric": "paged decode us/call + achieved HBM GB/s (% of peak) at B=32..128, kv 4K",
        "value": r["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["us_per_call"] / 1e3, 5), "us_per_call": r["us_per_call"],
        "hbm_peak_frac": r["hbm_peak_frac"], "frac_of_probe": r["frac_of_probe"], "per_call_us": r["per_call_us"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, pages scattered in a 1.5x pool)",
        "config": {"workload": workload_desc(args.workload), "B": w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"], "D": 128,
                   "page_size": w["ps"], "kv_lens": str(w["fixed"]) if w["fixed"] else "U[512,4096]",
                   "num_splits": r["num_splits"], "rotation_sets": r["rotation_sets"],
                   "algorithmic_bytes_per_call": r["algorithmic_bytes_per_call"]},
        "roofline": roofline,
        "probe": r["probe"],
        "cpu_baseline": cpu,
        "extra": extras,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(torch, workload):
    """The CPU oracle (never tuned) on set 0 of the workload: doubling prefixes
    of the batch until one takes >= 1 s or the whole batch is reached, then
    whole calls repeated until ~10 s are spent."""
    import oracle
    c0 = make_sets(workload, "cpu", 1)[0]
    lens = c0["kv_lens"].tolist()
    ps = c0["page_size"]

    def sample_bytes(m):
        return sum(n * c0["Hkv"] * c0["D"] * 4 + (n + ps - 1) // ps * 4 + 4 for n in lens[:m]) \
            + 2 * m * c0["Hq"] * c0["D"] * 2

    def run_oracle(m):
        idx = torch.arange(m)
        t0 = time.perf_counter()
        oracle.paged_decode(c0["q"][idx], c0["k_pool"], c0["v_pool"], c0["block_table"][idx], c0["kv_lens"][idx],
                            c0["scale"])
        return time.perf_counter() - t0

    t_budget, m, spent = 10.0, 1, 0.0
    while True:
        dt = run_oracle(m)
        spent += dt
        if dt >= 1.0 or m == c0["B"]:
            break
        m = min(c0["B"], m * 2)
    calls, tot_t = 1, dt
    while spent < t_budget:
        dt = run_oracle(m)
        spent += dt
        tot_t += dt
        calls += 1
    return {"value": round(calls * sample_bytes(m) / tot_t / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "first %d of %d sequences of set 0, %d call(s), %.1f s" % (m, c0["B"], calls, tot_t),
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def run_counters(torch, pa, dev, workload, num_splits):
    """Launches for hardware-counter runs: one decode split-kernel launch per
    rotated input set of the workload (the whole attn_decode call for the
    contiguous one), then a plain device copy of exactly 1 GiB, three times
    (reads 1 GiB, writes 1 GiB), which calibrates FETCH_SIZE / WRITE_SIZE.
    Prints the algorithmic bytes of each launch, in launch order."""
    import workloads
    per_launch = []
    if workload == "contig_b16":
        nb = contig_bytes()
        R = rotation_count(nb)
        for r in range(R):
            c = workloads.contig_decode_case(1002 + 7919 * r, 16, 32, 8, 128, 2048, device=dev)
            out = torch.empty_like(c["q"])
            pa.attn_decode(c["q"], c["k"], c["v"], out, c["scale"], num_splits=num_splits)
            torch.cuda.synchronize()
            per_launch.append(nb)
            del c
        kernel = "decode_split_kernel (contiguous, one KV head per row) of attn_decode"
    elif workload == "swa_fp8":
        per = swa_bytes(workloads.swa_fp8(device=dev))
        R = min(32, max(2, math.ceil(6.0e8 / per)))
        for r in range(R):
            c = workloads.swa_fp8(device=dev, seed=1006 + 7919 * r)
            out = torch.empty_like(c["q"])
            pa.attn_swa_fp8_decode(c["q"], c["cache"], c["inv_scale"], c["indices"], c["lens"], out,
                                   c["block_size"], c["scale"])
            torch.cuda.synchronize()
            per_launch.append(swa_bytes(c))
            del c
        kernel = "swa_kernel of attn_swa_fp8_decode"
    else:
        probe_set = make_sets(workload, dev, 1)
        R = rotation_count(decode_bytes(probe_set[0]))
        sets = probe_set + make_sets(workload, dev, R)[1:]
        c0 = sets[0]
        max_len = max(s["max_kv_len"] for s in sets)
        S = num_splits or pa.attn_plan_splits(c0["B"], c0["Hkv"], c0["Hq"] // c0["Hkv"], c0["D"], max_len,
                                              c0["page_size"], c0["k_pool"].stride(2))
        ws = torch.empty(max(pa.attn_decode_workspace_bytes(c0["B"], c0["Hq"], c0["D"], S), 256),
                         dtype=torch.uint8, device=dev)
        for s in sets:
            pa.attn_paged_decode_split(s["q"], s["k_pool"], s["v_pool"], s["block_table"], s["kv_lens"], max_len,
                                       s["page_size"], s["scale"], S, ws)
            torch.cuda.synchronize()
            per_launch.append(decode_bytes(s))
        kernel = "decode split kernel (attn_paged_decode_split), %d slices" % S
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": True, "workload": workload, "kernel": kernel,
                      "algorithmic_bytes_per_launch": per_launch, "copy_bytes": 1 << 30}), flush=True)


def run_extras(torch, pa, dev, args):
    """Short timings of the other workloads (same protocol)."""
    out = {}
    steps, warm = 20, 5
    for name in DECODE_WORKLOADS:
        if name == args.workload:
            continue
        out[name] = bench_decode(torch, pa, dev, name, steps, warm)
    out["contiguous_b16_kv2048"] = bench_contiguous(torch, pa, dev, steps, warm, 0)
    out["ragged_prefill"] = bench_prefill(torch, pa, dev, steps, warm, masked=False)
    out["ragged_prefill_masked"] = bench_prefill(torch, pa, dev, steps, warm, masked=True)
    out["dense_prefill_b4_l2048_causal"] = bench_dense_prefill(torch, pa, dev, steps, warm)
    out["short_q_prefill_g8_b16_q16_kv16384"] = bench_short_q_prefill(torch, pa, dev, steps, warm)
    out["swa_fp8"] = bench_swa(torch, pa, dev, steps, warm)
    out.update(bench_cache_ops(torch, pa, dev, steps, warm))
    return out


def bench_cache_ops(torch, pa, dev, steps, warm):
    """The cache writes and rotary that precede attention, HBM-bound: GB/s of
    algorithmic bytes (every byte read or written once), R rotated sets."""
    import workloads
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(1007)

    def timed(fn, sets, nbytes):
        # These kernels take a few microseconds, less than the host needs to
        # issue a call from Python, so the calls are captured once in a HIP
        # graph and the graph is replayed (as a serving loop would issue them).
        ms = time_graph(torch, fn, sets, steps, warm)
        return {"us_per_call": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "hbm_peak_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_call": int(nbytes),
                "rotation_sets": len(sets), "timing": "HIP graph of %d calls, 3 replays" % steps}

    # KV append: the ragged prefill's new tokens (8 sequences, U[1,512] each)
    # and a decode step (one token for each of 128 sequences).
    for name, B, ctx, q_range in (("kv_append_prefill_chunk", 8, (0, 2048), (1, 512)),
                                  ("kv_append_decode_step", 128, (0, 512), (1, 1))):
        sets = []
        for r in range(4):
            c = workloads.prefill_case(1008 + 7919 * r, B, 32, 8, 128, ctx, q_range, 16, device=dev)
            N = int(c["qo_indptr"][-1])
            c["kn"] = torch.randn(N, 8, 128, generator=g, device=dev).to(torch.bfloat16)
            c["vn"] = torch.randn(N, 8, 128, generator=g, device=dev).to(torch.bfloat16)
            c["start"] = torch.tensor(c["ctx_lens"], dtype=torch.int32, device=dev)
            sets.append(c)
        nb = sum(int(c["qo_indptr"][-1]) * 8 * 128 * 2 * 2 * 2 + (c["B"] + 1) * 8 for c in sets) / len(sets)

        def fn(c):
            pa.attn_paged_kv_append(c["kn"], c["vn"], c["qo_indptr"], c["start"], c["k_pool"], c["v_pool"],
                                    c["block_table"], 16)
        out[name] = timed(fn, sets, nb)
    # fp8 quantize-on-write of 4096 sliding-window rows (HD 512) into a
    # 32768-slot cache, dynamic scales.
    sets = []
    for r in range(4):
        x = torch.randn(4096, 512, generator=g, device=dev).to(torch.bfloat16)
        slots = torch.randperm(32768, generator=g, device=dev)[:4096]
        cache = torch.zeros(128, 256, 512, dtype=torch.uint8, device=dev)
        inv = torch.zeros(32768, 1, dtype=torch.bfloat16, device=dev)
        amax = torch.empty(4096, device=dev)
        sets.append(dict(x=x, slots=slots, cache=cache, inv=inv, amax=amax))
    nb = 4096 * (512 * 2 + 512 + 8 + 2 + 4)

    def fq(c):
        pa.attn_swa_fp8_append(c["x"], c["slots"], c["cache"], c["inv"], 256, amax=c["amax"])
    out["swa_fp8_append_4096_rows"] = timed(fq, sets, nb)
    # Rotary on Q [T, 32, 128] and K [T, 8, 128] of the ragged prefill's
    # tokens (T = 2052), positions up to 4096, in place.
    ang = torch.arange(4096, device=dev, dtype=torch.float64)[:, None] * \
        (10000.0 ** (-2.0 * torch.arange(64, device=dev, dtype=torch.float64) / 128))[None, :]
    cos, sin = ang.cos().float(), ang.sin().float()
    sets = []
    for r in range(4):
        sets.append(dict(q=torch.randn(2052, 32, 128, generator=g, device=dev).to(torch.bfloat16),
                         k=torch.randn(2052, 8, 128, generator=g, device=dev).to(torch.bfloat16),
                         pos=torch.randint(0, 4096, (2052,), generator=g, device=dev, dtype=torch.int32)))
    nb = 2052 * (32 + 8) * 128 * 2 * 2 + 2 * 2052 * 64 * 4 * 2 + 2 * 2052 * 4

    def fr(c):
        pa.attn_rotary_embed(c["q"], cos, sin, c["pos"])
        pa.attn_rotary_embed(c["k"], cos, sin, c["pos"])
    out["rotary_q_and_k_2052_tokens"] = timed(fr, sets, nb)
    return out


def prefill_flops(case):
    """4 * D * Hq per visible (query row, key) pair: keys j <= c_b + i of the
    n_b keys (the random mask is not subtracted: it removes no tile work)."""
    total = 0
    for c, qn, n in zip(case["ctx_lens"], case["q_lens"], case["kv_lens"].tolist()):
        for i in range(qn):
            total += min(n, c + i + 1)
    return 4 * case["D"] * case["Hq"] * total


def bench_prefill(torch, pa, dev, steps, warm, masked):
    """Ragged paged prefill: 8 sequences, context U[0,2048], new rows U[1,512],
    Hq=32 Hkv=8 D=128 ps=16, causal; optionally the 10%-dropped 3-D mask."""
    import workloads
    sets = [workloads.ragged_prefill(device=dev, masked=masked, seed=1005 + 7919 * r) for r in range(4)]
    R = pa.attn_prefill_tile_rows(128, 4)
    for s in sets:
        _, t2b, t2i = pa.attn_prefill_plan(s["q_lens"], R)
        s["t2b"], s["t2i"] = t2b.to(dev), t2i.to(dev)
        s["out"] = torch.empty_like(s["q"])
        s["flops"] = prefill_flops(s)

    def call(s):
        pa.attn_paged_prefill(s["q"], s["qo_indptr"], s["t2b"], s["t2i"], s["k_pool"], s["v_pool"],
                              s["block_table"], s["kv_lens"], s["out"], 16, s["scale"],
                              causal_offset=s["causal_offset"], mask=s["mask"], tile_rows=R)
    ms = time_calls(torch, call, sets, steps, warm)
    fl = sum(sets[i % len(sets)]["flops"] for i in range(steps)) / steps
    tf = fl / (ms * 1e-3) / 1e12
    return {"us_per_call": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1), "gflop_per_call": round(fl / 1e9, 2),
            "mfma_util": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "rotation_sets": len(sets)}


def bench_short_q_prefill(torch, pa, dev, steps, warm):
    """Short query runs over long contexts (the head-packing benchmark shape):
    16 sequences x 16 new rows after 16368 cached keys, Hq=32 Hkv=4 (G=8),
    D=128, ps=16, causal.  HBM-bound: algorithmic bytes are the K/V of every
    sequence once, Q and O, and the block table.  Timed with the planner's
    split count and unsplit (num_splits 1), two input sets rotated."""
    import workloads
    sets = [workloads.short_q_prefill(device=dev, seed=1007 + 7919 * r) for r in range(2)]
    R = pa.attn_prefill_tile_rows(128, 8)
    for s in sets:
        _, t2b, t2i = pa.attn_prefill_plan(s["q_lens"], R)
        s["t2b"], s["t2i"] = t2b.to(dev), t2i.to(dev)
        s["out"] = torch.empty_like(s["q"])
    c0 = sets[0]
    mx = max(c0["kv_lens"].tolist())
    total_q = c0["q"].shape[0]
    S = pa.attn_prefill_plan_splits(c0["t2b"].numel(), 32, 4, 128, mx)
    ws = torch.empty(max(256, pa.attn_prefill_workspace_bytes(total_q, 32, 128, S)), dtype=torch.uint8, device=dev)
    nbytes = (sum(c0["kv_lens"].tolist()) * 4 * 128 * 4 + 2 * total_q * 32 * 128 * 2
              + sum((n + 15) // 16 for n in c0["kv_lens"].tolist()) * 4)
    res = {}
    for label, n_split in (("split", S), ("unsplit", 1)):
        def call(s, n_split=n_split):
            pa.attn_paged_prefill_split(s["q"], s["qo_indptr"], s["t2b"], s["t2i"], s["k_pool"], s["v_pool"],
                                        s["block_table"], s["kv_lens"], s["out"], 16, s["scale"], mx,
                                        causal_offset=s["causal_offset"], num_splits=n_split, workspace=ws,
                                        tile_rows=R)
        ms = time_calls(torch, call, sets, steps, warm)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[label] = {"us_per_call": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                      "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4), "num_splits": n_split}
    res["rotation_sets"] = len(sets)
    res["mb_per_call"] = round(nbytes / 1e6, 1)
    return res


def bench_dense_prefill(torch, pa, dev, steps, warm):
    """Dense prefill, contiguous KV: B=4, Lq = Lk = 2048, Hq=32, Hkv=8, D=128,
    causal (each row sees its prefix), blhd layout."""
    g = torch.Generator(device=dev)
    g.manual_seed(1009)
    B, L = 4, 2048
    sets = []
    for r in range(2):
        sets.append(dict(q=torch.randn(B, L, 32, 128, generator=g, device=dev).to(torch.bfloat16),
                         k=torch.randn(B, L, 8, 128, generator=g, device=dev).to(torch.bfloat16),
                         v=torch.randn(B, L, 8, 128, generator=g, device=dev).to(torch.bfloat16),
                         out=torch.empty(B, L, 32, 128, dtype=torch.bfloat16, device=dev)))

    def call(s):
        pa.attn_prefill(s["q"], s["k"], s["v"], s["out"], 1.0 / math.sqrt(128), is_causal=True)
    ms = time_calls(torch, call, sets, steps, warm)
    fl = 4 * 128 * 32 * B * (L * (L + 1) // 2)
    tf = fl / (ms * 1e-3) / 1e12
    return {"us_per_call": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1), "gflop_per_call": round(fl / 1e9, 2),
            "mfma_util": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "rotation_sets": len(sets)}


def swa_bytes(case):
    T, NH, HD, W = case["T"], case["NH"], case["HD"], case["W"]
    lens = [min(int(x), W) for x in case["lens"].tolist()]
    return 2 * T * NH * HD * 2 + sum(n * (HD + 2 + 8) for n in lens) + 8 * T


def bench_swa(torch, pa, dev, steps, warm):
    """fp8 sliding-window decode: T=64, NH=128, HD=512, window 128."""
    import workloads
    per = swa_bytes(workloads.swa_fp8(device=dev))
    R = min(32, max(2, math.ceil(6.0e8 / per)))
    sets = [workloads.swa_fp8(device=dev, seed=1006 + 7919 * r) for r in range(R)]
    for s in sets:
        s["out"] = torch.empty_like(s["q"])

    def call(s):
        pa.attn_swa_fp8_decode(s["q"], s["cache"], s["inv_scale"], s["indices"], s["lens"], s["out"],
                               s["block_size"], s["scale"])
    ms = time_calls(torch, call, sets, steps, warm)
    msg = time_graph(torch, call, sets, steps, warm)
    nb = sum(swa_bytes(sets[i % R]) for i in range(steps)) / steps
    gbs = nb / (ms * 1e-3) / 1e9
    return {"us_per_call": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_call_graph": round(msg * 1e3, 2), "hbm_peak_frac_graph": round(nb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "us_per_call: calls issued back to back from Python (the host's issue time per call is "
                      "close to the kernel's); us_per_call_graph: the same calls replayed from a HIP graph",
            "bytes_per_call": int(nb), "rotation_sets": R}


def bench_contiguous(torch, pa, dev, steps, warm, num_splits):
    """Contiguous decode, B=16 Hq=32 Hkv=8 D=128 kv=2048 (bhld), same protocol."""
    import workloads
    c = workloads.contiguous_decode(device=dev)
    nb = contig_bytes()
    R = rotation_count(nb)
    cs = [c] + [workloads.contig_decode_case(1002 + 7919 * r, 16, 32, 8, 128, 2048, device=dev)
                for r in range(1, R)]
    for s in cs:
        s["out"] = torch.empty_like(s["q"])
    S = num_splits or pa.attn_plan_splits(16, 8, 4, 128, 2048, 0, c["k"].stride(1))
    ws = torch.empty(max(256, pa.attn_decode_workspace_bytes(16, 32, 128, S)), dtype=torch.uint8, device=dev)

    # num_splits 0 lets the library plan: with one length for every row it
    # takes one slice per row here (128 rows), which needs no combine.
    def ccall(s):
        pa.attn_decode(s["q"], s["k"], s["v"], s["out"], s["scale"], num_splits=num_splits, workspace=ws)
    ms = time_calls(torch, ccall, cs, steps, warm)
    del cs
    torch.cuda.empty_cache()
    gbs = nb / (ms * 1e-3) / 1e9
    pr = probe_ceiling(torch, pa, dev, nb)
    return {"us_per_call": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
            "num_splits": num_splits or "library planner (one slice per row: 128)", "rotation_sets": R, "probe": pr,
            "frac_of_probe": round(gbs / pr["GB/s"], 4)}


if __name__ == "__main__":
    main()
