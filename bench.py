"""Benchmark of the paged GQA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-extras]

A step is one attn_paged_decode call (split planner, paged split-KV kernel
and log-sum-exp combine) over one batch of the workload, with every input
already resident in HBM.  To keep reads cold, R independent input sets are
rotated so that more than 1 GB is touched between two uses of a set (more
than the 256 MB Infinity Cache plus the L2s).

Prints ONE JSON line: value = algorithmic HBM bytes per call / measured time
per call (GB/s); us_per_call beside it.  "roofline" covers the split kernel
(timed alone with HIP events on the launch stream, same split count as the
timed calls); "traffic" comes from the committed rocprofv3 counter summary
when its recorded kernel-source hash matches the current source, else null.
"cpu_baseline" times the CPU oracle on a bounded sample of the same workload.
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
COUNTERS = os.path.join(ROOT, "profiles", "decode_split_b128_counters.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_gqa_03_amd", "csrc", "decode.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="paged_b128",
                    choices=["paged_b128", "paged_b32", "paged_b128_kv4096", "paged_b32_kv4096", "contig_b16",
                             "ragged_prefill", "ragged_prefill_masked", "swa_fp8"])
    ap.add_argument("--num-splits", type=int, default=0, help="0 = planner")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="untimed: 3 split-kernel launches on set 0 and 3 copies of 1 GiB, for rocprofv3 --pmc")
    return ap.parse_args()


def decode_bytes(case):
    """Algorithmic bytes of one paged decode call: every K and V row once,
    the block-table entries used, kv_lens, Q read and O written."""
    lens = case["kv_lens"].tolist()
    ps, Hkv, D, B, Hq = case["page_size"], case["Hkv"], case["D"], case["B"], case["Hq"]
    kv = sum(n * Hkv * D * 2 * 2 for n in lens)
    bt = sum((n + ps - 1) // ps * 4 for n in lens)
    return kv + bt + 4 * B + 2 * B * Hq * D * 2


def make_sets(name, device, n_sets):
    import workloads
    B = 128 if "b128" in name else 32
    fixed = 4096 if "kv4096" in name else None
    base = 1004 if B == 128 else 1003
    return [workloads.serving_paged_decode(B, device=device, fixed_len=fixed, seed=base + 7919 * r)
            for r in range(n_sets)]


def rotation_count(bytes_per_call):
    """Input sets to rotate so >= 1.5 GB is read between two uses of a set."""
    return max(2, math.ceil(1.5e9 / bytes_per_call))


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic():
    """HBM bytes (read + write) of one split-kernel launch of this workload,
    from the committed rocprofv3 counter summary (calibrated FETCH_SIZE +
    WRITE_SIZE), and its read / algorithmic ratio; (None, None) when the
    summary is absent or was taken on another kernel source."""
    if not os.path.exists(COUNTERS):
        return None, None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("decode_src_sha256") != source_hash(DECODE_SRC):
        return None, None
    return c.get("hbm_bytes_per_launch"), c.get("read_over_algorithmic")


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
    probe = make_sets(args.workload, dev, 1)
    per_call = decode_bytes(probe[0])
    R = rotation_count(per_call)
    sets = probe + make_sets(args.workload, dev, R)[1:]
    for s in sets:
        s["out"] = torch.empty_like(s["q"])
        s["bytes"] = decode_bytes(s)
    c0 = sets[0]
    max_len = max(s["max_kv_len"] for s in sets)
    S = args.num_splits or pa.attn_plan_splits(c0["B"], c0["Hkv"], c0["Hq"] // c0["Hkv"], c0["D"], max_len,
                                               c0["page_size"], c0["k_pool"].stride(2))
    ws_bytes = pa.attn_decode_workspace_bytes(c0["B"], c0["Hq"], c0["D"], S)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    if args.counters:
        run_counters(torch, pa, c0, S, max_len, ws)
        return

    def call(s):
        pa.attn_paged_decode(s["q"], s["k_pool"], s["v_pool"], s["block_table"], s["kv_lens"], max_len,
                             s["out"], s["page_size"], s["scale"], num_splits=S, workspace=ws)

    # --- timed region: K whole calls --------------------------------------
    torch.cuda.synchronize()
    ms = time_calls(torch, call, sets, args.steps, args.warmup)
    mean_bytes = sum(sets[i % R]["bytes"] for i in range(args.steps)) / args.steps
    gbs = mean_bytes / (ms * 1e-3) / 1e9

    # --- per-kernel breakdown with HIP events on the launch stream ---------
    # The split kernel alone (attn_paged_decode_split: same launch, every
    # piece written as a partial) and the combine, each bracketed by events.
    stream = torch.cuda.current_stream()
    n_k = max(20, args.steps)
    marks = []
    for i in range(args.warmup + n_k):
        s = sets[i % R]
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        pa.attn_paged_decode_split(s["q"], s["k_pool"], s["v_pool"], s["block_table"], s["kv_lens"],
                                   max_len, s["page_size"], s["scale"], S, ws)
        e1.record(stream)
        pa.attn_decode_combine(ws, s["B"], s["Hq"], s["Hkv"], s["D"], S, s["k_pool"].stride(2), s["kv_lens"],
                               max_len, s["out"])
        e2.record(stream)
        if i >= args.warmup:
            marks.append((e0, e1, e2, s["bytes"]))
    torch.cuda.synchronize()
    ks = [(a.elapsed_time(b), b.elapsed_time(c), nb) for a, b, c, nb in marks]
    # Spread of the per-call times (event pair around each call's two
    # launches): median with p10 / p90.
    per_call = sorted((k[0] + k[1]) * 1e3 for k in ks)

    def pct(q):
        return round(per_call[min(len(per_call) - 1, int(q * (len(per_call) - 1) + 0.5))], 2)

    spread = {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "calls": len(per_call),
              "timing": "HIP events around each call's split and combine launches"}
    k_ms = sum(k[0] for k in ks) / len(ks)
    comb = sum(k[1] for k in ks) / len(ks)
    k_bytes = sum(k[2] for k in ks) / len(ks)
    kernel = "decode_split_kernel<128,4,8,paged> (balanced partition, %d slices)" % S
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    traffic, read_ratio = load_traffic() if args.workload == "paged_b128" else (None, None)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_read_over_algorithmic": read_ratio, "kernel": kernel,
                "kernel_us": round(k_ms * 1e3, 2), "combine_us": round(comb * 1e3, 2),
                "algorithmic_bytes_per_launch": int(k_bytes)}

    # --- CPU oracle on a bounded sample -------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        host = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in c0.items()
                if k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "scale")}
        lens = host["kv_lens"].tolist()

        def sample_bytes(m):
            return sum(n * c0["Hkv"] * c0["D"] * 4 + (n + 15) // 16 * 4 + 4 for n in lens[:m]) \
                + 2 * m * c0["Hq"] * c0["D"] * 2

        def run_oracle(m):
            idx = torch.arange(m)
            t0 = time.perf_counter()
            oracle.paged_decode(host["q"][idx], host["k_pool"], host["v_pool"], host["block_table"][idx],
                                host["kv_lens"][idx], host["scale"])
            return time.perf_counter() - t0

        # Doubling prefixes of the batch until one takes >= 1 s or the whole
        # batch is reached; then whole calls repeat until ~10 s are spent.
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
        cpu = {"value": round(calls * sample_bytes(m) / tot_t / 1e9, 3), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "first %d of %d sequences of set 0, %d call(s), %.1f s" % (m, c0["B"], calls, tot_t),
               "nproc": os.cpu_count(), "cpu_model": cpu_model()}

    # --- other workloads of the path (context lines, not the headline) -----
    extras = {}
    if not args.no_extras:
        extras = run_extras(torch, pa, dev, args)

    kv_desc = "4096" if "kv4096" in args.workload else "U[512,4096]"
    line = {
        "metric": "paged decode us/call + achieved HBM GB/s (% of peak) at B=32..128, kv 4K",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_call": round(ms * 1e3, 2),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4), "per_call_us": spread,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, pages scattered in a 1.5x pool)",
        "config": {"workload": "paged GQA decode B=%d Hq=32 Hkv=8 D=128 page_size=16 kv_lens %s"
                               % (c0["B"], kv_desc),
                   "B": c0["B"], "Hq": 32, "Hkv": 8, "D": 128, "page_size": 16, "kv_lens": kv_desc,
                   "num_splits": S, "rotation_sets": R, "algorithmic_bytes_per_call": int(mean_bytes)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extras,
    }
    print(json.dumps(line), flush=True)


def run_counters(torch, pa, c0, S, max_len, ws):
    """Launches for hardware-counter runs: the split kernel of the timed
    configuration, then a plain device copy of exactly 1 GiB (reads 1 GiB,
    writes 1 GiB) that calibrates FETCH_SIZE / WRITE_SIZE."""
    for _ in range(3):
        pa.attn_paged_decode_split(c0["q"], c0["k_pool"], c0["v_pool"], c0["block_table"], c0["kv_lens"],
                                   max_len, c0["page_size"], c0["scale"], S, ws)
    torch.cuda.synchronize()
    src = torch.empty(1 << 30, dtype=torch.uint8, device=c0["q"].device).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": True, "num_splits": S, "split_kernel_algorithmic_bytes": decode_bytes(c0),
                      "copy_bytes": 1 << 30}), flush=True)


def run_extras(torch, pa, dev, args):
    """Short timings of the other decode workloads (same protocol)."""
    import workloads
    out = {}
    steps, warm = 20, 5
    for name in ("paged_b32", "paged_b128_kv4096", "paged_b32_kv4096"):
        probe = make_sets(name, dev, 1)
        per = decode_bytes(probe[0])
        R = rotation_count(per)
        sets = probe + make_sets(name, dev, R)[1:]
        mx = max(s["max_kv_len"] for s in sets)
        c0 = sets[0]
        S = pa.attn_plan_splits(c0["B"], 8, 4, 128, mx, 16, c0["k_pool"].stride(2))
        ws = torch.empty(max(256, pa.attn_decode_workspace_bytes(c0["B"], 32, 128, S)), dtype=torch.uint8,
                         device=dev)
        for s in sets:
            s["out"] = torch.empty_like(s["q"])

        def call(s):
            pa.attn_paged_decode(s["q"], s["k_pool"], s["v_pool"], s["block_table"], s["kv_lens"], mx,
                                 s["out"], 16, s["scale"], num_splits=S, workspace=ws)
        ms = time_calls(torch, call, sets, steps, warm)
        nb = sum(decode_bytes(sets[i % R]) for i in range(steps)) / steps
        out[name] = {"us_per_call": round(ms * 1e3, 2), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                     "hbm_peak_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "num_splits": S,
                     "rotation_sets": R}
        del sets
        torch.cuda.empty_cache()
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
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for i in range(warm):
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
        for _ in range(3):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (3 * steps)
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
    nb = sum(swa_bytes(sets[i % R]) for i in range(steps)) / steps
    gbs = nb / (ms * 1e-3) / 1e9
    return {"us_per_call": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_call": int(nb), "rotation_sets": R}


def bench_contiguous(torch, pa, dev, steps, warm, num_splits):
    """Contiguous decode, B=16 Hq=32 Hkv=8 D=128 kv=2048 (bhld), same protocol."""
    import workloads
    c = workloads.contiguous_decode(device=dev)
    nb = 16 * 8 * 2048 * 128 * 4 + 2 * 16 * 32 * 128 * 2
    R = rotation_count(nb)
    cs = [c] + [workloads.contig_decode_case(1002 + 7919 * r, 16, 32, 8, 128, 2048, device=dev)
                for r in range(1, R)]
    for s in cs:
        s["out"] = torch.empty_like(s["q"])
    S = num_splits or pa.attn_plan_splits(16, 8, 4, 128, 2048, 0, c["k"].stride(1))
    ws = torch.empty(max(256, pa.attn_decode_workspace_bytes(16, 32, 128, S)), dtype=torch.uint8, device=dev)

    def ccall(s):
        pa.attn_decode(s["q"], s["k"], s["v"], s["out"], s["scale"], num_splits=S, workspace=ws)
    ms = time_calls(torch, ccall, cs, steps, warm)
    return {"us_per_call": round(ms * 1e3, 2), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
            "hbm_peak_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "num_splits": S, "rotation_sets": R}


if __name__ == "__main__":
    main()
