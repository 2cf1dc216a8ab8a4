"""Benchmark of the GQA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-breakdown]

A step is one call of the hot path over one batch of synthetic inputs (seeded, from
workloads.py). The headline workload is the Llama-2-7B-shaped GQA-8 decode (B1 H32 G8
D128, 2048 cached tokens, bf16); the others (70B-shaped ragged decode, causal prefill
B4 T2048, 32k-token fp8 MQA decode) are reported in "breakdown", and so are the headline
and fp8 decodes with the current token's KV-cache append done by the same call ("+append"),
three decodes over a cache in shuffled 16-row pages ("_paged16"), two decodes over INT4
caches, and a prefill of the last
512 positions of 4096-token sequences against the cache of the first 3584.

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronisations. Each step reads the next of several replicas of its inputs, together
at least 1 GiB, so the 256 MB Infinity Cache cannot hold the working set and the
figures are HBM figures. The K timed steps are captured once into a HIP graph and
replayed, so the host's launch cost does not idle the GPU; HIP events on the launch
stream around the replay give the per-step (= per-launch) duration used for the
roofline. The eager, host-launched per-call time is reported beside it.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
COLD_BYTES = 1 << 30            # replicas rotate through at least this much memory

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "grouped_query_attention_decode_amd", "csrc")

HEADLINE = "llama7b_gqa8_decode_L2048"
METRIC = "GQA decode KV-read GB/s (% HBM peak) + tok/s; prefill TFLOP/s (% MFMA peak)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Sources of the kernels that each kind of call runs (host layer and shared headers included).
_COMMON_SOURCES = ("gqa_api.hip", "gqa_internal.h", "dtypes.h", "mfma_util.h")
_FAMILY_SOURCES = {
    "decode": _COMMON_SOURCES + ("decode_mfma.hip", "splitkv.h", "splitkv_combine.hip", "kv_append.hip"),
    "prefill": _COMMON_SOURCES + ("prefill_mfma.hip",),
}


# Workloads measured in the breakdown beside those of workloads.WORKLOADS (also selectable
# with --workload, e.g. to profile them on their own).
EXTRA_WORKLOADS = {
    "mqa_int4_decode_B8_L32768": W.mqa_int4_long_decode,
    "llama70b_gqa8_decode_B16_ragged_int4": W.llama70b_ragged_decode_int4,
    "gqa8_chunked_prefill_B4_Tq512_L4096": W.chunked_prefill_512_of_4096,
    "gqa8_chunked_prefill_B4_Tq512_L4096_fp8": W.chunked_prefill_512_of_4096_fp8,
}

def kernel_sources_sha256(family: str) -> str:
    """Hash of the sources of one kernel family; counters taken on other sources do not apply."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(_FAMILY_SOURCES[family]):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from recorded FETCH_SIZE/WRITE_SIZE counters, scaled by the same
    counters on a plain copy of known size; None when absent or taken on other sources of the
    workload's kernel family."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if w is None:
        return None
    family = "prefill" if "prefill" in workload else "decode"
    if w.get("sources_sha256") != kernel_sources_sha256(family):
        return None
    return w.get("traffic_bytes_per_launch")


# ------------------------------------------------------------------------------------
# Algorithmic work per call (what the method must move / compute, nothing more).
# ------------------------------------------------------------------------------------

def decode_bytes(c: W.DecodeCase, append: bool = False) -> dict:
    """KV bytes = valid rows only: 2 (K and V) x sum_b L_b x G x D x element size. With a
    cache append, the new K/V rows are read (q's dtype) and written (cache dtype) once more."""
    esz = {W.F32: 4, W.BF16: 2, W.FP8: 1, W.INT4: 0.5}
    lens = c.seq_lens.clamp(0, c.T_cap).to(torch.int64)
    kv = int(2 * int(lens.sum()) * c.G * c.D * esz[c.kv_dtype])
    qo = 2 * c.B * c.H * c.D * esz[c.q_dtype]
    extra = 4 * c.B + (8 * c.B * c.G if c.kv_dtype in (W.FP8, W.INT4) else 0)   # seq_lens (+ scales)
    if append:
        n_rows = int(((c.seq_lens >= 1) & (c.seq_lens <= c.T_cap)).sum()) * c.G
        extra += int(2 * n_rows * c.D * (esz[c.q_dtype] + esz[c.kv_dtype]))
    if isinstance(c, W.PagedDecodeCase):  # block-table entries of the pages holding valid rows
        extra += 4 * int(((lens + c.page_size - 1) // c.page_size).sum())
    return {"kv": kv, "total": kv + qo + extra}


def decode_flops(c: W.DecodeCase) -> int:
    lens = c.seq_lens.clamp(0, c.T_cap).to(torch.int64)
    return 4 * c.H * c.D * int(lens.sum())


def prefill_flops(c: W.PrefillCase) -> int:
    """Causal: position i attends to i + 1 keys (diagonal included); 4*D flops per pair."""
    pairs = c.T * (c.T + 1) // 2 if c.causal else c.T * c.T
    return 4 * c.B * c.H * c.D * pairs


def prefill_bytes(c: W.PrefillCase) -> int:
    esz = 4 if c.dtype == W.F32 else 2
    return esz * (2 * c.q.numel() + c.k.numel() + c.v.numel())


# ------------------------------------------------------------------------------------

def make_decode_runner(gqa, c: W.DecodeCase, dev, append=False):
    paged = isinstance(c, W.PagedDecodeCase)
    kk, vv = (c.k_pages, c.v_pages) if paged else (c.k_cache, c.v_cache)
    kv_alloc = 2 * kk.numel() * kk.element_size()
    nrep = max(1, math.ceil(COLD_BYTES / kv_alloc))
    reps = []
    base = [c.q.to(dev), kk.to(dev), vv.to(dev)]
    for i in range(nrep):
        reps.append(base if i == 0 else [t.clone() for t in base])
    lens = c.seq_lens.to(dev)
    ks = c.k_scale.to(dev) if c.k_scale is not None else None
    vs = c.v_scale.to(dev) if c.v_scale is not None else None
    out = torch.empty_like(base[0])
    ws_bytes = gqa.decode_workspace_size(c.B, c.H, c.G, c.D, c.T_cap, c.kv_dtype)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    state = {"i": 0}
    new = {}
    if append:  # the current token's key and value, stored at row L-1 by the call itself
        g = torch.Generator().manual_seed(1)
        dt = c.q.dtype
        new = {"k_new": torch.randn(c.B, c.G, c.D, generator=g).to(dt).to(dev),
               "v_new": torch.randn(c.B, c.G, c.D, generator=g).to(dt).to(dev)}

    table = c.block_table.to(dev) if paged else None

    def step():
        q, k, v = reps[state["i"] % nrep]
        state["i"] += 1
        if paged:
            gqa.decode_paged(q, k, v, table, lens, out=out, scale=c.scale, k_scale=ks, v_scale=vs, workspace=ws,
                             **new)
        else:
            gqa.decode(q, k, v, lens, out=out, scale=c.scale, k_scale=ks, v_scale=vs, workspace=ws, **new)

    return step, nrep, out


def chunk_flops(c: W.ChunkCase) -> int:
    """Causal: query i of a sequence of L keys sees L - Tq + i + 1 keys; 4*D flops per pair."""
    lens = c.seq_lens.clamp(0, c.T_cap).to(torch.int64)
    pairs = 0
    for L in lens.tolist():
        if c.causal:
            pairs += sum(max(0, min(L, L - c.Tq + i + 1)) for i in range(c.Tq))
        else:
            pairs += L * c.Tq
    return 4 * c.H * c.D * pairs


def bench_chunk(gqa, c, steps, warmup, dev):
    """A ChunkCase (contiguous cache) or a PagedChunkCase (its cache in pages)."""
    paged = isinstance(c, W.PagedChunkCase)
    kc, vc = (c.k_pages, c.v_pages) if paged else (c.k_cache, c.v_cache)
    kv_alloc = 2 * kc.numel() * kc.element_size()
    nrep = max(1, math.ceil(COLD_BYTES / kv_alloc))
    base = [c.q.to(dev), kc.to(dev), vc.to(dev)]
    reps = [base] + [[t.clone() for t in base] for _ in range(nrep - 1)]
    lens = c.seq_lens.to(dev)
    table = c.block_table.to(dev) if paged else None
    ks = c.k_scale.to(dev) if c.k_scale is not None else None
    vs = c.v_scale.to(dev) if c.v_scale is not None else None
    out = torch.empty_like(base[0])
    state = {"i": 0}

    def step():
        q, k, v = reps[state["i"] % nrep]
        state["i"] += 1
        if paged:
            gqa.prefill_paged(q, k, v, table, lens, out=out, scale=c.scale, causal=c.causal, k_scale=ks, v_scale=vs)
        else:
            gqa.prefill_cached(q, k, v, lens, out=out, scale=c.scale, causal=c.causal, k_scale=ks, v_scale=vs)

    t = time_steps(step, steps, warmup)
    fl = chunk_flops(c)
    s = t["ms_per_step"] * 1e-3
    achieved = fl / (t["launch_ms_mean"] * 1e-3) / 1e12
    kv_esz = 1 if c.kv_dtype == W.FP8 else 2
    lsum = int(c.seq_lens.clamp(0, c.T_cap).sum())
    return {
        "workload": c.name, "B": c.B, "H": c.H, "G": c.G, "D": c.D, "Tq": c.Tq, "T_cap": c.T_cap,
        "seq_lens": c.seq_lens.tolist(), "causal": c.causal, "kv_dtype": c.kv_dtype, "flops": fl,
        "algorithmic_bytes": 2 * (2 * c.q.numel()) + kv_esz * 2 * lsum * c.G * c.D, "tflops": fl / s / 1e12,
        "ms_per_step": t["ms_per_step"], "launch_us_mean": t["launch_ms_mean"] * 1e3,
        "eager_us_per_call": t["eager_ms_per_call"] * 1e3, "timing": t["timing"], "replicas": nrep,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": measured_traffic(c.name)},
    }


def make_prefill_runner(gqa, c: W.PrefillCase, dev):
    per = prefill_bytes(c)
    nrep = max(1, math.ceil(COLD_BYTES / per))
    base = [c.q.to(dev), c.k.to(dev), c.v.to(dev)]
    reps = [base if i == 0 else [t.clone() for t in base] for i in range(nrep)]
    out = torch.empty_like(base[0])
    state = {"i": 0}

    def step():
        q, k, v = reps[state["i"] % nrep]
        state["i"] += 1
        gqa.prefill(q, k, v, out=out, scale=c.scale, causal=c.causal)

    return step, nrep, out


def time_steps(step, steps, warmup, graph=True):
    """Time exactly `steps` calls of `step` after `warmup` untimed calls.

    With graph=True the timed calls are captured once into a HIP graph (each call still
    reads its own input replica) and the graph is replayed between two device
    synchronisations, so host-side launch cost does not leave the GPU idle; HIP events on
    the launch stream bracket the replay. Returns per-step figures in milliseconds, plus the
    eager (host-launched) per-call time for reference.
    """
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Eager per-call time (host launch cost included), for reference.
    n_eager = min(steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_eager):
        step()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n_eager
    res = {"eager_ms_per_call": eager_ms}
    if graph:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for _ in range(steps):
                    step()
        torch.cuda.synchronize()
        g.replay()  # untimed replay: graph upload, first-touch effects
        torch.cuda.synchronize()
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            t_begin.record(stream)
            g.replay()
            t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_begin.elapsed_time(t_end)
        res.update({"ms_per_step": total_ms / steps, "launch_ms_mean": total_ms / steps, "timing": "hip_graph"})
        del g
    else:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_begin.record()
        for i in range(steps):
            starts[i].record()
            step()
            ends[i].record()
        t_end.record()
        torch.cuda.synchronize()
        total_ms = t_begin.elapsed_time(t_end)
        per = sorted(st.elapsed_time(en) for st, en in zip(starts, ends))
        res.update({"ms_per_step": total_ms / steps, "launch_ms_mean": sum(per) / len(per), "timing": "eager"})
    return res


def bench_decode(gqa, c, steps, warmup, dev, append=False):
    step, nrep, _ = make_decode_runner(gqa, c, dev, append)
    t = time_steps(step, steps, warmup)
    by = decode_bytes(c, append)
    s = t["ms_per_step"] * 1e-3
    launch = t["launch_ms_mean"] * 1e-3
    achieved = by["total"] / launch / 1e9
    return {
        "workload": c.name, "B": c.B, "H": c.H, "G": c.G, "D": c.D, "T_cap": c.T_cap,
        "sum_seq_lens": int(c.seq_lens.sum()), "kv_dtype": c.kv_dtype, "cache_append": append,
        "page_size": c.page_size if isinstance(c, W.PagedDecodeCase) else None,
        "splits": gqa.decode_num_splits(c.B, c.H, c.G, c.D, c.T_cap, c.kv_dtype),
        "kv_bytes": by["kv"], "algorithmic_bytes": by["total"], "flops": decode_flops(c),
        "kv_read_GBps": by["kv"] / s / 1e9, "tok_per_s": c.B / s,
        "ms_per_step": t["ms_per_step"], "launch_us_mean": t["launch_ms_mean"] * 1e3,
        "eager_us_per_call": t["eager_ms_per_call"] * 1e3, "timing": t["timing"], "replicas": nrep,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if append or isinstance(c, W.PagedDecodeCase) else measured_traffic(c.name)},
    }


def bench_prefill(gqa, c, steps, warmup, dev):
    step, nrep, _ = make_prefill_runner(gqa, c, dev)
    t = time_steps(step, steps, warmup)
    fl = prefill_flops(c)
    s = t["ms_per_step"] * 1e-3
    launch = t["launch_ms_mean"] * 1e-3
    achieved = fl / launch / 1e12
    return {
        "workload": c.name, "B": c.B, "H": c.H, "G": c.G, "D": c.D, "T": c.T, "causal": c.causal,
        "flops": fl, "algorithmic_bytes": prefill_bytes(c), "tflops": fl / s / 1e12,
        "ms_per_step": t["ms_per_step"], "launch_us_mean": t["launch_ms_mean"] * 1e3,
        "eager_us_per_call": t["eager_ms_per_call"] * 1e3, "timing": t["timing"], "replicas": nrep,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": measured_traffic(c.name)},
    }


def hbm_achievable(dev, nbytes=1 << 30, reps=5):
    """What a plain streaming kernel reaches on this device (context beside the published
    peak): a device copy that reads and writes nbytes, median of reps."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    res = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        res[f"{name}_GBps"] = moved / sorted(times)[len(times) // 2] / 1e9
    del src, dst
    torch.cuda.empty_cache()
    res["bytes"] = nbytes
    res["note"] = "torch device copy of 1 GiB fp32; GB/s counts bytes read plus bytes written"
    return res


def cpu_baseline_decode(c: W.DecodeCase, budget_s=10.0):
    """The fp64 oracle on the host cores, on the same decode step (whole step, repeated)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_num_threads(threads)
    k, v = oracle.decode_kv_f64(c)
    q = oracle.to_f64(c.q)
    lens = c.seq_lens.numpy()
    times = []
    t_stop = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.decode_arrays(q, k, v, lens, c.scale)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_stop or len(times) >= 2000:
            break
    times.sort()
    med = times[len(times) // 2]
    by = decode_bytes(c)
    return {"value": by["kv"] / med / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"whole {c.name} decode step (fp64 C oracle, OpenMP), median of {len(times)} runs; "
                      f"{med * 1e3:.2f} ms per step, {c.B / med:.1f} tok/s",
            "seconds_per_step": med}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=[k for k in W.WORKLOADS if k != "toy"] + list(EXTRA_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter reference)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures a single GPU; the multi-GPU path is not implemented "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "copies": 5}))
        return

    import grouped_query_attention_decode_amd as gqa
    gqa.library()

    def run_case(case, steps, warmup):
        log(f"[bench] {case.name}: steps={steps} warmup={warmup}")
        r = bench_chunk(gqa, case, steps, warmup, dev)
        log(f"[bench] {case.name}: {json.dumps(r)}")
        return case, r

    def run(name, steps, warmup, append=False):
        case = (W.WORKLOADS.get(name) or EXTRA_WORKLOADS[name])(0)
        tag = name + ("+append" if append else "")
        log(f"[bench] {tag}: steps={steps} warmup={warmup}")
        if isinstance(case, W.PrefillCase):
            r = bench_prefill(gqa, case, steps, warmup, dev)
        elif isinstance(case, W.ChunkCase):
            r = bench_chunk(gqa, case, steps, warmup, dev)
        else:
            r = bench_decode(gqa, case, steps, warmup, dev, append)
        log(f"[bench] {tag}: {json.dumps(r)}")
        return case, r

    case, head = run(args.workload, args.steps, args.warmup)
    breakdown = {}
    if not args.no_breakdown:
        for name in W.WORKLOADS:
            if name in ("toy", args.workload):
                continue
            _, r = run(name, max(20, args.steps // 4), max(5, args.warmup // 2))
            breakdown[name] = r
        # The decode step with the current token's cache append done by the same call.
        for name in dict.fromkeys((args.workload, "mqa_fp8_decode_B8_L32768")):
            if isinstance((W.WORKLOADS.get(name) or EXTRA_WORKLOADS[name])(0), W.DecodeCase):
                _, r = run(name, max(20, args.steps // 4), max(5, args.warmup // 2), append=True)
                breakdown[name + "+append"] = r
        # INT4 caches (4-bit fields, one scale per sequence and KV head), and prefill of a
        # 512-token chunk against a 3584-token cache.
        for name in EXTRA_WORKLOADS:
            if name != args.workload:
                _, breakdown[name] = run(name, max(20, args.steps // 4), max(5, args.warmup // 2))
        # The chunked prefill against the same cache in shuffled pages of 16 rows.
        pcc = W.make_paged_chunk(W.chunked_prefill_512_of_4096(0), 16, seed=1)
        _, breakdown[pcc.name] = run_case(pcc, max(20, args.steps // 4), max(5, args.warmup // 2))
        # The same decodes over a cache in shuffled pages of 16 rows.
        for name in ("llama7b_gqa8_decode_L2048", "llama70b_gqa8_decode_B16_ragged", "mqa_fp8_decode_B8_L32768"):
            pc = W.make_paged(W.WORKLOADS[name](0), 16, seed=1)
            log(f"[bench] {pc.name}")
            r = bench_decode(gqa, pc, max(20, args.steps // 4), max(5, args.warmup // 2), dev)
            log(f"[bench] {pc.name}: {json.dumps(r)}")
            breakdown[pc.name] = r

    is_prefill = isinstance(case, (W.PrefillCase, W.ChunkCase))
    achievable = None if args.no_breakdown else hbm_achievable(dev)
    cpu = None
    if not args.no_cpu_baseline and not is_prefill:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline_decode(case)
        log(f"[bench] cpu baseline: {json.dumps(cpu)}")

    if is_prefill:
        value, unit, dtype = head["tflops"], "TFLOP/s", "bf16"
    else:
        value, unit = head["kv_read_GBps"], "GB/s"
        dtype = {W.BF16: "bf16", W.FP8: "fp8_e4m3fn", W.F32: "f32", W.INT4: "int4"}[case.kv_dtype]
    cfg = {"workload": case.name, "global_batch": case.B, "heads": case.H, "kv_heads": case.G,
           "head_dim": case.D, "parallelism": "none (1 GPU)"}
    if isinstance(case, W.ChunkCase):
        cfg["seq_len"], cfg["chunk_len"] = case.T_cap, case.Tq
    elif is_prefill:
        cfg["seq_len"] = case.T
    else:
        cfg["kv_cache_len"] = case.T_cap
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded N(0,1))",
        "config": cfg,
        "tok_per_s": head.get("tok_per_s"),
        "hbm_frac": (value / HBM_PEAK_GBS) if not is_prefill else None,
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "hbm_achievable": achievable,
        "detail": head,
        "breakdown": breakdown,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
