"""Benchmark of the GQA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path FAMILY]
                    [--no-cpu-baseline] [--no-breakdown]
    python bench.py --timeline --workload NAME --steps K     (needs the timeline build)
    python bench.py --summarize-trace KERNEL_TRACE.csv --steps K
    python bench.py --summarize-counters FETCH.csv WRITE.csv --steps K --workload NAME
    python bench.py --summarize-calibration FETCH.csv WRITE.csv
    python bench.py --copy-calibration

A step is one call of the hot path over one batch of synthetic inputs (seeded, from
workloads.py). The headline is the largest decode: the Llama-2-70B-shaped GQA-8 decode of a
ragged batch (B16 H64 G8 D128, lengths drawn from [1024, 4096], bf16); the causal prefill
(B4 H32 G8 D128 T2048, bf16) is the required second entry ("prefill"). The rest go in
"breakdown": the Llama-2-7B-shaped decode, the 32k-token fp8 MQA decode, decodes with the
current token's cache append done by the same call ("+append"), decodes over a cache in
shuffled 16-row pages ("_paged16"), decodes over INT4 caches, and prefills of the last 512
positions of 4096-token sequences against the cache of the first 3584.

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronisations. Each step reads the next of several replicas of its inputs, together at
least 1 GiB, and a plain streaming read of another 1 GiB (gqa_hbm_stream_read) runs before
the timed steps, so the 256 MB Infinity Cache holds none of their data whatever K is: the
figures are HBM figures. The K timed steps are captured once into a HIP graph and replayed,
so the host's launch cost does not idle the GPU; HIP events on the launch stream around the
replay give the per-step (= per-launch) duration used for the roofline. The eager,
host-launched per-call time is reported beside it.

The fp64 oracle is timed on the host cores beside the GPU (the headline decode, the causal
prefill and the fp8 MQA decode), with the core count and CPU model.

Prints one JSON line. The --summarize-* modes turn rocprofv3 output of such a run into the
summaries kept under profiles/ (the timed dispatches only: the last K of each kernel);
--timeline prints the per-workgroup timeline of K cold decode calls (the diagnostic build of the
library, include/gqa_measure.h).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import re
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

HEADLINE = "llama70b_gqa8_decode_B16_ragged"
PREFILL = "gqa8_causal_prefill_B4_T2048"
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

# Breakdown entries derived from the named workloads: the cache append done by the decode call
# itself ("+append"), and the caches scattered into shuffled pages of 16 rows ("_paged16").
# Selectable with --workload too, so that their counters can be recorded like the others'.
APPEND_DECODES = ("llama70b_gqa8_decode_B16_ragged", "llama7b_gqa8_decode_L2048", "mqa_fp8_decode_B8_L32768")
PAGED_DECODES = ("llama7b_gqa8_decode_L2048", "llama70b_gqa8_decode_B16_ragged", "mqa_fp8_decode_B8_L32768")
PAGED_CHUNK = "gqa8_chunked_prefill_B4_Tq512_L4096"
DERIVED_WORKLOADS = ([n + "+append" for n in APPEND_DECODES] + [n + "_paged16" for n in PAGED_DECODES]
                     + [PAGED_CHUNK + "_paged16"])


def derived_case(name):
    """(case, append) of a derived workload name."""
    if name.endswith("+append"):
        return W.WORKLOADS[name[:-len("+append")]](0), True
    base = name[:-len("_paged16")]
    if base == PAGED_CHUNK:
        return W.make_paged_chunk(W.chunked_prefill_512_of_4096(0), 16, seed=1), False
    return W.make_paged(W.WORKLOADS[base](0), 16, seed=1), False


# Narrow-group decodes (R = 2, 4, 8 query heads per KV head) for the comparison of the
# vector-ALU and matrix-core kernel families (--workload with --path); not in the breakdown.
NARROW_WORKLOADS = {
    "gqa_decode_B1_H16_G8_L2048": lambda seed: W.narrow_group_decode(16, seed),
    "gqa_decode_B1_H32_G8_L2048": lambda seed: W.narrow_group_decode(32, seed),
    "gqa_decode_B1_H64_G8_L2048": lambda seed: W.narrow_group_decode(64, seed),
}


def _code_only(text: str) -> str:
    """C/C++ source text without its comments, every run of white space made one space: what
    the kernels are built from, whatever the wording or layout of the comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_sources_sha256(family: str) -> str:
    """Hash of the code (comments left out) of one kernel family's sources; counters taken on
    other code do not apply."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(_FAMILY_SOURCES[family]):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
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

def make_decode_runner(gqa, c: W.DecodeCase, dev, append=False, path="auto"):
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
                             path=path, **new)
        else:
            gqa.decode(q, k, v, lens, out=out, scale=c.scale, k_scale=ks, v_scale=vs, workspace=ws, path=path, **new)

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


def bench_chunk(gqa, c, steps, warmup, dev, flush):
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

    t = time_steps(step, steps, warmup, flush)
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


class Flusher:
    """Evicts the Infinity Cache (and the L2s) before a timed region: a plain streaming read of
    a 1 GiB buffer (gqa_hbm_stream_read), four times the 256 MB cache, on the current stream."""

    def __init__(self, gqa, dev, nbytes=1 << 30):
        self.gqa = gqa
        self.buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
        self.sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def __call__(self):
        self.gqa.hbm_stream_read(self.buf, self.sink)
        torch.cuda.synchronize()


def time_steps(step, steps, warmup, flush, graph=True):
    """Time exactly `steps` calls of `step` after `warmup` untimed calls, cold: `flush` empties
    the caches right before each timed region, and every call reads its own input replica.

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
    flush()
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
        flush()
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
        flush()
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


def bench_decode(gqa, c, steps, warmup, dev, flush, append=False, path="auto"):
    step, nrep, _ = make_decode_runner(gqa, c, dev, append, path)
    t = time_steps(step, steps, warmup, flush)
    by = decode_bytes(c, append)
    s = t["ms_per_step"] * 1e-3
    launch = t["launch_ms_mean"] * 1e-3
    achieved = by["total"] / launch / 1e9
    return {
        "workload": c.name, "B": c.B, "H": c.H, "G": c.G, "D": c.D, "T_cap": c.T_cap,
        "sum_seq_lens": int(c.seq_lens.sum()), "kv_dtype": c.kv_dtype, "cache_append": append, "path": path,
        "page_size": c.page_size if isinstance(c, W.PagedDecodeCase) else None,
        "splits": gqa.decode_num_splits(c.B, c.H, c.G, c.D, c.T_cap, c.kv_dtype),
        "kv_bytes": by["kv"], "algorithmic_bytes": by["total"], "flops": decode_flops(c),
        "kv_read_GBps": by["kv"] / s / 1e9, "tok_per_s": c.B / s,
        "ms_per_step": t["ms_per_step"], "launch_us_mean": t["launch_ms_mean"] * 1e3,
        "eager_us_per_call": t["eager_ms_per_call"] * 1e3, "timing": t["timing"], "replicas": nrep,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(c.name + ("+append" if append else ""))},
    }


def bench_prefill(gqa, c, steps, warmup, dev, flush):
    step, nrep, _ = make_prefill_runner(gqa, c, dev)
    t = time_steps(step, steps, warmup, flush)
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


def hbm_achievable(gqa, flusher, reps=11):
    """What plain streaming reaches on this device, beside the published peak: the in-tree
    streaming-read kernel (gqa_hbm_stream_read) over a 1 GiB buffer, four times the Infinity
    Cache, so every launch reads from HBM; median of `reps` launches timed with HIP events on
    the launch stream. A 1 GiB torch device copy is reported beside it (read + write)."""
    buf, sink = flusher.buf, flusher.sink
    nbytes = buf.numel() * buf.element_size()
    gqa.hbm_stream_read(buf, sink)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gqa.hbm_stream_read(buf, sink)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    read_gbs = nbytes / sorted(times)[len(times) // 2] / 1e9
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=buf.device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ctimes = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ctimes.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return {"read_GBps": read_gbs, "read_frac_of_peak": read_gbs / HBM_PEAK_GBS,
            "copy_GBps": 2 * nbytes / sorted(ctimes)[len(ctimes) // 2] / 1e9, "bytes": nbytes,
            "note": "read: gqa_hbm_stream_read (in-tree plain streaming-read kernel), median of "
                    f"{reps} launches over 1 GiB; copy: torch device copy of 1 GiB, bytes read plus written"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_time(fn, budget_s, max_runs, min_runs=1):
    times = []
    t_stop = time.perf_counter() + budget_s
    while len(times) < min_runs or (time.perf_counter() < t_stop and len(times) < max_runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    times.sort()
    return times[len(times) // 2], len(times)


def cpu_baseline_decode(c: W.DecodeCase, budget_s=10.0):
    """The fp64 oracle as it stands, on the host cores, on the whole decode step (repeated for
    about budget_s seconds, median)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_num_threads(threads)
    k, v = oracle.decode_kv_f64(c)
    q = oracle.to_f64(c.q)
    lens = c.seq_lens.numpy()
    med, n = _median_time(lambda: oracle.decode_arrays(q, k, v, lens, c.scale), budget_s, 2000)
    by = decode_bytes(c)
    return {"value": by["kv"] / med / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole {c.name} decode step (fp64 C oracle, OpenMP over (b, h) rows), median of {n} "
                      f"runs; {med * 1e3:.2f} ms per step, {c.B / med:.1f} tok/s",
            "seconds_per_step": med, "gflops": decode_flops(c) / med / 1e9, "cpu_model": cpu_model()}


def cpu_baseline_prefill(c: W.PrefillCase, runs=3):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample of the prefill: the
    first sequence of the batch (all H heads, all T rows), median of `runs` runs; the per-step
    time is that times B (the sequences are independent and equal in work)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_num_threads(threads)
    q, k, v = oracle.to_f64(c.q[:1]), oracle.to_f64(c.k[:1]), oracle.to_f64(c.v[:1])
    med, n = _median_time(lambda: oracle.prefill_arrays(q, k, v, c.scale, c.causal), 0.0, runs, min_runs=runs)
    fl = prefill_flops(c) / c.B
    step_s = med * c.B
    return {"value": fl / med / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"sequence 0 of {c.name} (1 of {c.B}: {c.H} heads x {c.T} causal rows, "
                      f"{fl / 1e9:.1f} GFLOP), fp64 C oracle with OpenMP over rows, median of {n} runs of "
                      f"{med:.2f} s; whole step {step_s:.2f} s",
            "seconds_per_step": step_s, "gflops": fl / med / 1e9, "cpu_model": cpu_model()}


def _with_ratio(cpu, gpu_value):
    if cpu is not None:
        cpu["gpu_over_oracle"] = gpu_value / cpu["value"] if cpu["value"] > 0 else None
    return cpu


# ------------------------------------------------------------------------------------
# Summaries of rocprofv3 output (the files kept under profiles/).
# ------------------------------------------------------------------------------------

def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _kernel_name(row):
    return row.get("Kernel_Name") or row.get("KernelName") or row.get("Name") or "?"


def summarize_trace(path, steps):
    """Per kernel: the last `steps` dispatches of a rocprofv3 --kernel-trace CSV, which in a
    bench.py run are those of the timed graph replay (warm-up, eager and untimed-replay calls
    come before it; the cache-flush kernel is listed apart)."""
    rows = _read_csv(path)
    by = {}
    for r in rows:
        start, end = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        did = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
        by.setdefault(_kernel_name(r), []).append((start, did, (end - start) * 1e-3))
    out = {}
    for name, recs in by.items():
        recs.sort()
        d = [x[2] for x in recs]
        last = sorted(d[-steps:])
        out[name] = {"dispatches": len(d), "timed": len(last), "median_us": last[len(last) // 2],
                     "mean_us": sum(last) / len(last), "min_us": last[0], "max_us": last[-1]}
    return out


def _counter_per_dispatch(path, counter):
    rows = _read_csv(path)
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (_kernel_name(r), int(r.get("Dispatch_Id") or r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by = {}
    for (name, did), v in sorted(per.items(), key=lambda kv: kv[0][1]):
        by.setdefault(name, []).append(v)
    return by


def summarize_pmc(path, steps):
    """Median of every counter per kernel over its last `steps` dispatches of a rocprofv3
    --pmc CSV: {kernel: {counter: value}}."""
    rows = _read_csv(path)
    per = {}
    for r in rows:
        key = (_kernel_name(r), r["Counter_Name"], int(r.get("Dispatch_Id") or r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by = {}
    for (name, ctr, did), v in sorted(per.items(), key=lambda kv: kv[0][2]):
        by.setdefault(name, {}).setdefault(ctr, []).append(v)
    out = {}
    for name, ctrs in by.items():
        out[name] = {}
        for ctr, vals in ctrs.items():
            last = sorted(vals[-steps:])
            out[name][ctr] = last[len(last) // 2]
    return out


def summarize_counters(fetch_csv, write_csv, steps):
    """Median FETCH_SIZE / WRITE_SIZE (KiB) per kernel over its last `steps` dispatches."""
    f, w = _counter_per_dispatch(fetch_csv, "FETCH_SIZE"), _counter_per_dispatch(write_csv, "WRITE_SIZE")
    out = {}
    for name in f:
        fl, wl = sorted(f[name][-steps:]), sorted(w.get(name, [0.0])[-steps:])
        out[name] = {"fetch_kib_median": fl[len(fl) // 2], "write_kib_median": wl[len(wl) // 2]}
    return out


# ------------------------------------------------------------------------------------
# Per-workgroup timeline of a decode (the diagnostic timeline build of the library).
# ------------------------------------------------------------------------------------

def timeline_summary(stamps, label):
    """Text summary of one decode call's per-workgroup timeline: per phase, the 0/10/50/90/100th
    percentiles over the workgroups, in microseconds from the first workgroup's entry (slots as
    described in include/gqa_measure.h; the clock runs at 100 MHz)."""
    import numpy as np
    a = stamps.astype(np.int64)
    used = np.nonzero(a[:, 0])[0]
    if len(used) == 0:
        return [f"== {label}: no stamps"]
    a = a[:int(used.max()) + 1]
    nwg = a.shape[0]
    t0 = a[:, 0].min()
    us = lambda col: (a[:, col] - t0) * 0.01
    pc = lambda x: " ".join(f"{v:6.2f}" for v in np.percentile(x, [0, 10, 50, 90, 100])) if len(x) else "-"
    n = a[:, 21]
    ok = n > 0
    last = 2 + 6 * np.clip(n - 1, 0, 2)
    idx = np.arange(nwg)
    at = lambda off: (a[idx, last + off] - t0) * 0.01
    arrived = a[idx, last + 4] != 0
    exit_ = us(20)
    out = [f"== {label}: {nwg} workgroups, span {exit_.max():.2f} us (first entry to last exit)",
           f"  {'phase (us from the first entry)':44s}    p0    p10    p50    p90   p100",
           f"  {'entry':44s} {pc(us(0))}",
           f"  {'length(s) / layout known':44s} {pc(us(1))}",
           f"  {'first piece: first block done':44s} {pc(us(3)[a[:, 3] != 0])}",
           f"  {'last piece: block loop done':44s} {pc(at(2)[ok])}",
           f"  {'exit':44s} {pc(exit_[ok])}",
           f"  {'last piece, durations:':44s}",
           f"  {'  block loop done -> exit':44s} {pc((exit_ - at(2))[ok])}",
           f"  {'  merge of the waves, partials issued':44s} {pc((at(3) - at(2))[ok])}",
           f"  {'    the other waves done (barrier)':44s} {pc((us(22) - at(2))[ok])}",
           f"  {'    partial sums written to LDS':44s} {pc((us(23) - us(22))[ok])}",
           f"  {'    summed, partials issued':44s} {pc((at(3) - us(23))[ok])}",
           f"  {'  arrival counted (split ranges)':44s} {pc((at(4) - at(3))[ok & arrived])}",
           f"  {'  then to the end (last arriver: its merge)':44s} "
           f"{pc((at(5) - np.where(arrived, at(4), at(3)))[ok])}"]
    for k in (1, 2, 3):
        m = n == k
        if m.any():
            out.append(f"  workgroups with {k} piece(s): {int(m.sum()):4d}, exit median {np.median(exit_[m]):6.2f} "
                       f"max {exit_[m].max():6.2f}")
    # Placement (slot 31): CU = (XCC, shader engine, shader array, CU) from HW_ID and XCC_ID.
    hw = a[:, 31] & 0xFFFFFFFF
    xcc = (a[:, 31] >> 32) & 0xF
    cu = xcc * 1024 + ((hw >> 13) & 7) * 64 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
    per_cu = np.unique(cu[ok | (a[:, 0] != 0)], return_counts=True)[1]
    hist = {int(k): int(v) for k, v in zip(*np.unique(per_cu, return_counts=True))}
    out.append(f"  placement: {len(per_cu)} CUs used, CUs by workgroups held {hist}; XCD = blockIdx mod 8 for "
               f"{int(((idx % 8) == xcc)[a[:, 0] != 0].sum())} of {int((a[:, 0] != 0).sum())} workgroups")
    out.append("  by blockIdx mod 8 (the XCD the dispatcher sends it to): exit median / max, last loop done median")
    for x in range(8):
        m = ((idx % 8) == x) & ok
        if m.any():
            out.append(f"    {x}: {np.median(exit_[m]):6.2f} / {exit_[m].max():6.2f}   {np.median(at(2)[m]):6.2f}")
    return out


def run_timeline(args):
    """--timeline: cold decode calls of --workload on the timeline build, one summary each."""
    from grouped_query_attention_decode_amd import build as B
    import grouped_query_attention_decode_amd as gqa
    if "GQA_LIBRARY_PATH" not in os.environ:
        gqa.LIBRARY_PATH = B.TIMELINE_LIBRARY
    if not os.path.exists(gqa.LIBRARY_PATH):
        sys.exit(f"{gqa.LIBRARY_PATH} is not built: python -m grouped_query_attention_decode_amd.build --timeline")
    dev = "cuda:0"
    torch.cuda.set_device(0)
    gqa.library()
    case = (W.WORKLOADS.get(args.workload) or EXTRA_WORKLOADS.get(args.workload) or
            NARROW_WORKLOADS.get(args.workload) or (lambda s: None))(0)
    if not isinstance(case, W.DecodeCase):
        sys.exit("--timeline takes a contiguous decode workload")
    flush = Flusher(gqa, dev)
    q, k, v, lens = case.q.to(dev), case.k_cache.to(dev), case.v_cache.to(dev), case.seq_lens.to(dev)
    ks = case.k_scale.to(dev) if case.k_scale is not None else None
    vs = case.v_scale.to(dev) if case.v_scale is not None else None
    need = gqa.decode_workspace_size(case.B, case.H, case.G, case.D, case.T_cap, case.kv_dtype)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    call = lambda: gqa.decode(q, k, v, lens, out=out, scale=case.scale, k_scale=ks, v_scale=vs, workspace=ws)
    for _ in range(max(args.warmup, 3)):
        call()
    torch.cuda.synchronize()
    for r in range(args.steps):
        gqa.timeline_clear()
        flush()
        call()
        torch.cuda.synchronize()
        print("\n".join(timeline_summary(gqa.timeline_read(), f"{case.name}, cold call {r}")), flush=True)


def _summaries(args):
    """The --summarize-* modes: read rocprofv3 CSV output, print (and for counters record) the
    figures kept under profiles/. No GPU needed."""
    if args.summarize_pmc:
        res = summarize_pmc(args.summarize_pmc, args.steps)
        ctrs = sorted({c for r in res.values() for c in r})
        print(f"{'kernel':58s} " + " ".join(f"{c:>16s}" for c in ctrs))
        for name, r in res.items():
            print(f"{name[:58]:58s} " + " ".join(f"{r.get(c, float('nan')):16.4g}" for c in ctrs))
        return
    if args.summarize_trace:
        res = summarize_trace(args.summarize_trace, args.steps)
        print(f"{'kernel':58s} {'disp':>5s} {'timed':>5s} {'median_us':>10s} {'mean_us':>9s} {'min_us':>8s} {'max_us':>8s}")
        for name, r in sorted(res.items(), key=lambda kv: -kv[1]["median_us"] * kv[1]["timed"]):
            print(f"{name[:58]:58s} {r['dispatches']:5d} {r['timed']:5d} {r['median_us']:10.2f} {r['mean_us']:9.2f} "
                  f"{r['min_us']:8.2f} {r['max_us']:8.2f}")
        return
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {"copy_calibration": None, "workloads": {}}
    if args.summarize_calibration:
        fetch_csv, write_csv = args.summarize_calibration
        res = summarize_counters(fetch_csv, write_csv, 5)
        name = max(res, key=lambda n: res[n]["fetch_kib_median"])
        copy_bytes = 1 << 30
        rec["copy_calibration"] = {
            "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py "
                       "--copy-calibration",
            "kernel": name, "copy_bytes": copy_bytes,
            "fetch_scale": copy_bytes / (res[name]["fetch_kib_median"] * 1024),
            "write_scale": copy_bytes / (res[name]["write_kib_median"] * 1024)}
        print(json.dumps(rec["copy_calibration"]))
    else:
        fetch_csv, write_csv = args.summarize_counters
        cal = rec.get("copy_calibration")
        if not cal:
            sys.exit("record the copy calibration first (--summarize-calibration)")
        res = summarize_counters(fetch_csv, write_csv, args.steps)
        # The library's kernels of one call; not the cache flush, not torch's set-up kernels.
        res = {n: r for n, r in res.items() if "gqa::" in n and "stream_read" not in n}
        total = sum(r["fetch_kib_median"] * 1024 * cal["fetch_scale"] + r["write_kib_median"] * 1024 * cal["write_scale"]
                    for r in res.values())
        family = "prefill" if "prefill" in args.workload else "decode"
        rec.setdefault("workloads", {})[args.workload] = {
            "kernels": res, "traffic_bytes_per_launch": total, "sources_sha256": kernel_sources_sha256(family),
            "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py "
                       f"--workload {args.workload} --steps {args.steps} --warmup 2 --no-cpu-baseline --no-breakdown"}
        print(json.dumps(rec["workloads"][args.workload]))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=[k for k in W.WORKLOADS if k != "toy"] + list(EXTRA_WORKLOADS) + list(NARROW_WORKLOADS)
                    + DERIVED_WORKLOADS)
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma", "generic"],
                    help="decode kernel family for --workload (the breakdown always runs auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter reference)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="per-kernel durations of the last --steps dispatches of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-pmc", metavar="COUNTER_CSV",
                    help="per-kernel medians of every counter of a rocprofv3 --pmc run (last --steps dispatches)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record HBM traffic per launch of --workload in profiles/traffic.json")
    ap.add_argument("--summarize-calibration", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record the counter scale of a --copy-calibration run in profiles/traffic.json")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup timeline of --steps cold calls of a decode --workload (needs the "
                         "timeline build: python -m grouped_query_attention_decode_amd.build --timeline)")
    args = ap.parse_args()
    if args.summarize_trace or args.summarize_counters or args.summarize_calibration or args.summarize_pmc:
        return _summaries(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sharding is a design note "
              "only), so only --gpus 1 runs", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.timeline:
        return run_timeline(args)

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
    flush = Flusher(gqa, dev)
    small_steps, small_warmup = max(20, args.steps // 4), max(5, args.warmup // 2)

    def run_case(case, steps, warmup):
        log(f"[bench] {case.name}: steps={steps} warmup={warmup}")
        if isinstance(case, W.PrefillCase):
            r = bench_prefill(gqa, case, steps, warmup, dev, flush)
        elif isinstance(case, (W.ChunkCase, W.PagedChunkCase)):
            r = bench_chunk(gqa, case, steps, warmup, dev, flush)
        else:
            r = bench_decode(gqa, case, steps, warmup, dev, flush)
        log(f"[bench] {case.name}: {json.dumps(r)}")
        return r

    def run(name, steps, warmup, append=False, path="auto"):
        if name in DERIVED_WORKLOADS:
            case, append = derived_case(name)
            if not append:
                return case, run_case(case, steps, warmup)
            name = case.name
        case = (W.WORKLOADS.get(name) or EXTRA_WORKLOADS.get(name) or NARROW_WORKLOADS[name])(0)
        if path != "auto" and isinstance(case, W.DecodeCase):
            log(f"[bench] {name} path={path}: steps={steps} warmup={warmup}")
            r = bench_decode(gqa, case, steps, warmup, dev, flush, path=path)
            log(f"[bench] {name} path={path}: {json.dumps(r)}")
            return case, r
        if not append:
            return case, run_case(case, steps, warmup)
        log(f"[bench] {name}+append: steps={steps} warmup={warmup}")
        r = bench_decode(gqa, case, steps, warmup, dev, flush, append=True)
        log(f"[bench] {name}+append: {json.dumps(r)}")
        return case, r

    case, head = run(args.workload, args.steps, args.warmup, path=args.path)
    is_prefill = isinstance(case, (W.PrefillCase, W.ChunkCase, W.PagedChunkCase))
    # The causal prefill is the required second entry beside a decode headline.
    prefill_case, prefill = (None, None)
    if args.workload != PREFILL and not args.no_breakdown:
        prefill_case, prefill = run(PREFILL, args.steps, args.warmup)
    breakdown = {}
    if not args.no_breakdown:
        for name in W.WORKLOADS:
            if name in ("toy", args.workload, PREFILL):
                continue
            _, breakdown[name] = run(name, small_steps, small_warmup)
        # The decode step with the current token's cache append done by the same call.
        for name in APPEND_DECODES:
            if name + "+append" != args.workload:
                _, breakdown[name + "+append"] = run(name, small_steps, small_warmup, append=True)
        # INT4 caches (4-bit fields, one scale per sequence and KV head), and prefill of a
        # 512-token chunk against a 3584-token cache.
        for name in EXTRA_WORKLOADS:
            if name != args.workload:
                _, breakdown[name] = run(name, small_steps, small_warmup)
        # The chunked prefill, and the decodes, against the same caches in shuffled pages of 16 rows.
        for name in [PAGED_CHUNK + "_paged16"] + [n + "_paged16" for n in PAGED_DECODES]:
            if name != args.workload:
                _, breakdown[name] = run(name, small_steps, small_warmup)

    achievable = hbm_achievable(gqa, flush)
    del flush
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baselines (oracle) ...")
        if is_prefill:
            cpu = _with_ratio(cpu_baseline_prefill(case), head["tflops"]) if isinstance(case, W.PrefillCase) else None
        else:
            cpu = _with_ratio(cpu_baseline_decode(case), head["kv_read_GBps"])
        if prefill is not None:
            prefill["cpu_baseline"] = _with_ratio(cpu_baseline_prefill(prefill_case), prefill["tflops"])
        mqa = "mqa_fp8_decode_B8_L32768"
        if mqa in breakdown:
            breakdown[mqa]["cpu_baseline"] = _with_ratio(cpu_baseline_decode(W.WORKLOADS[mqa](0), budget_s=5.0),
                                                         breakdown[mqa]["kv_read_GBps"])
        log(f"[bench] cpu baseline: {json.dumps(cpu)}")

    if is_prefill:
        value, unit, dtype = head["tflops"], "TFLOP/s", "bf16"
    else:
        value, unit = head["kv_read_GBps"], "GB/s"
        dtype = {W.BF16: "bf16", W.FP8: "fp8_e4m3fn", W.F32: "f32", W.INT4: "int4"}[case.kv_dtype]
    cfg = {"workload": args.workload, "global_batch": case.B, "heads": case.H, "kv_heads": case.G,
           "head_dim": case.D, "parallelism": "none (1 GPU)"}
    if isinstance(case, (W.ChunkCase, W.PagedChunkCase)):
        cfg["seq_len"], cfg["chunk_len"] = case.T_cap, case.Tq
    elif is_prefill:
        cfg["seq_len"] = case.T
    else:
        cfg["kv_cache_len"] = case.T_cap
        cfg["sum_seq_lens"] = int(case.seq_lens.clamp(0, case.T_cap).sum())
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded N(0,1))",
        "config": cfg,
        "tok_per_s": head.get("tok_per_s"),
        "hbm_frac": (value / HBM_PEAK_GBS) if not is_prefill else None,
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "prefill": prefill,
        "hbm_achievable": achievable,
        "detail": head,
        "breakdown": breakdown,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
