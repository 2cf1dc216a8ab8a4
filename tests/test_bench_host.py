"""Host logic of bench.py, on the CPU: the algorithmic work a roofline divides by, the
rocprofv3 summaries kept under profiles/, the rule that recorded traffic goes stale when the
kernel sources change, and the refusal of more than one GPU. No kernel runs here."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ---- algorithmic work ------------------------------------------------------------------

def test_decode_bytes_llama7b_shape():
    # B1 H32 G8 D128, 2048 bf16 tokens: K and V 2 * 2048 * 8 * 128 * 2 bytes, q and out
    # 2 * 32 * 128 * 2, one int32 length.
    c = W.make_decode(1, 32, 8, 128, 2048)
    by = bench.decode_bytes(c)
    assert by["kv"] == 8_388_608
    assert by["total"] == 8_388_608 + 16_384 + 4


def test_decode_bytes_counts_valid_rows_only():
    # Ragged lengths with a large capacity: only rows below each length count; a length past
    # the capacity counts as the capacity, a non-positive one as zero.
    c = W.make_decode(4, 8, 2, 16, [5, 0, 40, -3], T_cap=32)
    by = bench.decode_bytes(c)
    assert by["kv"] == 2 * (5 + 0 + 32 + 0) * 2 * 16 * 2
    assert by["total"] == by["kv"] + 2 * 4 * 8 * 16 * 2 + 4 * 4


@pytest.mark.parametrize("kv_dtype, row_bytes", [(W.FP8, 16), (W.INT4, 8)])
def test_decode_bytes_narrow_caches_add_their_scales(kv_dtype, row_bytes):
    c = W.make_decode(2, 4, 1, 16, [6, 9], kv_dtype=kv_dtype)
    by = bench.decode_bytes(c)
    assert by["kv"] == 2 * (6 + 9) * 1 * row_bytes
    # q and out in bf16, two lengths, a k and a v scale per (sequence, KV head)
    assert by["total"] == by["kv"] + 2 * 2 * 4 * 16 * 2 + 2 * 4 + 2 * 2 * 4


def test_decode_bytes_with_append_adds_the_new_rows():
    c = W.make_decode(2, 4, 2, 16, [3, 7], T_cap=8)
    plain, app = bench.decode_bytes(c), bench.decode_bytes(c, append=True)
    # a K and a V row per (sequence, KV head), read in q's dtype and written in the cache's
    # (both bf16)
    assert app["total"] - plain["total"] == 2 * (2 * 2) * 16 * (2 + 2)


def test_prefill_flops_closed_form_and_brute_force():
    # The causal prefill of the benchmark: 4 * B * H * D * T (T + 1) / 2.
    assert 4 * 4 * 32 * 128 * (2048 * 2049 // 2) == 137_506_062_336
    c = W.make_prefill(2, 4, 2, 8, 5)
    pairs = sum(1 for i in range(5) for j in range(5) if j <= i)
    assert bench.prefill_flops(c) == 4 * 2 * 4 * 8 * pairs
    c.causal = False
    assert bench.prefill_flops(c) == 4 * 2 * 4 * 8 * 25


@pytest.mark.parametrize("causal", [True, False])
def test_chunk_flops_brute_force(causal):
    # Query i of a chunk of Tq sits at position L - Tq + i and sees keys up to it (causal) or
    # all L; a query before position 0 sees nothing.
    Tq, lens = 4, [6, 2, 4]
    c = W.make_chunk(3, 4, 2, 8, Tq, lens, causal=causal)
    pairs = 0
    for L in lens:
        for i in range(Tq):
            p = L - Tq + i
            pairs += sum(1 for j in range(L) if (j <= p or not causal))
    assert bench.chunk_flops(c) == 4 * 4 * 8 * pairs


def test_derived_workloads_resolve():
    c, append = bench.derived_case("llama7b_gqa8_decode_L2048+append")
    assert isinstance(c, W.DecodeCase) and append and c.name == "llama7b_gqa8_decode_L2048"
    c, append = bench.derived_case("llama7b_gqa8_decode_L2048_paged16")
    assert isinstance(c, W.PagedDecodeCase) and not append and c.name == "llama7b_gqa8_decode_L2048_paged16"
    # the traffic key of a derived entry is its name
    assert {"llama7b_gqa8_decode_L2048+append", "llama7b_gqa8_decode_L2048_paged16",
            "gqa8_chunked_prefill_B4_Tq512_L4096_paged16"} <= set(bench.DERIVED_WORKLOADS)


# ---- rocprofv3 summaries ---------------------------------------------------------------

def _write_csv(path, fieldnames, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fieldnames)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_trace_takes_the_last_dispatches(tmp_path):
    # Kernel A: 3 early (warm-up) dispatches of 100 us, then 5 timed ones of 1..5 us; the
    # rows are out of order in the file. Kernel B: one dispatch.
    rows, t = [], 0
    for d in [100, 100, 100, 3, 1, 5, 2, 4]:
        rows.append({"Kernel_Name": "A", "Start_Timestamp": t, "End_Timestamp": t + d * 1000, "Dispatch_Id": len(rows)})
        t += 200_000
    rows.append({"Kernel_Name": "B", "Start_Timestamp": 5, "End_Timestamp": 7005, "Dispatch_Id": 99})
    rows.reverse()
    p = tmp_path / "trace.csv"
    _write_csv(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Dispatch_Id"], rows)
    res = bench.summarize_trace(str(p), 5)
    assert res["A"]["dispatches"] == 8 and res["A"]["timed"] == 5
    assert res["A"]["median_us"] == 3.0 and res["A"]["min_us"] == 1.0 and res["A"]["max_us"] == 5.0
    assert res["A"]["mean_us"] == pytest.approx(3.0)
    assert res["B"]["timed"] == 1 and res["B"]["median_us"] == 7.0


def test_summarize_counters_sums_each_dispatch_then_takes_medians(tmp_path):
    # Two rows per dispatch (counter instances) add up; the last 3 dispatches are kept.
    f_rows, w_rows = [], []
    for did, (fa, wa) in enumerate([(1000, 1000), (10, 1), (20, 2), (30, 3)]):
        for part in (0.25, 0.75):
            f_rows.append({"Kernel_Name": "k", "Dispatch_Id": did, "Counter_Name": "FETCH_SIZE", "Counter_Value": fa * part})
            w_rows.append({"Kernel_Name": "k", "Dispatch_Id": did, "Counter_Name": "WRITE_SIZE", "Counter_Value": wa * part})
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    names = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    _write_csv(fp, names, f_rows)
    _write_csv(wp, names, w_rows)
    res = bench.summarize_counters(str(fp), str(wp), 3)
    assert res["k"] == {"fetch_kib_median": 20.0, "write_kib_median": 2.0}


def test_summarize_pmc_per_counter_medians(tmp_path):
    rows = []
    for did, (u, v) in enumerate([(90, 9), (1, 10), (2, 20), (3, 30)]):
        rows.append({"Kernel_Name": "k", "Dispatch_Id": did, "Counter_Name": "MfmaUtil", "Counter_Value": u})
        rows.append({"Kernel_Name": "k", "Dispatch_Id": did, "Counter_Name": "LdsUtil", "Counter_Value": v})
    p = tmp_path / "pmc.csv"
    _write_csv(p, ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"], rows)
    res = bench.summarize_pmc(str(p), 3)
    assert res["k"] == {"MfmaUtil": 2.0, "LdsUtil": 20.0}


def test_recorded_traffic_goes_stale_when_the_sources_change(tmp_path, monkeypatch):
    rec = {"copy_calibration": {"fetch_scale": 2.0, "write_scale": 1.0},
           "workloads": {"w_decode": {"traffic_bytes_per_launch": 123.0,
                                      "sources_sha256": bench.kernel_sources_sha256("decode")},
                         "w_prefill": {"traffic_bytes_per_launch": 456.0, "sources_sha256": "0" * 64}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic("w_decode") == 123.0
    assert bench.measured_traffic("w_prefill") is None  # taken on other prefill sources
    assert bench.measured_traffic("absent") is None
    p.write_text("not json")
    assert bench.measured_traffic("w_decode") is None


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    monkeypatch.setattr(bench, "CSRC", str(src))
    monkeypatch.setattr(bench, "_FAMILY_SOURCES", {"decode": ("k.hip", "h.h")})
    (src / "h.h").write_text("#pragma once\nconstexpr int kN = 4;  // four\n")
    (src / "k.hip").write_text("/* a kernel */\nint f(int x) { return x + kN; }  // plus\n")
    h0 = bench.kernel_sources_sha256("decode")
    (src / "k.hip").write_text("/* the same kernel,\n   other words */\nint f(int x) { return x + kN; }\n// done\n")
    assert bench.kernel_sources_sha256("decode") == h0
    (src / "k.hip").write_text("/* a kernel */\nint f(int x) { return x - kN; }  // plus\n")
    assert bench.kernel_sources_sha256("decode") != h0
    (src / "k.hip").write_text("/* a kernel */\nint f(int x) { return x + kN; }  // plus\n")
    (src / "h.h").write_text("#pragma once\nconstexpr int kN = 5;  // four\n")
    assert bench.kernel_sources_sha256("decode") != h0


def test_committed_traffic_records_name_their_sources():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    cal = rec["copy_calibration"]
    assert cal["fetch_scale"] > 0 and cal["write_scale"] > 0
    for name, w in rec["workloads"].items():
        assert len(w["sources_sha256"]) == 64, name
        assert w["traffic_bytes_per_launch"] > 0, name
        assert all("gqa::" in k for k in w["kernels"]), name


def test_timeline_summary_of_synthetic_stamps():
    import numpy as np
    a = np.zeros((4096, 32), dtype=np.uint64)
    # three workgroups, clock ticks of 10 ns: entries at 0, 50, 100; one piece each (slots 2-7),
    # the third merged last (arrival at +4); exits at 2000, 2500, 3000 ticks
    for w in range(3):
        base = 1000 + 50 * w
        a[w, 0] = base
        a[w, 1] = base + 100
        a[w, 2:8] = [base + 100, base + 300, base + 800, base + 900, base + 950, base + 960 + 400 * (w == 2)]
        a[w, 20] = base + 1000 + 450 * w
        a[w, 21] = 1
        a[w, 22] = base + 850   # waves done 0.5 us after wave 0's loop
        a[w, 23] = base + 870   # partial sums written 0.2 us later
    # placement: XCC 0 CU 1, XCC 1 CU 1, and the third workgroup on that same CU of XCC 1
    # (HW_ID: CU in bits 11:8; XCC_ID above bit 32)
    a[0, 31] = 1 << 8
    a[1, 31] = (1 << 32) | (1 << 8)
    a[2, 31] = (1 << 32) | (1 << 8)
    lines = bench.timeline_summary(a, "synthetic")
    text = "\n".join(lines)
    assert "3 workgroups, span 20.00 us" in lines[0]   # last exit 3000 ticks, first entry 1000
    entry = next(l for l in lines if l.strip().startswith("entry"))
    assert entry.split()[1:] == ["0.00", "0.10", "0.50", "0.90", "1.00"]
    loop = next(l for l in lines if "block loop done ->" in l)
    assert loop.split()[-5:] == ["2.00", "2.90", "6.50", "10.10", "11.00"]
    assert "workgroups with 1 piece(s):    3" in text
    waves = next(l for l in lines if "the other waves done" in l)
    assert waves.split()[-5:] == ["0.50"] * 5
    sums = next(l for l in lines if "partial sums written" in l)
    assert sums.split()[-5:] == ["0.20"] * 5
    place = next(l for l in lines if "placement" in l)
    assert "2 CUs used, CUs by workgroups held {1: 1, 2: 1}" in place
    assert "blockIdx mod 8 for 2 of 3 workgroups" in place


# ---- one GPU only ------------------------------------------------------------------------

@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
