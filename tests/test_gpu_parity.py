"""HIP path vs the fp64 oracle, element by element, through the C ABI (needs a gfx950 GPU).

Tolerances (max abs error): fp32 inputs 1e-5, bf16 inputs with fp32 accumulation
2e-2, fp8-E4M3FN KV 5e-2 (the oracle sees the same dequantised values).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-5, W.BF16: 2e-2, W.FP8: 5e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def dev_decode(gqa, case, path="auto", num_splits=0, out=None, layout="auto"):
    d = "cuda"
    ks = case.k_scale.to(d) if case.k_scale is not None else None
    vs = case.v_scale.to(d) if case.v_scale is not None else None
    _say(f"[gpu] decode {case.name} B{case.B} H{case.H} G{case.G} D{case.D} T_cap{case.T_cap} "
         f"kv={case.kv_dtype} path={path} splits={num_splits} layout={layout}")
    o = gqa.decode(case.q.to(d), case.k_cache.to(d), case.v_cache.to(d), case.seq_lens.to(d), out=out,
                   scale=case.scale, k_scale=ks, v_scale=vs, num_splits=num_splits, path=path, layout=layout)
    torch.cuda.synchronize()
    return o


def dev_prefill(gqa, case, path="auto"):
    d = "cuda"
    _say(f"[gpu] prefill {case.name} B{case.B} H{case.H} G{case.G} D{case.D} T{case.T} "
         f"causal={case.causal} dtype={case.dtype} path={path}")
    o = gqa.prefill(case.q.to(d), case.k.to(d), case.v.to(d), scale=case.scale, causal=case.causal, path=path)
    torch.cuda.synchronize()
    return o


def check(got, want, tol, what):
    got = got.detach().cpu().to(torch.float64).numpy()
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want)))
    _say(f"    {what}: max abs err {err:.3e} (tol {tol})")
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


DECODE_PATHS = ["generic", "valu", "mfma"]


def supported(gqa, case, path):
    """Whether a forced path accepts these shapes (host-side check only)."""
    if path == "generic":
        return True
    if case.D != 128:
        return False
    if path == "valu":
        return case.kv_dtype == W.BF16 and case.q_dtype == W.BF16
    return case.q_dtype == W.BF16 and case.kv_dtype in (W.BF16, W.FP8)


def run_all_paths(gqa, case, want, splits=(0,)):
    """Every kernel family that takes these shapes, at each split count; with the library's own
    split choice (0) the matrix-core family also runs in both work layouts."""
    ran = 0
    for path in DECODE_PATHS:
        if not supported(gqa, case, path):
            continue
        runs = [(s, "auto") for s in splits]
        if path == "mfma" and 0 in splits:
            runs += [(0, "uniform"), (0, "flat")]
        for s, layout in runs:
            try:
                got = dev_decode(gqa, case, path=path, num_splits=s, layout=layout)
            except gqa.GqaError as e:
                if e.status == 2 and path != "generic":   # kernel family not built for these shapes
                    _say(f"    {path}: unsupported, skipped")
                    break
                raise
            check(got, want, TOL[case.kv_dtype], f"{case.name} path={path} splits={s} layout={layout}")
            ran += 1
    assert ran > 0


# ---------------------------------------------------------------------------------------
# The five named workloads at full size.
# ---------------------------------------------------------------------------------------

def test_toy_prefill_then_two_decode_steps(gqa):
    p = W.toy_prefill(0)
    check(dev_prefill(gqa, p), oracle.prefill(p), TOL[W.F32], "toy prefill T=5")
    for step in W.toy_decode_steps(0):
        run_all_paths(gqa, step, oracle.decode(step), splits=(0, 1, 2, 7))


def test_llama7b_gqa8_decode(gqa):
    c = W.llama7b_gqa8_decode(0)
    run_all_paths(gqa, c, oracle.decode(c))


def test_llama70b_ragged_decode(gqa):
    c = W.llama70b_ragged_decode(0)
    assert int(c.seq_lens.sum()) == 40165
    run_all_paths(gqa, c, oracle.decode(c))


def test_mqa_fp8_long_decode(gqa):
    c = W.mqa_fp8_long_decode(0)
    run_all_paths(gqa, c, oracle.decode(c))


@pytest.fixture(scope="module")
def causal_prefill_2048_want():
    """The oracle's whole output for the B4 H32 G8 D128 T2048 causal prefill (fp64, every row;
    seconds on the host cores), computed once for the tests below."""
    c = W.causal_prefill_2048(0)
    return c, oracle.prefill(c)


@pytest.mark.parametrize("path", ["auto", "generic"])
def test_causal_prefill_2048(gqa, causal_prefill_2048_want, path):
    """Every one of the B * H * T = 262 144 output rows (all 128 head dims) against the oracle,
    in the launch configuration the benchmark times (auto path: the matrix-core kernel)."""
    c, want = causal_prefill_2048_want
    got = dev_prefill(gqa, c, path=path)
    check(got, want, TOL[W.BF16], f"prefill B4 H32 T2048 causal path={path}, all rows")


# ---------------------------------------------------------------------------------------
# Ragged, multi-tile and degenerate decode cases.
# ---------------------------------------------------------------------------------------

DECODE_CASES = [
    # B, H, G, D, seq_lens, T_cap, q_dtype, kv_dtype
    (2, 8, 2, 128, [1, 77], 96, W.BF16, W.BF16),
    (3, 32, 8, 128, [300, 1, 1023], 1100, W.BF16, W.BF16),
    (2, 64, 8, 128, [4096, 1500], 4096, W.BF16, W.BF16),
    (2, 16, 16, 128, [129, 257], 300, W.BF16, W.BF16),       # MHA (G = H)
    (2, 32, 1, 128, [5000, 65], 5000, W.BF16, W.BF16),       # MQA bf16
    (2, 32, 1, 128, [2049, 700], 2100, W.BF16, W.FP8),       # MQA fp8
    (3, 16, 2, 128, [1, 333, 1024], 1024, W.BF16, W.FP8),
    (1, 12, 3, 64, [517], 600, W.BF16, W.BF16),              # head dim 64 (generic)
    (2, 6, 3, 80, [40, 3], 41, W.F32, W.F32),                # odd sizes, fp32
    (1, 4, 2, 3, [7], 7, W.F32, W.F32),
    # Batches of many ragged sequences (the balanced flat layout of the matrix-core path):
    # more than 64 sequences, empty ones and one-key ones among them.
    (70, 8, 2, 128, [0 if i % 9 == 4 else (1 if i % 11 == 3 else (i * 37) % 300 + 1) for i in range(70)],
     300, W.BF16, W.BF16),
    (67, 32, 1, 128, [0 if i % 7 == 2 else (i * 53) % 200 + 1 for i in range(67)], 200, W.BF16, W.FP8),
    (5, 64, 1, 128, [700, 0, 1, 333, 64], 700, W.BF16, W.BF16),   # 64 heads per KV head
    (4, 16, 2, 128, [0, 0, 0, 0], 50, W.BF16, W.BF16),             # no keys at all
]


@pytest.mark.parametrize("B,H,G,D,lens,T_cap,qd,kvd", DECODE_CASES)
def test_decode_cases(gqa, B, H, G, D, lens, T_cap, qd, kvd):
    c = W.make_decode(B, H, G, D, lens, T_cap=T_cap, q_dtype=qd, kv_dtype=kvd, seed=B * 7 + H + D,
                      name=f"decode_B{B}H{H}G{G}D{D}")
    run_all_paths(gqa, c, oracle.decode(c), splits=(0, 1, 3))


@pytest.mark.parametrize("B,kvd", [(256, W.BF16), (257, W.BF16), (600, W.BF16), (600, W.FP8), (300, W.INT4)])
def test_decode_flat_large_batches(gqa, B, kvd):
    """The flat layout past the 256 lengths a workgroup keeps in LDS: from 257 sequences on, the
    lengths, the first segment of a run and every later segment are read from memory. Ragged
    lengths 1..120 with empty sequences between them."""
    lens = [0 if i % 13 == 5 else (i * 29) % 120 + 1 for i in range(B)]
    c = W.make_decode(B, 8, 2, 128, lens, T_cap=128, kv_dtype=kvd, seed=B + 5, name=f"flat_B{B}")
    want = oracle.decode(c)
    for layout in ("flat", "auto"):
        check(dev_decode(gqa, c, layout=layout), want, TOL.get(kvd, 5e-2), f"{c.name} {kvd} layout={layout}")


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 1024])
def test_decode_forced_splits(gqa, splits):
    """Split counts from one to far more than there are keys (empty splits)."""
    c = W.make_decode(2, 16, 2, 128, [200, 31], T_cap=256, seed=3, name="splits")
    run_all_paths(gqa, c, oracle.decode(c), splits=(splits,))


def test_decode_length_readings(gqa):
    """seq_lens <= 0 gives a zero row; seq_lens > T_cap reads T_cap rows."""
    c = W.make_decode(3, 8, 2, 128, [64, 64, 64], T_cap=64, seed=5, name="lens")
    c.seq_lens = torch.tensor([0, 1000, -4], dtype=torch.int32)
    want = oracle.decode(c)
    assert np.all(want[0] == 0) and np.all(want[2] == 0)
    run_all_paths(gqa, c, want, splits=(0, 1, 4))


def test_decode_scale_and_constant_values(gqa):
    """V constant per KV head -> every head of group g outputs g + 1 (pins the group map)."""
    c = W.make_decode(2, 16, 4, 128, [100, 37], T_cap=128, seed=9, name="vconst", poison=False)
    for g in range(4):
        c.v_cache[:, g] = float(g + 1)
    want = oracle.decode(c)
    for h in range(16):
        assert np.allclose(want[:, h], h // 4 + 1)
    run_all_paths(gqa, c, want)


def test_decode_deterministic(gqa):
    c = W.make_decode(4, 32, 8, 128, "uniform:1:3000", T_cap=3000, seed=11, name="determinism")
    for path, layout in [(p, "auto") for p in DECODE_PATHS] + [("mfma", "flat")]:
        if not supported(gqa, c, path):
            continue
        try:
            a = dev_decode(gqa, c, path=path, layout=layout).clone()
        except gqa.GqaError as e:
            if e.status == 2:
                continue
            raise
        for _ in range(3):
            b = dev_decode(gqa, c, path=path, layout=layout)
            assert torch.equal(a, b), f"path {path} layout {layout} not bitwise reproducible"


# ---------------------------------------------------------------------------------------
# Prefill cases.
# ---------------------------------------------------------------------------------------

PREFILL_CASES = [
    # B, H, G, D, T, causal, dtype
    (1, 4, 2, 3, 5, True, W.F32),
    (2, 8, 2, 128, 200, True, W.BF16),
    (1, 8, 2, 128, 200, False, W.BF16),
    (1, 32, 8, 128, 517, True, W.BF16),
    (2, 4, 4, 128, 129, True, W.BF16),      # MHA
    (1, 8, 1, 128, 300, True, W.BF16),      # MQA
    (1, 8, 1, 128, 64, False, W.BF16),
    (1, 2, 1, 128, 1, True, W.BF16),        # a single position
    (1, 6, 3, 96, 70, True, W.F32),
    (1, 4, 2, 64, 100, False, W.BF16),
    (1, 28, 4, 128, 300, True, W.BF16),     # R = 7 (query heads per KV head not a power of two)
    (2, 40, 8, 128, 130, False, W.BF16),    # R = 5
    (1, 36, 3, 128, 257, True, W.BF16),     # R = 12
    (1, 48, 1, 128, 70, True, W.BF16),      # R = 48: two positions per workgroup
]


@pytest.mark.parametrize("B,H,G,D,T,causal,dt", PREFILL_CASES)
def test_prefill_cases(gqa, B, H, G, D, T, causal, dt):
    c = W.make_prefill(B, H, G, D, T, dtype=dt, causal=causal, seed=T + D, name=f"prefill_B{B}H{H}G{G}D{D}T{T}")
    want = oracle.prefill(c)
    paths = ("auto", "generic") + (("mfma",) if D == 128 and dt == W.BF16 else ())
    for path in paths:
        check(dev_prefill(gqa, c, path=path), want, TOL[dt], f"{c.name} causal={causal} path={path}")


def test_decode_matches_prefill_rows(gqa):
    """Incremental decode over the growing cache equals the causal prefill row."""
    B, H, G, D, T = 1, 32, 8, 128, 300
    p = W.make_prefill(B, H, G, D, T, seed=21, name="inc")
    d = "cuda"
    full = dev_prefill(gqa, p).float().cpu()
    kc, vc = p.k.to(d), p.v.to(d)
    for t in (0, 1, 63, 64, 200, T - 1):
        lens = torch.tensor([t + 1], dtype=torch.int32, device=d)
        o = gqa.decode(p.q[:, :, t].contiguous().to(d), kc, vc, lens, scale=p.scale)
        torch.cuda.synchronize()
        err = float((o.float().cpu() - full[:, :, t]).abs().max())
        assert err <= 2e-2, f"step {t}: {err}"
