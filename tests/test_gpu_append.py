"""Decode with cache append vs the oracle, through the C ABI (needs a gfx950 GPU).

The call stores the current token's key and value at row seq_lens[b]-1 and attends over the
cache including that row. Checked on every kernel family and work layout:
  * the caches afterwards equal oracle.append's byte for byte (the appended row, and every
    other row untouched -- NaN-poisoned rows included, compared as bytes);
  * the output equals the oracle's decode over the appended caches (same tolerances as the
    decode parity tests);
  * the row is never read before it is written: the input caches hold NaN at row L-1.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-5, W.BF16: 2e-2, W.FP8: 5e-2}
TORCH_DT = {W.F32: torch.float32, W.BF16: torch.bfloat16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def _bytes(t):
    return t.detach().cpu().contiguous().view(torch.uint8)


def poison_append_rows(case):
    """NaN at row L-1 of every (b, g) that will receive the new token."""
    nan_code = 0x7F
    for b in range(case.B):
        L = int(case.seq_lens[b])
        if 1 <= L <= case.T_cap:
            if case.kv_dtype == W.FP8:
                case.k_cache.view(torch.uint8)[b, :, L - 1] = nan_code
                case.v_cache.view(torch.uint8)[b, :, L - 1] = nan_code
            else:
                case.k_cache[b, :, L - 1] = float("nan")
                case.v_cache[b, :, L - 1] = float("nan")


def new_rows(case, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    dt = TORCH_DT[case.q_dtype]
    kn = (torch.randn(case.B, case.G, case.D, generator=g) * scale).to(dt)
    vn = (torch.randn(case.B, case.G, case.D, generator=g) * scale).to(dt)
    return kn, vn


def run_append(gqa, case, kn, vn, path, layout="auto", num_splits=0, misalign=False):
    d = "cuda"
    kc, vc = case.k_cache.to(d), case.v_cache.to(d)
    ks = case.k_scale.to(d) if case.k_scale is not None else None
    vs = case.v_scale.to(d) if case.v_scale is not None else None
    kd, vd = kn.to(d), vn.to(d)
    if misalign:  # rows that start 2 bytes past a 16-byte boundary
        n = kn.numel()
        kb = torch.empty(n + 8, dtype=kn.dtype, device=d)
        vb = torch.empty(n + 8, dtype=vn.dtype, device=d)
        kd = kb[1:1 + n].view(kn.shape)
        vd = vb[1:1 + n].view(vn.shape)
        kd.copy_(kn.to(d))
        vd.copy_(vn.to(d))
        assert kd.data_ptr() % 16 != 0
    _say(f"[gpu] append {case.name} B{case.B} H{case.H} G{case.G} D{case.D} T_cap{case.T_cap} "
         f"kv={case.kv_dtype} path={path} layout={layout} splits={num_splits} misalign={misalign}")
    out = gqa.decode(case.q.to(d), kc, vc, case.seq_lens.to(d), scale=case.scale, k_scale=ks, v_scale=vs,
                     path=path, layout=layout, num_splits=num_splits, k_new=kd, v_new=vd)
    torch.cuda.synchronize()
    return out, kc, vc


def supported(case, path):
    if path == "generic":
        return True
    if case.D != 128 or case.q_dtype != W.BF16:
        return False
    if path == "valu":
        return case.kv_dtype == W.BF16
    return case.kv_dtype in (W.BF16, W.FP8)


def check_append(gqa, case, kn, vn, runs):
    kc_want, vc_want = oracle.append(case, kn, vn)
    appended = W.DecodeCase(**{**case.__dict__, "k_cache": kc_want, "v_cache": vc_want})
    want = oracle.decode(appended)
    ran = 0
    for path, layout, splits, misalign in runs:
        if not supported(case, path):
            continue
        try:
            out, kc, vc = run_append(gqa, case, kn, vn, path, layout, splits, misalign)
        except gqa.GqaError as e:
            if e.status == 2 and path != "generic":
                _say(f"    {path}/{layout}: unsupported, skipped")
                continue
            raise
        what = f"{case.name} path={path} layout={layout} splits={splits} misalign={misalign}"
        assert torch.equal(_bytes(kc), _bytes(kc_want)), f"{what}: K cache differs from the oracle's append"
        assert torch.equal(_bytes(vc), _bytes(vc_want)), f"{what}: V cache differs from the oracle's append"
        got = out.detach().cpu().to(torch.float64).numpy()
        assert np.all(np.isfinite(got)), f"{what}: non-finite output"
        err = float(np.max(np.abs(got - want)))
        _say(f"    {what}: caches exact, max abs err {err:.3e}")
        assert err <= TOL[case.kv_dtype], f"{what}: {err}"
        ran += 1
    assert ran > 0


ALL_RUNS = [("generic", "auto", 0, False), ("valu", "auto", 0, False), ("mfma", "auto", 0, False),
            ("mfma", "uniform", 0, False), ("mfma", "flat", 0, False), ("mfma", "uniform", 1, False),
            ("mfma", "uniform", 5, False), ("generic", "auto", 3, False), ("mfma", "auto", 0, True)]

APPEND_CASES = [
    # B, H, G, D, seq_lens, T_cap, q_dtype, kv_dtype
    (2, 32, 8, 128, [1000, 77], 1024, W.BF16, W.BF16),
    (3, 16, 2, 128, [1, 333, 1024], 1024, W.BF16, W.FP8),        # L = 1 and L = T_cap
    (2, 32, 1, 128, [2049, 700], 2100, W.BF16, W.FP8),           # MQA fp8 (two head blocks)
    (5, 64, 1, 128, [700, 0, 1, 333, 64], 700, W.BF16, W.BF16),  # 64 heads per KV head, an empty sequence
    (2, 16, 16, 128, [129, 257], 300, W.BF16, W.BF16),           # MHA
    (2, 6, 3, 80, [40, 3], 41, W.F32, W.F32),                    # fp32, generic only
    (1, 12, 3, 64, [517], 600, W.BF16, W.BF16),                  # head dim 64, generic only
    # many ragged sequences: the flat layout's pieces, empty and one-key sequences among them
    (70, 8, 2, 128, [0 if i % 9 == 4 else (1 if i % 11 == 3 else (i * 37) % 300 + 1) for i in range(70)],
     300, W.BF16, W.BF16),
    (67, 32, 1, 128, [0 if i % 7 == 2 else (i * 53) % 200 + 1 for i in range(67)], 200, W.BF16, W.FP8),
]


@pytest.mark.parametrize("B,H,G,D,lens,T_cap,qd,kvd", APPEND_CASES)
def test_append_cases(gqa, B, H, G, D, lens, T_cap, qd, kvd):
    c = W.make_decode(B, H, G, D, lens, T_cap=T_cap, q_dtype=qd, kv_dtype=kvd, seed=B * 5 + H + D + 1,
                      name=f"append_B{B}H{H}G{G}D{D}")
    poison_append_rows(c)
    kn, vn = new_rows(c, seed=B + H)
    check_append(gqa, c, kn, vn, ALL_RUNS)


def test_append_out_of_range_lengths(gqa):
    """seq_lens <= 0 or > T_cap: nothing is written (and the output follows the decode readings)."""
    c = W.make_decode(4, 8, 2, 128, [64, 64, 64, 64], T_cap=64, seed=5, name="append_lens")
    c.seq_lens = torch.tensor([0, 1000, -4, 65], dtype=torch.int32)
    kn, vn = new_rows(c, seed=1)
    kc_want, vc_want = oracle.append(c, kn, vn)
    assert torch.equal(_bytes(kc_want), _bytes(c.k_cache))  # the oracle writes nothing either
    check_append(gqa, c, kn, vn, ALL_RUNS)


@pytest.mark.parametrize("B", [20, 300])
def test_append_out_of_range_lengths_in_batches(gqa, B):
    """The flat layout decides from the stored length whether row L-1 exists: from the lengths it
    keeps on chip for batches of up to 256 sequences (B = 20), from memory above that (B = 300).
    Lengths <= 0 and > T_cap sit among valid ones; only the valid ones are appended to."""
    T_cap = 64
    raw = [[0, -2, T_cap + 7, 1, T_cap, 33][i % 6] if i % 3 else (i * 13) % T_cap + 1 for i in range(B)]
    c = W.make_decode(B, 8, 2, 128, [min(max(x, 0), T_cap) for x in raw], T_cap=T_cap, seed=B, name=f"append_lens_B{B}")
    c.seq_lens = torch.tensor(raw, dtype=torch.int32)
    poison_append_rows(c)
    kn, vn = new_rows(c, seed=B + 1)
    check_append(gqa, c, kn, vn, [("mfma", "flat", 0, False), ("mfma", "auto", 0, False), ("generic", "auto", 0, False)])


def test_append_fp8_saturates(gqa):
    """New values far beyond the slab's scale saturate at +-448 * scale."""
    c = W.make_decode(2, 16, 2, 128, [100, 37], T_cap=128, kv_dtype=W.FP8, seed=8, name="append_sat")
    kn, vn = new_rows(c, seed=2, scale=1e4)
    codes = oracle.quant_e4m3fn(kn.float().numpy()[0, 0], float(c.k_scale[0]))
    assert np.any(codes == 0x7E) and np.any(codes == 0xFE)
    check_append(gqa, c, kn, vn, [("mfma", "auto", 0, False), ("generic", "auto", 0, False)])


@pytest.mark.parametrize("path", ["mfma", "generic"])
def test_append_fp8_every_bf16_value(gqa, path):
    """All 65536 bf16 bit patterns (NaN and infinities included) through the fp8 append: the
    stored codes equal the oracle's encoder, bit for bit. The output is not checked (it is NaN)."""
    B, G, D = 64, 8, 128
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    kn = pats.reshape(B, G, D)
    vn = pats.flip(0).reshape(B, G, D).contiguous()
    c = W.make_decode(B, 8, G, D, 1, T_cap=1, kv_dtype=W.FP8, seed=3, name="append_all_bf16")
    c.k_scale = torch.full((B * G,), 1.0, dtype=torch.float32)
    c.v_scale = torch.linspace(0.01, 3.0, B * G, dtype=torch.float32)
    kc_want, vc_want = oracle.append(c, kn, vn)
    _, kc, vc = run_append(gqa, c, kn, vn, path)
    for got, want, name in ((kc, kc_want, "K"), (vc, vc_want, "V")):
        gb, wb = _bytes(got).reshape(-1), _bytes(want).reshape(-1)
        bad = torch.nonzero(gb != wb).reshape(-1)
        if bad.numel():
            i = int(bad[0])
            x = (kn if name == "K" else vn).reshape(-1)[i]
            _say(f"    {name}: {bad.numel()} codes differ; first at {i}: x={float(x)!r} got {int(gb[i]):#04x} "
                 f"want {int(wb[i]):#04x}")
        assert bad.numel() == 0, f"{name} codes differ on {path}"


def test_append_decode_loop_matches_prefill(gqa):
    """A decode loop that appends each token itself reproduces the causal prefill rows."""
    B, H, G, D, T = 2, 32, 8, 128, 70
    p = W.make_prefill(B, H, G, D, T, seed=23, name="loop")
    d = "cuda"
    full = gqa.prefill(p.q.to(d), p.k.to(d), p.v.to(d), scale=p.scale).float().cpu()
    torch.cuda.synchronize()
    kc = torch.full((B, G, T, D), float("nan"), dtype=torch.bfloat16, device=d)
    vc = torch.full((B, G, T, D), float("nan"), dtype=torch.bfloat16, device=d)
    for t in range(T):
        lens = torch.full((B,), t + 1, dtype=torch.int32, device=d)
        o = gqa.decode(p.q[:, :, t].contiguous().to(d), kc, vc, lens, scale=p.scale,
                       k_new=p.k[:, :, t].contiguous().to(d), v_new=p.v[:, :, t].contiguous().to(d))
        torch.cuda.synchronize()
        err = float((o.float().cpu() - full[:, :, t]).abs().max())
        assert err <= 2e-2, f"step {t}: {err}"
    assert torch.equal(kc.cpu(), p.k) and torch.equal(vc.cpu(), p.v)
