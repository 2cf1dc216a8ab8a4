"""INT4 KV cache vs the oracle, through the C ABI (needs a gfx950 GPU).

The oracle decodes the same packed fields with the same per-(sequence, KV head) scales, so the
tolerance is the one for quantised caches (5e-2). Padding rows hold the largest field (0xFF),
which changes the result if a kernel reads them. Covered: the matrix-core family in both
layouts and at forced split counts, the generic family (head dims 64 and 80), paged caches,
R up to 64, ragged and empty sequences; and the cache append, byte-exact, including every bf16
bit pattern through the INT4 encoder.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = 5e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def check(got, want, what):
    got = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want)))
    _say(f"    {what}: max abs err {err:.3e}")
    assert err <= TOL, f"{what}: {err} > {TOL}"


def dev_decode(gqa, c, path="auto", layout="auto", num_splits=0, k_new=None, v_new=None):
    d = "cuda"
    _say(f"[gpu] int4 {c.name} B{c.B} H{c.H} G{c.G} D{c.D} T_cap{c.T_cap} path={path} layout={layout} "
         f"splits={num_splits} append={k_new is not None}")
    kc, vc = c.k_cache.to(d), c.v_cache.to(d)
    out = gqa.decode(c.q.to(d), kc, vc, c.seq_lens.to(d), scale=c.scale, k_scale=c.k_scale.to(d),
                     v_scale=c.v_scale.to(d), path=path, layout=layout, num_splits=num_splits,
                     k_new=None if k_new is None else k_new.to(d), v_new=None if v_new is None else v_new.to(d))
    torch.cuda.synchronize()
    return out, kc, vc


RUNS = [("auto", "auto", 0), ("mfma", "uniform", 0), ("mfma", "flat", 0), ("mfma", "uniform", 1),
        ("mfma", "uniform", 5), ("generic", "auto", 0), ("generic", "auto", 3)]

INT4_CASES = [
    # B, H, G, D, seq_lens, T_cap
    (2, 32, 8, 128, [1000, 77], 1024),
    (3, 16, 2, 128, [1, 333, 1024], 1024),
    (2, 32, 1, 128, [2049, 700], 2100),                  # MQA, two head blocks
    (5, 64, 1, 128, [700, 0, 1, 333, 64], 700),          # R = 64, an empty sequence
    (40, 8, 2, 128, [0 if i % 9 == 4 else (i * 37) % 300 + 1 for i in range(40)], 300),
    (2, 12, 3, 64, [517, 40], 600),                      # generic only
    (1, 8, 2, 80, [129], 130),
]


@pytest.mark.parametrize("B,H,G,D,lens,T_cap", INT4_CASES)
def test_int4_decode(gqa, B, H, G, D, lens, T_cap):
    c = W.make_decode(B, H, G, D, lens, T_cap=T_cap, kv_dtype=W.INT4, seed=B + H + D, name=f"i4_B{B}H{H}G{G}D{D}")
    want = oracle.decode(c)
    ran = 0
    for path, layout, splits in RUNS:
        if D != 128 and path == "mfma":
            continue
        try:
            out, _, _ = dev_decode(gqa, c, path, layout, splits)
        except gqa.GqaError as e:
            if e.status == 2 and layout == "flat":
                continue
            raise
        check(out, want, f"{c.name} path={path} layout={layout} splits={splits}")
        ran += 1
    assert ran >= 2


@pytest.mark.parametrize("ps", [16, 64])
def test_int4_paged(gqa, ps):
    c = W.make_decode(6, 32, 8, 128, [900, 1, 0, 257, 512, 64], T_cap=1024, kv_dtype=W.INT4, seed=ps, name="i4p")
    p = W.make_paged(c, ps, seed=ps + 2)
    want = oracle.decode_paged(p)
    d = "cuda"
    for layout, splits in [("auto", 0), ("uniform", 0), ("flat", 0), ("uniform", 3)]:
        _say(f"[gpu] int4 paged page{ps} layout={layout} splits={splits}")
        out = gqa.decode_paged(p.q.to(d), p.k_pages.to(d), p.v_pages.to(d), p.block_table.to(d), p.seq_lens.to(d),
                               scale=p.scale, k_scale=p.k_scale.to(d), v_scale=p.v_scale.to(d), layout=layout,
                               num_splits=splits)
        torch.cuda.synchronize()
        check(out, want, f"paged page{ps} layout={layout} splits={splits}")


def test_int4_append(gqa):
    c = W.make_decode(3, 32, 8, 128, [1, 500, 1024], T_cap=1024, kv_dtype=W.INT4, seed=4, name="i4_app")
    g = torch.Generator().manual_seed(4)
    kn = (torch.randn(3, 8, 128, generator=g) * 2).to(torch.bfloat16)
    vn = (torch.randn(3, 8, 128, generator=g) * 2).to(torch.bfloat16)
    kc_want, vc_want = oracle.append(c, kn, vn)
    appended = W.DecodeCase(**{**c.__dict__, "k_cache": kc_want, "v_cache": vc_want})
    want = oracle.decode(appended)
    for path, layout in [("auto", "auto"), ("mfma", "flat"), ("generic", "auto")]:
        out, kc, vc = dev_decode(gqa, c, path, layout, k_new=kn, v_new=vn)
        assert torch.equal(kc.cpu(), kc_want) and torch.equal(vc.cpu(), vc_want), f"{path}/{layout}: cache bytes"
        check(out, want, f"append path={path} layout={layout}")


def test_int4_append_every_bf16_value(gqa):
    """All 65536 bf16 patterns (NaN and infinities included) through the INT4 append: the stored
    fields equal the oracle's encoder, bit for bit."""
    B, G, D = 64, 8, 128
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    kn = pats.reshape(B, G, D)
    vn = pats.flip(0).reshape(B, G, D).contiguous()
    c = W.make_decode(B, 8, G, D, 1, T_cap=1, kv_dtype=W.INT4, seed=3, name="i4_all")
    c.k_scale = torch.full((B * G,), 0.75, dtype=torch.float32)
    c.v_scale = torch.linspace(0.01, 3.0, B * G, dtype=torch.float32)
    kc_want, vc_want = oracle.append(c, kn, vn)
    _, kc, vc = dev_decode(gqa, c, "auto", k_new=kn, v_new=vn)
    for got, want, name in ((kc, kc_want, "K"), (vc, vc_want, "V")):
        bad = torch.nonzero(got.cpu().reshape(-1) != want.reshape(-1)).reshape(-1)
        if bad.numel():
            i = int(bad[0])
            _say(f"    {name}: {bad.numel()} bytes differ; first at {i}: got {int(got.cpu().reshape(-1)[i]):#04x} "
                 f"want {int(want.reshape(-1)[i]):#04x}")
        assert bad.numel() == 0, f"{name} fields differ"
