"""Paged-cache decode vs the oracle, through the C ABI (needs a gfx950 GPU).

Cases are contiguous decode cases scattered into shuffled pages (workloads.make_paged, with
poison in every row that is not a valid cache row); the oracle gathers the logical cache
back through the table. Checked: every layout and forced split counts, bf16 and fp8 caches,
page sizes 16 to 512 (blocks of 32 rows then span up to three pages, or share one), ragged and
empty sequences, table entries outside the pool for pages past the length (clamped, never
read into the result), and the fused cache append writing the row's page.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.BF16: 2e-2, W.FP8: 5e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def dev_paged(gqa, p, layout="auto", num_splits=0, k_new=None, v_new=None, table=None):
    d = "cuda"
    ks = p.k_scale.to(d) if p.k_scale is not None else None
    vs = p.v_scale.to(d) if p.v_scale is not None else None
    kp, vp = p.k_pages.to(d), p.v_pages.to(d)
    bt = (p.block_table if table is None else table).to(d)
    _say(f"[gpu] paged {p.name} B{p.B} H{p.H} G{p.G} page{p.page_size} pps{p.pages_per_seq} pages{p.num_pages} "
         f"kv={p.kv_dtype} layout={layout} splits={num_splits} append={k_new is not None}")
    out = gqa.decode_paged(p.q.to(d), kp, vp, bt, p.seq_lens.to(d), scale=p.scale, k_scale=ks, v_scale=vs,
                           layout=layout, num_splits=num_splits,
                           k_new=None if k_new is None else k_new.to(d), v_new=None if v_new is None else v_new.to(d))
    torch.cuda.synchronize()
    return out, kp, vp


def check(got, want, tol, what):
    got = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want)))
    _say(f"    {what}: max abs err {err:.3e}")
    assert err <= tol, f"{what}: {err} > {tol}"


RUNS = [("auto", 0), ("uniform", 0), ("flat", 0), ("uniform", 1), ("uniform", 7)]

PAGED_CASES = [
    # B, H, G, seq_lens, T_cap, kv, page_size
    (1, 32, 8, [2048], 2048, W.BF16, 16),
    (2, 32, 8, [1000, 77], 1024, W.BF16, 32),
    (3, 16, 2, [1, 333, 1024], 1024, W.FP8, 16),
    (2, 32, 1, [2049, 700], 2100, W.FP8, 64),
    (5, 64, 1, [700, 0, 1, 333, 64], 700, W.BF16, 512),
    (20, 8, 2, [0 if i % 7 == 3 else (i * 41) % 300 + 1 for i in range(20)], 300, W.BF16, 16),
    (18, 32, 8, [(i * 97) % 1500 + 1 for i in range(18)], 1500, W.FP8, 128),
]


@pytest.mark.parametrize("B,H,G,lens,T_cap,kv,ps", PAGED_CASES)
def test_paged_cases(gqa, B, H, G, lens, T_cap, kv, ps):
    c = W.make_decode(B, H, G, 128, lens, T_cap=T_cap, kv_dtype=kv, seed=B + H + ps, name=f"pg_B{B}H{H}G{G}")
    p = W.make_paged(c, ps, seed=ps + 1)
    want = oracle.decode_paged(p)
    for layout, splits in RUNS:
        if layout == "flat" and B * G * p.T_cap >= 2 ** 31:
            continue
        try:
            out, _, _ = dev_paged(gqa, p, layout, splits)
        except gqa.GqaError as e:
            if e.status == 2 and layout == "flat":
                continue
            raise
        check(out, want, TOL[kv], f"{p.name} page{ps} layout={layout} splits={splits}")


def test_paged_out_of_pool_entries(gqa):
    """Table entries for pages past each sequence's length hold ids outside the pool: they
    are clamped (no fault) and, covering no valid row, do not change the result."""
    c = W.make_decode(3, 32, 8, 128, [100, 17, 300], T_cap=320, seed=5, name="pg_clamp")
    p = W.make_paged(c, 16, seed=9)
    bt = p.block_table.clone()
    for b, L in enumerate(c.seq_lens.tolist()):
        used = -(-L // 16)
        bt[b, used:] = torch.tensor([-7, 1 << 30] * 20, dtype=torch.int32)[:bt.shape[1] - used]
    want = oracle.decode_paged(p)
    for layout, splits in RUNS:
        out, _, _ = dev_paged(gqa, p, layout, splits, table=bt)
        check(out, want, TOL[W.BF16], f"clamped table layout={layout} splits={splits}")


@pytest.mark.parametrize("kv,ps", [(W.BF16, 16), (W.FP8, 32), (W.BF16, 256)])
def test_paged_append(gqa, kv, ps):
    """The cache append writes row L-1 in its page, byte-exact, and nothing else."""
    c = W.make_decode(4, 32, 8, 128, [1, 500, 257, 0], T_cap=512, kv_dtype=kv, seed=ps, name="pg_app")
    p = W.make_paged(c, ps, seed=3)
    g = torch.Generator().manual_seed(ps)
    kn = torch.randn(4, 8, 128, generator=g).to(torch.bfloat16)
    vn = torch.randn(4, 8, 128, generator=g).to(torch.bfloat16)
    logical = oracle.contiguous_case(p)
    kc_want, vc_want = oracle.append(logical, kn, vn)
    appended = W.DecodeCase(name="pg_app", q=p.q, k_cache=kc_want, v_cache=vc_want, seq_lens=p.seq_lens,
                            scale=p.scale, q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, k_scale=p.k_scale,
                            v_scale=p.v_scale)
    want = oracle.decode(appended)
    for layout, splits in [("auto", 0), ("uniform", 3), ("flat", 0)]:
        out, kp, vp = dev_paged(gqa, p, layout, splits, k_new=kn, v_new=vn)
        check(out, want, TOL[kv], f"append page{ps} layout={layout} splits={splits}")
        got = W.PagedDecodeCase(**{**p.__dict__, "k_pages": kp.cpu(), "v_pages": vp.cpu()})
        kg, vg = oracle.paged_kv(got)
        for a, b, n in ((kg, kc_want, "K"), (vg, vc_want, "V")):
            ab = a.contiguous().view(torch.uint8)[:, :, :b.shape[2]]
            assert torch.equal(ab, b.contiguous().view(torch.uint8)), f"{n} logical cache differs"
        # spare pages (in no table row) are untouched
        used = set(p.block_table.flatten().tolist())
        spare = [i for i in range(p.num_pages) if i not in used]
        assert torch.equal(kp.cpu()[spare].view(torch.uint8), p.k_pages[spare].view(torch.uint8))


PREFILL_PAGED_CASES = [
    # B, H, G, Tq, lens, T_cap, kv dtype, causal, page size
    (3, 32, 8, 100, [1000, 64, 0], 1024, W.BF16, True, 16),
    (2, 32, 8, 70, [500, 300], 512, W.BF16, False, 64),
    (2, 32, 8, 33, [700, 33], 720, W.FP8, True, 32),
    (1, 28, 4, 129, [900], 960, W.BF16, True, 16),     # R = 7
    (2, 8, 8, 50, [40, 200], 256, W.FP8, False, 128),  # MHA, a chunk longer than one sequence
]


@pytest.mark.parametrize("B,H,G,Tq,lens,T_cap,kvd,causal,ps", PREFILL_PAGED_CASES)
def test_prefill_paged(gqa, B, H, G, Tq, lens, T_cap, kvd, causal, ps):
    """A chunk against shuffled pages vs the oracle, and bit for bit vs the same chunk against
    the contiguous cache (the same rows through the same arithmetic)."""
    c = W.make_chunk(B, H, G, 128, Tq, lens, T_cap=T_cap, causal=causal, seed=Tq + ps, name="pchunk", kv_dtype=kvd)
    p = W.make_paged_chunk(c, ps, seed=ps + 1)
    d = "cuda"
    ks = c.k_scale.to(d) if c.k_scale is not None else None
    vs = c.v_scale.to(d) if c.v_scale is not None else None
    _say(f"[gpu] prefill_paged B{B} H{H} G{G} Tq{Tq} lens={lens} kv={kvd} causal={causal} page{ps}")
    got = gqa.prefill_paged(p.q.to(d), p.k_pages.to(d), p.v_pages.to(d), p.block_table.to(d), p.seq_lens.to(d),
                            scale=p.scale, causal=causal, k_scale=ks, v_scale=vs)
    flat = gqa.prefill_cached(c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d), scale=c.scale,
                              causal=causal, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    check(got, oracle.prefill_paged(p), 5e-2 if kvd == W.FP8 else 2e-2, "prefill_paged")
    assert torch.equal(got.cpu(), flat.cpu()), "paged and contiguous chunks differ"


@pytest.mark.parametrize("kvd", [W.BF16, W.FP8])
def test_prefill_paged_out_of_pool_entries(gqa, kvd):
    """Chunked prefill: table entries for pages past each sequence's length hold ids outside
    the pool (clamped, no fault) and do not change the result."""
    c = W.make_chunk(3, 32, 8, 128, 40, [300, 40, 0], T_cap=320, causal=True, seed=61, name="pchunk_clamp",
                     kv_dtype=kvd)
    p = W.make_paged_chunk(c, 16, seed=62)
    bt = p.block_table.clone()
    for b, L in enumerate(c.seq_lens.tolist()):
        used = -(-L // 16)
        bt[b, used:] = torch.tensor([-7, 1 << 30] * 20, dtype=torch.int32)[:bt.shape[1] - used]
    d = "cuda"
    ks = c.k_scale.to(d) if c.k_scale is not None else None
    vs = c.v_scale.to(d) if c.v_scale is not None else None
    _say(f"[gpu] prefill_paged out-of-pool table entries kv={kvd}")
    got = gqa.prefill_paged(p.q.to(d), p.k_pages.to(d), p.v_pages.to(d), bt.to(d), p.seq_lens.to(d),
                            scale=p.scale, causal=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    check(got, oracle.prefill_paged(p), TOL[kvd], f"prefill_paged clamped table kv={kvd}")
