"""Prefill of a query chunk against a cache vs the oracle, through the C ABI (needs a gfx950 GPU).

Cache rows at or beyond each sequence's length are NaN, so a kernel that reads past the
length fails. Covered: causal and not, the matrix-core and generic families, chunks longer
than the cache holds (leading zero rows), a chunk that is the whole sequence (= plain
prefill), MHA and MQA groupings, fp32 caches (generic) and fp8 caches (matrix cores and
generic), the 12-dim toy's last two tokens, and a prefill split into chunks that reproduces
the one-shot prefill.
"""

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


def dev_chunk(gqa, c, path="auto"):
    d = "cuda"
    ks = c.k_scale.to(d) if c.k_scale is not None else None
    vs = c.v_scale.to(d) if c.v_scale is not None else None
    _say(f"[gpu] chunk {c.name} B{c.B} H{c.H} G{c.G} D{c.D} Tq{c.Tq} T_cap{c.T_cap} lens={c.seq_lens.tolist()} "
         f"causal={c.causal} q={c.dtype} kv={c.kv_dtype} path={path}")
    out = gqa.prefill_cached(c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d), scale=c.scale,
                             causal=c.causal, k_scale=ks, v_scale=vs, path=path)
    torch.cuda.synchronize()
    return out


def check(got, want, tol, what):
    got = got.detach().cpu().to(torch.float64).numpy()
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want)))
    _say(f"    {what}: max abs err {err:.3e}")
    assert err <= tol, f"{what}: {err} > {tol}"


CHUNK_CASES = [
    # B, H, G, D, Tq, lens, T_cap, q dtype, kv dtype, causal
    (2, 32, 8, 128, 200, [1000, 300], 1024, W.BF16, W.BF16, True),
    (2, 32, 8, 128, 200, [1000, 300], 1024, W.BF16, W.BF16, False),
    (1, 8, 1, 128, 64, [64], 64, W.BF16, W.BF16, True),            # the whole sequence: plain prefill
    (3, 16, 2, 128, 100, [50, 100, 2000], 2048, W.BF16, W.BF16, True),  # 50 < Tq: leading zero rows
    (2, 8, 8, 128, 70, [500, 70], 512, W.BF16, W.BF16, True),      # MHA
    (1, 64, 1, 128, 33, [700], 800, W.BF16, W.BF16, True),         # MQA, R = 64
    (2, 6, 3, 80, 9, [40, 3], 41, W.F32, W.F32, True),             # fp32, odd head dim (generic)
    (2, 32, 8, 128, 33, [300, 40], 300, W.BF16, W.FP8, True),      # fp8 cache
    (2, 32, 8, 128, 100, [1000, 64], 1024, W.BF16, W.FP8, False),  # fp8, not causal
    (3, 8, 8, 128, 70, [500, 70, 0], 512, W.BF16, W.FP8, True),    # fp8 MHA, an empty sequence
    (1, 28, 4, 128, 129, [777], 800, W.BF16, W.FP8, True),         # fp8, R = 7
    (2, 28, 4, 128, 50, [600, 50], 640, W.BF16, W.BF16, True),      # R = 7
    (1, 40, 8, 128, 33, [400], 400, W.BF16, W.BF16, False),        # R = 5, not causal
]


@pytest.mark.parametrize("B,H,G,D,Tq,lens,T_cap,qd,kvd,causal", CHUNK_CASES)
def test_chunk_cases(gqa, B, H, G, D, Tq, lens, T_cap, qd, kvd, causal):
    c = W.make_chunk(B, H, G, D, Tq, lens, T_cap=T_cap, dtype=qd, kv_dtype=kvd, causal=causal, seed=Tq + D + B,
                     name=f"chunk_B{B}H{H}G{G}D{D}Tq{Tq}")
    want = oracle.prefill_cached(c)
    for path in ("auto", "generic"):
        check(dev_chunk(gqa, c, path), want, TOL[kvd], f"{c.name} causal={causal} path={path}")


def test_toy_last_two_tokens(gqa):
    """The 12-dim, 4-head toy: its last two tokens as one chunk against the 7-token cache."""
    q, k, v = W.toy_tokens(0)
    c = W.ChunkCase(name="toy_chunk", q=q[:, :, 5:7].contiguous(), k_cache=k, v_cache=v,
                    seq_lens=torch.tensor([7], dtype=torch.int32), scale=1.0 / 3 ** 0.5, causal=True, dtype=W.F32,
                    kv_dtype=W.F32)
    check(dev_chunk(gqa, c), oracle.prefill_cached(c), TOL[W.F32], "toy chunk")


def test_chunks_compose_prefill(gqa):
    """A causal prefill of 600 tokens computed as chunks [0,128), [128,400), [400,600) against
    the growing cache matches the oracle's one-shot prefill."""
    B, H, G, D, T = 2, 32, 8, 128, 600
    p = W.make_prefill(B, H, G, D, T, seed=31, name="compose")
    want = oracle.prefill(p)
    d = "cuda"
    kc = torch.full((B, G, 640, D), float("nan"), dtype=torch.bfloat16, device=d)
    vc = torch.full((B, G, 640, D), float("nan"), dtype=torch.bfloat16, device=d)
    for s, e in ((0, 128), (128, 400), (400, 600)):
        kc[:, :, s:e] = p.k[:, :, s:e].to(d)
        vc[:, :, s:e] = p.v[:, :, s:e].to(d)
        lens = torch.full((B,), e, dtype=torch.int32, device=d)
        out = gqa.prefill_cached(p.q[:, :, s:e].contiguous().to(d), kc, vc, lens, scale=p.scale)
        torch.cuda.synchronize()
        check(out, want[:, :, s:e], TOL[W.BF16], f"chunk [{s},{e})")
