"""Seeded random shapes vs the oracle, through the C ABI (needs a gfx950 GPU).

Each case draws its configuration from a fixed seed: decode (contiguous or paged, with or
without the fused cache append, forced or automatic splits, uniform or flat layout), prefill
and chunked prefill (contiguous or paged cache); head dims 64 to 128, 1 to 64 query heads per KV head, ragged lengths
with empty sequences, lengths past the capacity and rows of NaN beyond each length; bf16,
fp32, fp8 and INT4 caches. Every combination drawn is a supported one (the flat layout only
where the matrix-core family runs), and every result must match the oracle within the
tolerance of its cache type.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-5, W.BF16: 2e-2, W.FP8: 5e-2, W.INT4: 5e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def _check(got, want, tol, what):
    got = got.detach().cpu().to(torch.float64).numpy()
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want)))
    _say(f"    max abs err {err:.3e}")
    assert err <= tol, f"{what}: {err} > {tol}"


def _heads(rng, max_h=64):
    G = int(rng.choice([1, 2, 4, 8]))
    R = int(rng.choice([r for r in (1, 2, 3, 4, 8, 16, 32, 64) if G * r <= max_h]))
    return G * R, G


def _lens(rng, B, T_cap):
    lens = [int(rng.integers(0, T_cap + 1)) for _ in range(B)]
    if B > 1:
        lens[int(rng.integers(0, B))] = T_cap            # a full cache
    if B > 2 and rng.random() < 0.5:
        lens[int(rng.integers(0, B))] = 0                # an empty sequence
    return lens


def decode_case(i):
    rng = np.random.default_rng(1000 + i)
    kvd = str(rng.choice([W.BF16, W.BF16, W.FP8, W.INT4, W.F32]))
    D = 128 if rng.random() < 0.7 else int(rng.choice([64, 80, 96]))
    H, G = _heads(rng)
    B = int(rng.integers(1, 7))
    T_cap = int(rng.integers(1, 3001))
    lens = _lens(rng, B, T_cap)
    qd = W.F32 if kvd == W.F32 else W.BF16
    c = W.make_decode(B, H, G, D, lens, T_cap=T_cap, q_dtype=qd, kv_dtype=kvd, seed=i, name=f"rand{i}")
    layout = str(rng.choice(["auto", "uniform", "flat"]))
    splits = 0 if layout == "flat" else int(rng.choice([0, 0, 1, 3, 7]))
    paged = kvd != W.F32 and D == 128 and rng.random() < 0.3
    append = not paged and kvd != W.F32 and rng.random() < 0.3
    page = int(rng.choice([16, 32, 64]))
    if layout == "flat" and (D != 128 or kvd == W.F32):
        layout = "auto"  # the flat layout belongs to the matrix-core family (D = 128, bf16 q)
    return c, layout, splits, paged, append, page


@pytest.mark.parametrize("i", range(96))
def test_random_decode(gqa, i):
    c, layout, splits, paged, append, page = decode_case(i)
    d = "cuda"
    _say(f"[gpu] random decode {i}: B{c.B} H{c.H} G{c.G} D{c.D} T_cap{c.T_cap} lens={c.seq_lens.tolist()} "
         f"kv={c.kv_dtype} layout={layout} splits={splits} paged={paged and page} append={append}")
    ks = c.k_scale.to(d) if c.k_scale is not None else None
    vs = c.v_scale.to(d) if c.v_scale is not None else None
    try:
        if paged:
            p = W.make_paged(c, page, seed=i)
            want = oracle.decode_paged(p)
            out = gqa.decode_paged(p.q.to(d), p.k_pages.to(d), p.v_pages.to(d), p.block_table.to(d),
                                   p.seq_lens.to(d), scale=p.scale, k_scale=ks, v_scale=vs, layout=layout,
                                   num_splits=splits)
        elif append:
            g = torch.Generator().manual_seed(i)
            kn = torch.randn(c.B, c.G, c.D, generator=g).to(c.q.dtype)
            vn = torch.randn(c.B, c.G, c.D, generator=g).to(c.q.dtype)
            kc, vc = oracle.append(c, kn, vn)
            want = oracle.decode(W.DecodeCase(**{**c.__dict__, "k_cache": kc, "v_cache": vc}))
            out = gqa.decode(c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d), scale=c.scale,
                             k_scale=ks, v_scale=vs, layout=layout, num_splits=splits, k_new=kn.to(d),
                             v_new=vn.to(d))
        else:
            want = oracle.decode(c)
            out = gqa.decode(c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d), scale=c.scale,
                             k_scale=ks, v_scale=vs, layout=layout, num_splits=splits)
        torch.cuda.synchronize()
    except gqa.GqaError as e:
        # every combination drawn here is one the library documents as supported
        raise AssertionError(f"random decode {i}: {e} (status {e.status})") from e
    _check(out, want, TOL[c.kv_dtype], f"random decode {i}")


@pytest.mark.parametrize("i", range(24))
def test_random_prefill(gqa, i):
    rng = np.random.default_rng(2000 + i)
    dt = str(rng.choice([W.BF16, W.BF16, W.F32]))
    D = 128 if rng.random() < 0.7 else int(rng.choice([64, 96]))
    H, G = _heads(rng, max_h=32)
    B = int(rng.integers(1, 3))
    T = int(rng.integers(1, 301))
    causal = bool(rng.random() < 0.7)
    c = W.make_prefill(B, H, G, D, T, dtype=dt, causal=causal, seed=i, name=f"randp{i}")
    d = "cuda"
    _say(f"[gpu] random prefill {i}: B{B} H{H} G{G} D{D} T{T} causal={causal} dtype={dt}")
    out = gqa.prefill(c.q.to(d), c.k.to(d), c.v.to(d), scale=c.scale, causal=causal)
    torch.cuda.synchronize()
    _check(out, oracle.prefill(c), TOL[dt], f"random prefill {i}")


@pytest.mark.parametrize("i", range(24))
def test_random_chunk(gqa, i):
    rng = np.random.default_rng(3000 + i)
    D = 128 if rng.random() < 0.7 else 64
    H, G = _heads(rng, max_h=32)
    B = int(rng.integers(1, 4))
    T_cap = int(rng.integers(1, 1501))
    Tq = int(rng.integers(1, 101))
    lens = _lens(rng, B, T_cap)
    causal = bool(rng.random() < 0.7)
    kvd = W.FP8 if rng.random() < 0.25 else W.BF16
    paged = D == 128 and rng.random() < 0.3
    page = int(rng.choice([16, 32, 64]))
    c = W.make_chunk(B, H, G, D, Tq, lens, T_cap=T_cap, causal=causal, seed=i, name=f"randc{i}", kv_dtype=kvd)
    d = "cuda"
    _say(f"[gpu] random chunk {i}: B{B} H{H} G{G} D{D} Tq{Tq} T_cap{T_cap} lens={lens} causal={causal} kv={kvd} "
         f"paged={paged and page}")
    ks = c.k_scale.to(d) if c.k_scale is not None else None
    vs = c.v_scale.to(d) if c.v_scale is not None else None
    if paged:
        p = W.make_paged_chunk(c, page, seed=i)
        out = gqa.prefill_paged(p.q.to(d), p.k_pages.to(d), p.v_pages.to(d), p.block_table.to(d),
                                p.seq_lens.to(d), scale=p.scale, causal=causal, k_scale=ks, v_scale=vs)
    else:
        out = gqa.prefill_cached(c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d), scale=c.scale,
                                 causal=causal, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    _check(out, oracle.prefill_cached(c), TOL[kvd], f"random chunk {i}")
