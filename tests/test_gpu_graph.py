"""Graph capture of the C-ABI calls (needs a gfx950 GPU).

Decode (vector-ALU and matrix-core paths, split key ranges, both work layouts, merges in a
second kernel or inside the decode kernel), the paged decode, the decode with its cache
append, prefill and the chunked prefill against an fp8 cache, contiguous or paged, are
captured into a HIP graph on a side stream; the graph is replayed several times with unrelated eager work and synchronisations in
between, and every replay must reproduce the eager result bit for bit: partial results are
merged in a fixed order (the only atomics are integer arrival counters), and every replay
reuses one workspace, so the counters must be back at zero after each call.
"""

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available()
    g.library()
    return g


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("path,splits,layout", [("valu", 8, "auto"), ("mfma", 8, "auto"), ("valu", 1, "auto"),
                                                ("mfma", 0, "uniform"), ("mfma", 0, "flat")])
def test_decode_graph_replays(gqa, path, splits, layout):
    d = "cuda"
    c = W.make_decode(3, 32, 8, 128, [700, 1500, 0], T_cap=1536, seed=31, name="graph")
    q, kc, vc, sl = c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d)
    ws = torch.zeros(max(1, gqa.decode_workspace_size(c.B, c.H, c.G, c.D, c.T_cap, c.kv_dtype, splits)),
                     dtype=torch.uint8, device=d)
    ref = gqa.decode(q, kc, vc, sl, scale=c.scale, num_splits=splits, path=path, workspace=ws, layout=layout)
    torch.cuda.synchronize()
    ref = ref.clone()
    out = torch.empty_like(q)
    g = _capture(lambda: gqa.decode(q, kc, vc, sl, out=out, scale=c.scale, num_splits=splits, path=path,
                                    workspace=ws, layout=layout))
    other = W.make_decode(1, 16, 2, 128, [300], T_cap=320, seed=32, name="other")
    oq, ok, ov, osl = other.q.to(d), other.k_cache.to(d), other.v_cache.to(d), other.seq_lens.to(d)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"
        gqa.decode(oq, ok, ov, osl, scale=other.scale)   # unrelated eager work in between
        torch.cuda.synchronize()


def test_prefill_graph_replays(gqa):
    d = "cuda"
    c = W.make_prefill(1, 8, 2, 128, 333, seed=33, name="graph_prefill")
    q, k, v = c.q.to(d), c.k.to(d), c.v.to(d)
    ref = gqa.prefill(q, k, v, scale=c.scale, causal=True).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    g = _capture(lambda: gqa.prefill(q, k, v, out=out, scale=c.scale, causal=True))
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"
        gqa.prefill(q[:, :, :100].contiguous(), k[:, :, :100].contiguous(), v[:, :, :100].contiguous(),
                    scale=c.scale, causal=False)
        torch.cuda.synchronize()


def _other_calls(gqa, name):
    """(eager call writing `out`, out) for the paged decode, the decode with its cache append,
    and the chunked prefill against an fp8 cache and against pages."""
    d = "cuda"
    if name in ("paged_decode_fp8", "decode_append"):
        kvd = W.FP8 if name == "paged_decode_fp8" else W.BF16
        c = W.make_decode(3, 32, 8, 128, [700, 1500, 1], T_cap=1536, seed=34, name=name, kv_dtype=kvd)
        ks = c.k_scale.to(d) if c.k_scale is not None else None
        vs = c.v_scale.to(d) if c.v_scale is not None else None
        ws = torch.zeros(max(1, gqa.decode_workspace_size(c.B, c.H, c.G, c.D, c.T_cap, c.kv_dtype)),
                         dtype=torch.uint8, device=d)
        out = torch.empty_like(c.q, device=d)
        if name == "paged_decode_fp8":
            p = W.make_paged(c, 16, seed=35)
            args = [t.to(d) for t in (p.q, p.k_pages, p.v_pages, p.block_table, p.seq_lens)]
            return (lambda: gqa.decode_paged(*args, out=out, scale=p.scale, k_scale=ks, v_scale=vs,
                                             workspace=ws)), out
        # The append writes the same row at seq_lens - 1 on every call, so replays are idempotent.
        g = torch.Generator().manual_seed(36)
        kn = torch.randn(c.B, c.G, c.D, generator=g).to(torch.bfloat16).to(d)
        vn = torch.randn(c.B, c.G, c.D, generator=g).to(torch.bfloat16).to(d)
        args = [t.to(d) for t in (c.q, c.k_cache, c.v_cache, c.seq_lens)]
        return (lambda: gqa.decode(*args, out=out, scale=c.scale, workspace=ws, k_new=kn, v_new=vn)), out
    kvd = W.FP8
    c = W.make_chunk(2, 32, 8, 128, 96, [900, 200], T_cap=1024, seed=37, name=name, kv_dtype=kvd)
    ks, vs = c.k_scale.to(d), c.v_scale.to(d)
    out = torch.empty_like(c.q, device=d)
    if name == "chunk_fp8":
        args = [t.to(d) for t in (c.q, c.k_cache, c.v_cache, c.seq_lens)]
        return (lambda: gqa.prefill_cached(*args, out=out, scale=c.scale, causal=True, k_scale=ks,
                                           v_scale=vs)), out
    p = W.make_paged_chunk(c, 32, seed=38)
    args = [t.to(d) for t in (p.q, p.k_pages, p.v_pages, p.block_table, p.seq_lens)]
    return (lambda: gqa.prefill_paged(*args, out=out, scale=p.scale, causal=True, k_scale=ks, v_scale=vs)), out


@pytest.mark.parametrize("name", ["paged_decode_fp8", "decode_append", "chunk_fp8", "chunk_paged_fp8"])
def test_other_calls_graph_replays(gqa, name):
    call, out = _other_calls(gqa, name)
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(call)
    other = W.make_decode(1, 16, 2, 128, [300], T_cap=320, seed=39, name="other")
    oq, ok, ov, osl = (t.to("cuda") for t in (other.q, other.k_cache, other.v_cache, other.seq_lens))
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}: replay {rep} differs from the eager result"
        gqa.decode(oq, ok, ov, osl, scale=other.scale)   # unrelated eager work in between
        torch.cuda.synchronize()
