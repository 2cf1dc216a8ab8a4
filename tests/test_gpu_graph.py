"""Graph capture of the C-ABI calls (needs a gfx950 GPU).

Decode (vector-ALU and matrix-core paths, split key ranges, both work layouts, merges in a
second kernel or inside the decode kernel) and prefill are captured into a HIP graph on a side
stream; the graph is replayed several times with unrelated eager work and synchronisations in
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
