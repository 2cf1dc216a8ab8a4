"""The C ABI's own memory and stream handling on the GPU, and the binding's argument checks.

* gqa_decode called through ctypes with opts.workspace = NULL on cases that split the cache:
  the call takes stream-ordered memory, zero-fills its arrival counters with a kernel, and
  must still match the oracle (in-kernel merge and separate combine kernel alike).
* A NULL workspace while the stream is captured into a graph is refused (GQA_ERR_WORKSPACE)
  before anything is enqueued.
* The binding on a stream that is not the current one: its temporary workspace and its
  output are created on that stream.
* The binding's argument checks (out of the wrong dtype, shape or device, a workspace that is
  too small, tensors on another device): ValueError, and no kernel is launched.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.BF16: 2e-2, W.FP8: 5e-2}
WSP = 3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def _err(got, want):
    return float(np.max(np.abs(got.detach().cpu().double().numpy() - want)))


def _dev(case):
    d = "cuda"
    ks = case.k_scale.to(d) if case.k_scale is not None else None
    vs = case.v_scale.to(d) if case.v_scale is not None else None
    return case.q.to(d), case.k_cache.to(d), case.v_cache.to(d), case.seq_lens.to(d), ks, vs


def _abi_decode_null_workspace(gqa, case, stream):
    q, k, v, lens, ks, vs = _dev(case)
    out = torch.full_like(q, float("nan"))
    o = gqa.new_opts(q_dtype=gqa.DTYPES["bf16"], kv_dtype={W.BF16: 1, W.FP8: 2}[case.kv_dtype],
                     kv_capacity=case.T_cap)
    if ks is not None:
        o.k_scale, o.v_scale = ks.data_ptr(), vs.data_ptr()
    assert not o.workspace
    torch.cuda.synchronize()
    st = gqa.library().gqa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), out.data_ptr(),
                                  case.B, case.H, case.G, case.D, float(case.scale), int(stream.cuda_stream),
                                  ctypes.byref(o))
    torch.cuda.synchronize()
    return st, out


@pytest.mark.parametrize("which", ["fused_merge", "combine_kernel", "flat_ragged"])
def test_abi_null_workspace(gqa, which):
    if which == "fused_merge":      # B1 H32 G8 L2048: 16 ranges merged inside the decode kernel
        case = W.llama7b_gqa8_decode(0)
    elif which == "combine_kernel":  # MQA with 32 heads per KV head: partials too big to merge in-kernel
        case = W.make_decode(2, 32, 1, 128, [6000, 2500], T_cap=6000, kv_dtype=W.FP8, seed=31, name="mqa_null_ws")
    else:                            # 20 ragged sequences: the flat layout with its merge
        lens = [(i * 397) % 1500 + 1 for i in range(20)]
        case = W.make_decode(20, 64, 8, 128, lens, T_cap=1536, seed=32, name="flat_null_ws")
    s = gqa.decode_num_splits(case.B, case.H, case.G, case.D, case.T_cap, case.kv_dtype)
    assert s > 1, "the case must split its cache"
    _say(f"[gpu] gqa_decode via ctypes, NULL workspace, {case.name} splits={s}")
    stream = torch.cuda.Stream()
    for rep in range(2):  # twice: fresh counters each call
        st, out = _abi_decode_null_workspace(gqa, case, stream)
        assert st == 0, gqa.status_string(st)
        err = _err(out, oracle.decode(case))
        _say(f"    call {rep}: max abs err {err:.3e}")
        assert err <= TOL[case.kv_dtype]


def test_abi_null_workspace_refused_under_capture(gqa):
    case = W.llama7b_gqa8_decode(0)
    q, k, v, lens, _, _ = _dev(case)
    out = torch.empty_like(q)
    o = gqa.new_opts(kv_capacity=case.T_cap)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    _say("[gpu] NULL workspace under graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            st = gqa.library().gqa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), out.data_ptr(),
                                          case.B, case.H, case.G, case.D, float(case.scale),
                                          int(stream.cuda_stream), ctypes.byref(o))
    torch.cuda.synchronize()
    del g
    assert st == WSP, gqa.status_string(st)


@pytest.mark.parametrize("kind", ["decode", "decode_fp8", "prefill", "chunk"])
def test_binding_on_a_stream_that_is_not_current(gqa, kind):
    """No workspace and no out given: both are made on `stream`, which is never made current."""
    stream = torch.cuda.Stream()
    assert stream != torch.cuda.current_stream()
    _say(f"[gpu] binding on a side stream: {kind}")
    if kind.startswith("decode"):
        case = (W.llama7b_gqa8_decode(0) if kind == "decode" else
                W.make_decode(3, 32, 1, 128, [5000, 17, 3000], T_cap=5000, kv_dtype=W.FP8, seed=41, name="fp8"))
        q, k, v, lens, ks, vs = _dev(case)
        want = oracle.decode(case)
        torch.cuda.synchronize()
        out = gqa.decode(q, k, v, lens, scale=case.scale, k_scale=ks, v_scale=vs, stream=stream)
    elif kind == "prefill":
        case = W.make_prefill(2, 16, 4, 128, 300, seed=42, name="side_prefill")
        want = oracle.prefill(case)
        q, k, v = case.q.cuda(), case.k.cuda(), case.v.cuda()
        torch.cuda.synchronize()
        out = gqa.prefill(q, k, v, scale=case.scale, causal=True, stream=stream)
    else:
        case = W.make_chunk(2, 32, 8, 128, 48, [700, 60], T_cap=704, seed=43, name="side_chunk")
        want = oracle.prefill_cached(case)
        q, k, v, lens = case.q.cuda(), case.k_cache.cuda(), case.v_cache.cuda(), case.seq_lens.cuda()
        torch.cuda.synchronize()
        out = gqa.prefill_cached(q, k, v, lens, scale=case.scale, stream=stream)
    stream.synchronize()
    err = _err(out, want)
    _say(f"    max abs err {err:.3e}")
    assert err <= TOL[W.FP8 if kind == "decode_fp8" else W.BF16]


def test_binding_rejects_bad_arguments(gqa):
    """Every case is refused in Python before the library is called (no kernel runs)."""
    case = W.make_decode(2, 16, 4, 128, [300, 20], T_cap=320, seed=51, name="bad_args")
    q, k, v, lens, _, _ = _dev(case)
    need = gqa.decode_workspace_size(case.B, case.H, case.G, case.D, case.T_cap, case.kv_dtype)
    assert need > 0
    _say("[gpu] binding argument checks (no launches)")
    bad = [
        dict(out=torch.empty(2, 16, 128, dtype=torch.float32, device="cuda")),   # wrong dtype
        dict(out=torch.empty(2, 16, 64, dtype=torch.bfloat16, device="cuda")),   # too small
        dict(out=torch.empty(2, 8, 128, dtype=torch.bfloat16, device="cuda")),   # wrong shape
        dict(out=torch.empty(2, 16, 128, dtype=torch.bfloat16)),                 # on the host
        dict(out=q),                                                             # aliases q
        dict(workspace=torch.zeros(need - 1, dtype=torch.uint8, device="cuda")),  # too small
        dict(workspace=torch.zeros(need, dtype=torch.uint8)),                    # on the host
        dict(path="matrix"), dict(layout="diagonal"),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            gqa.decode(q, k, v, lens, **kw)
    with pytest.raises(ValueError):
        gqa.decode(q, k, v, lens.cpu())
    fc = W.make_decode(2, 16, 4, 128, [300, 20], T_cap=320, kv_dtype=W.FP8, seed=52, name="bad_scales")
    fq, fk, fv, fl, fks, fvs = _dev(fc)
    with pytest.raises(ValueError):
        gqa.decode(fq, fk, fv, fl, k_scale=fks.cpu(), v_scale=fvs)
    with pytest.raises(ValueError):
        gqa.decode(fq, fk, fv, fl, k_scale=fks[:1], v_scale=fvs)
    pc = W.make_prefill(1, 8, 2, 128, 40, seed=53, name="bad_prefill")
    pq, pk, pv = pc.q.cuda(), pc.k.cuda(), pc.v.cuda()
    for kw in (dict(out=torch.empty(1, 8, 40, 128, dtype=torch.float32, device="cuda")),
               dict(out=torch.empty(1, 8, 39, 128, dtype=torch.bfloat16, device="cuda"))):
        with pytest.raises(ValueError):
            gqa.prefill(pq, pk, pv, **kw)
    torch.cuda.synchronize()
