"""gqa_decode_noalloc (split partials in the library's static device scratch) against
gqa_decode (caller workspace) on the same inputs, through the C ABI. Several calls in a row
share the one scratch array, later ones with smaller inputs; each must equal gqa_decode's
output bit for bit (same kernels, same split plan) and the oracle within the bf16 / fp8
tolerances."""

import ctypes
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


def _call(gqa, fn, case, dev, workspace=None):
    q, k, v, lens, ks, vs = dev
    out = torch.full_like(q, float("nan"))
    o = gqa.new_opts(q_dtype=1, kv_dtype={W.BF16: 1, W.FP8: 2}[case.kv_dtype], kv_capacity=case.T_cap)
    if ks is not None:
        o.k_scale, o.v_scale = ks.data_ptr(), vs.data_ptr()
    if workspace is not None:
        o.workspace, o.workspace_bytes = workspace.data_ptr(), workspace.numel()
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), out.data_ptr(), case.B, case.H, case.G,
            case.D, float(case.scale), int(torch.cuda.current_stream().cuda_stream), ctypes.byref(o))
    torch.cuda.synchronize()
    assert st == 0, gqa.status_string(st)
    return out


def test_noalloc_matches_decode_over_successive_calls(gqa):
    lib = gqa.library()
    cases = [
        W.llama70b_ragged_decode(0),   # flat layout, in-kernel merge, 7 MB of partials
        W.mqa_fp8_long_decode(0),      # uniform layout, combine kernel, fp8 cache
        W.llama7b_gqa8_decode(0),      # smaller: 16 ranges merged in-kernel
        W.make_decode(3, 16, 4, 128, [900, 1, 333], T_cap=900, seed=61, name="small_ragged"),  # smaller still
    ]
    for case in cases:
        s = gqa.decode_num_splits(case.B, case.H, case.G, case.D, case.T_cap, case.kv_dtype)
        _say(f"[gpu] gqa_decode_noalloc vs gqa_decode: {case.name} B{case.B} H{case.H} G{case.G} "
             f"T_cap{case.T_cap} splits={s}")
        d = "cuda"
        dev = (case.q.to(d), case.k_cache.to(d), case.v_cache.to(d), case.seq_lens.to(d),
               case.k_scale.to(d) if case.k_scale is not None else None,
               case.v_scale.to(d) if case.v_scale is not None else None)
        need = gqa.decode_workspace_size(case.B, case.H, case.G, case.D, case.T_cap, case.kv_dtype)
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=d)
        ref = _call(gqa, lib.gqa_decode, case, dev, ws)
        for rep in range(2):
            got = _call(gqa, lib.gqa_decode_noalloc, case, dev)
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{case.name} call {rep}: not bit-equal"
        err = float(np.max(np.abs(got.cpu().double().numpy() - oracle.decode(case))))
        _say(f"    bit-equal to gqa_decode; max abs err vs oracle {err:.3e}")
        assert err <= TOL[case.kv_dtype]


def test_noalloc_binding(gqa):
    case = W.make_decode(2, 32, 8, 128, [1500, 700], T_cap=1536, seed=62, name="noalloc_binding")
    d = "cuda"
    q, k, v, lens = case.q.to(d), case.k_cache.to(d), case.v_cache.to(d), case.seq_lens.to(d)
    out = torch.empty_like(q)
    _say("[gpu] decode_noalloc binding")
    gqa.decode_noalloc(q, k, v, lens, out, scale=case.scale)
    ref = gqa.decode(q, k, v, lens, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
