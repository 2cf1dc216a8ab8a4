"""Decode with scores that climb or fall along the cache, vs the oracle, through the C ABI
(needs a gfx950 GPU).

The decode softmax keeps a reference maximum that moves only when a head's block maximum
outgrows it by a margin, so random N(0, 1) data rarely moves it after the first block. Here
q = u (entries +-1) and K row t = a_t u, so the base-2 scaled score of key t is
slope * t: slopes below the margin per 32-key block (the reference lags and probabilities
grow up to the margin), above it (it moves on every block), and negative (the first block
holds the maximum and later probabilities underflow). bf16, fp8 and INT4 caches, 4 and 32
query heads per KV head, one long key range and the automatic split.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.BF16: 2e-2, W.FP8: 5e-2, W.INT4: 5e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    return g


def ramp_case(B, H, G, lens, T_cap, kv_dtype, slope, seed):
    D = 128
    g = torch.Generator().manual_seed(seed)
    u = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.float32)
    # score_t (base 2) = (q . k_t) / sqrt(D) * log2(e) = sqrt(D) * a_t * log2(e) = slope * t
    a = slope * torch.arange(T_cap, dtype=torch.float32) / (math.sqrt(D) * math.log2(math.e))
    k = a[None, None, :, None] * u + 0.02 * torch.randn(B, G, T_cap, D, generator=g)
    v = torch.randn(B, G, T_cap, D, generator=g)
    # heads of a group climb at different rates (0.5x to 1.5x)
    q = torch.stack([u * (0.5 + h / max(H - 1, 1)) for h in range(H)])[None].expand(B, H, D).contiguous()
    lens_t = torch.tensor(lens, dtype=torch.int32)
    k_scale = v_scale = None
    if kv_dtype == W.FP8:
        k_st, k_scale = W.quantize_fp8_slabs(k, lens_t)
        v_st, v_scale = W.quantize_fp8_slabs(v, lens_t)
    elif kv_dtype == W.INT4:
        k_st, k_scale = W.quantize_int4_slabs(k, lens_t)
        v_st, v_scale = W.quantize_int4_slabs(v, lens_t)
    else:
        for b in range(B):
            k[b, :, lens[b]:] = float("nan")
            v[b, :, lens[b]:] = float("nan")
        k_st, v_st = k.to(torch.bfloat16), v.to(torch.bfloat16)
    return W.DecodeCase(name=f"ramp{slope}", q=q.to(torch.bfloat16), k_cache=k_st, v_cache=v_st, seq_lens=lens_t,
                        scale=1.0 / math.sqrt(D), q_dtype=W.BF16, kv_dtype=kv_dtype, k_scale=k_scale,
                        v_scale=v_scale)


CASES = [
    # H, G, kv dtype, slope per key (base 2)
    (32, 8, W.BF16, 0.2),
    (32, 8, W.BF16, 1.0),
    (32, 8, W.BF16, -0.5),
    (32, 1, W.BF16, 0.2),
    (32, 1, W.FP8, 0.3),
    (32, 8, W.FP8, 1.0),
    (32, 1, W.INT4, 1.0),
    (32, 8, W.INT4, 0.2),
]


@pytest.mark.parametrize("H,G,kvd,slope", CASES)
def test_ramped_scores(gqa, H, G, kvd, slope):
    lens = [2048, 1500, 33]
    c = ramp_case(3, H, G, lens, 2048, kvd, slope, seed=int(100 * abs(slope)) + H + G)
    want = oracle.decode(c)
    d = "cuda"
    ks = c.k_scale.to(d) if c.k_scale is not None else None
    vs = c.v_scale.to(d) if c.v_scale is not None else None
    for splits in (1, 0):
        _say(f"[gpu] ramp slope={slope} H{H} G{G} kv={kvd} splits={splits}")
        out = gqa.decode(c.q.to(d), c.k_cache.to(d), c.v_cache.to(d), c.seq_lens.to(d), scale=c.scale,
                         k_scale=ks, v_scale=vs, num_splits=splits, path="mfma")
        torch.cuda.synchronize()
        got = out.detach().cpu().to(torch.float64).numpy()
        assert np.all(np.isfinite(got)), "non-finite output"
        err = float(np.max(np.abs(got - want)))
        _say(f"    max abs err {err:.3e}")
        assert err <= TOL[kvd], f"slope {slope} splits {splits}: {err} > {TOL[kvd]}"
