"""Pins for the oracle's INT4 KV format (CPU only), beyond the shared pin list: agreement with
torch's round-half-even on random quotients, and the decode of an INT4 case equalling the
decode of the same values held in fp32 (the format changes storage, not the attention)."""

import numpy as np
import torch

import oracle
import workloads as W


def test_encoder_matches_torch_round():
    g = torch.Generator().manual_seed(5)
    x = torch.cat([torch.randn(20000, generator=g) * 4, (torch.rand(5000, generator=g) * 20 - 10),
                   torch.arange(-9, 8, 0.5)]).to(torch.float32)
    want = (torch.round(x).clamp(-8, 7) + 8).to(torch.int32).numpy()
    got = np.array([oracle.int4_encode(float(v)) for v in x.numpy()])
    assert np.array_equal(got, want)


def test_quantise_matches_input_generator():
    """workloads' slab quantiser and the oracle's encoder give the same fields."""
    c = W.make_decode(2, 8, 2, 64, [50, 17], T_cap=64, kv_dtype=W.INT4, seed=3, name="i4")
    g = torch.Generator("cpu").manual_seed(3)
    _ = torch.randn(2, 8, 64, generator=g)
    k = torch.randn(2, 2, 64, 64, generator=g)
    for b, L in enumerate([50, 17]):
        for gg in range(2):
            want = oracle.quant_int4(k[b, gg, :L].numpy(), float(c.k_scale[b * 2 + gg]))
            assert np.array_equal(c.k_cache[b, gg, :L].numpy(), want)


def test_int4_decode_is_decode_of_values():
    c = W.make_decode(3, 16, 4, 32, [40, 1, 64], T_cap=64, kv_dtype=W.INT4, seed=9, name="i4d")
    k, v = oracle.decode_kv_f64(c)
    assert k.shape == (3, 4, 64, 32)
    ref = oracle.decode_arrays(c.q, k, v, c.seq_lens.numpy(), c.scale)
    assert np.array_equal(oracle.decode(c), ref)
    # every stored value is an integer multiple of its slab's scale, |multiple| <= 8
    m = k / c.k_scale.numpy().astype(np.float64).reshape(3, 4, 1, 1)
    assert np.allclose(m, np.round(m), atol=0) and np.abs(m).max() <= 8
