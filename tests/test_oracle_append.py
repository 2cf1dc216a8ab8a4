"""Pins for the oracle's fp8 encoder and cache append (CPU only).

The encoder is pinned against the format itself (every finite code decodes and encodes back
to itself; every midpoint between neighbouring codes goes to the even one), against
saturation and NaN, and against an independent library routine (torch's float8_e4m3fn cast,
which rounds to nearest even) on random values inside the finite range.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W


@pytest.fixture(scope="module")
def o():
    return oracle.load()


FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_every_finite_code_round_trips(o):
    for c in FINITE:
        assert o.e4m3fn_encode(o.e4m3fn_value(c)) == c, hex(c)


def test_midpoints_round_to_even(o):
    pos = sorted(FINITE[:127], key=o.e4m3fn_value)  # 0x00 .. 0x7E, increasing values
    for lo, hi in zip(pos, pos[1:]):
        mid = (o.e4m3fn_value(lo) + o.e4m3fn_value(hi)) / 2
        assert np.float32(mid) == mid            # every midpoint is a float
        even = lo if (lo & 1) == 0 else hi
        assert o.e4m3fn_encode(mid) == even, (hex(lo), hex(hi))
        assert o.e4m3fn_encode(-mid) == even | 0x80
        # just off the midpoint goes to the nearer code
        assert o.e4m3fn_encode(np.nextafter(np.float32(mid), np.float32(0))) == lo
        assert o.e4m3fn_encode(np.nextafter(np.float32(mid), np.float32(1e9))) == hi


def test_saturation_and_specials(o):
    assert o.e4m3fn_encode(448.0) == 0x7E and o.e4m3fn_value(0x7E) == 448.0
    for big in (449.0, 464.0, 1e6, float("inf")):
        assert o.e4m3fn_encode(big) == 0x7E
        assert o.e4m3fn_encode(-big) == 0xFE
    assert o.e4m3fn_encode(float("nan")) == 0x7F
    assert o.e4m3fn_encode(0.0) == 0x00 and o.e4m3fn_encode(-0.0) == 0x80
    assert o.e4m3fn_encode(2.0 ** -10) == 0x00          # half the smallest subnormal: tie to 0
    assert o.e4m3fn_encode(1.5 * 2.0 ** -10) == 0x01


def test_matches_torch_cast_inside_the_range(o):
    g = torch.Generator().manual_seed(7)
    x = torch.cat([torch.randn(20000, generator=g) * 60, torch.randn(20000, generator=g) * 0.01,
                   (torch.rand(5000, generator=g) * 2 - 1) * 448])
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = o.quant_e4m3fn(x.numpy(), 1.0)
    assert np.array_equal(got, want)


def test_quotient_taken_in_fp32(o):
    x = np.float32(1.3)
    s = np.float32(0.37)
    assert o.quant_e4m3fn([x], s)[0] == o.e4m3fn_encode(np.float32(x / s))


@pytest.mark.parametrize("kv", [W.BF16, W.FP8, W.F32])
def test_append_writes_one_row(o, kv):
    qd = W.F32 if kv == W.F32 else W.BF16
    c = W.make_decode(3, 8, 2, 16, [5, 1, 9], T_cap=9, q_dtype=qd, kv_dtype=kv, seed=3, name="append")
    g = torch.Generator().manual_seed(4)
    kn = (torch.randn(3, 2, 16, generator=g) * 2).to(c.q.dtype)
    vn = (torch.randn(3, 2, 16, generator=g) * 2).to(c.q.dtype)
    kc, vc = o.append(c, kn, vn)
    raw = lambda t: t.contiguous().view(torch.uint8)   # bytes: the poisoned rows are NaN
    for b, L in enumerate([5, 1, 9]):
        for gg in range(2):
            rows = [r for r in range(9) if r != L - 1]
            assert torch.equal(raw(kc[b, gg, rows]), raw(c.k_cache[b, gg, rows]))   # nothing else moved
            assert torch.equal(raw(vc[b, gg, rows]), raw(c.v_cache[b, gg, rows]))
            if kv == W.FP8:
                back = o.dequant_e4m3fn(kc[b:b + 1, gg, L - 1], c.k_scale[b * 2 + gg:b * 2 + gg + 1])[0]
                sc = float(c.k_scale[b * 2 + gg])
                x = np.clip(kn[b, gg].float().numpy(), -448 * sc, 448 * sc)         # saturation at 448
                step = sc * np.maximum(np.abs(x) / sc, 2 ** -6) / 8
                assert np.all(np.abs(back - x) <= step + 1e-12)                     # within one code step
                big = np.abs(kn[b, gg].float().numpy()) > 448 * sc
                assert np.all(np.abs(back[big]) == 448 * sc)
            else:
                assert torch.equal(kc[b, gg, L - 1], kn[b, gg].to(kc.dtype))
                assert torch.equal(vc[b, gg, L - 1], vn[b, gg].to(vc.dtype))
