"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with: hand-worked values (tests/golden), a library routine computing the
same definition (torch's CPU scaled_dot_product_attention in float64, with and
without its grouped-query option), a pure-Python brute force, closed forms, or
invariants that follow from the definition. They run against the real oracle in
``test_oracle_pins.py`` and against builds with planted mistakes in
``test_oracle_mutants.py`` (each planted mistake must trip at least one pin).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    table = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0), "nan": float("nan"),
             "31/7": 31.0 / 7.0}
    return table[x]


def _arr(nested):
    if isinstance(nested, list):
        return [_arr(x) for x in nested]
    return _num(nested)


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a)) and err <= tol, f"{what}: max abs err {err} > {tol}"


# --------------------------------------------------------------------------------------

def pin_hand_worked(orc):
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if c["kind"] == "decode":
            out = orc.decode_arrays(np.array(_arr(c["q"])), np.array(_arr(c["k"])), np.array(_arr(c["v"])),
                                    np.array(c["seq_lens"], dtype=np.int32), c["scale"])
        else:
            out = orc.prefill_arrays(np.array(_arr(c["q"])), np.array(_arr(c["k"])), np.array(_arr(c["v"])),
                                     c["scale"], c["causal"])
        _close(out, np.array(_arr(c["out"])), 1e-12, c["name"])


def pin_toy_three_ways(orc):
    """The 12-dim 4-head toy (H4 G2 D3): prefill of 5 tokens, then decode at L=6 and 7.

    Oracle vs pure-Python brute force vs torch's SDPA (fp64, grouped-query option)."""
    for seed in range(3):
        p = W.toy_prefill(seed)
        q, k, v = (p.q.double(), p.k.double(), p.v.double())
        want_sdpa = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=p.scale, enable_gqa=True)
        want_brute = brute.attention(q.tolist(), k.tolist(), v.tolist(), True, p.scale)
        got = orc.prefill(p)
        _close(got, want_sdpa.numpy(), 1e-13, f"toy prefill vs SDPA seed {seed}")
        _close(got, np.array(want_brute), 1e-13, f"toy prefill vs brute seed {seed}")
        for step in W.toy_decode_steps(seed):
            L = int(step.seq_lens[0])
            qd = step.q.double()[:, :, None, :]
            kd = step.k_cache.double()[:, :, :L]
            vd = step.v_cache.double()[:, :, :L]
            want = F.scaled_dot_product_attention(qd, kd, vd, scale=step.scale, enable_gqa=True)[:, :, 0]
            wb = brute.attention(qd.tolist(), kd.tolist(), vd.tolist(), True, step.scale, q_offset=L - 1)
            got = orc.decode(step)
            _close(got, want.numpy(), 1e-13, f"toy decode L={L} vs SDPA")
            _close(got, np.array(wb)[:, :, 0], 1e-13, f"toy decode L={L} vs brute")


def pin_sdpa_prefill(orc):
    for (B, H, G, D, T, seed) in [(2, 8, 2, 16, 37, 1), (1, 6, 3, 5, 19, 2), (2, 4, 4, 8, 11, 3),
                                  (1, 8, 1, 32, 23, 4)]:
        q = _rand((B, H, T, D), seed)
        k = _rand((B, G, T, D), seed + 100)
        v = _rand((B, G, T, D), seed + 200)
        scale = 1.0 / math.sqrt(D)
        for causal in (True, False):
            want = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale, enable_gqa=True)
            got = orc.prefill_arrays(q, k, v, scale, causal)
            _close(got, want.numpy(), 1e-12, f"prefill vs SDPA B{B}H{H}G{G}D{D}T{T} causal={causal}")
            rows = [0, T - 1, (B * H * T) // 2, B * H * T - 1]
            c = W.PrefillCase("x", q, k, v, scale, causal, W.F32)
            got_rows = orc.prefill_rows(c, rows)
            _close(got_rows, got.reshape(-1, D)[rows], 0.0, "prefill_rows vs prefill")


def pin_sdpa_decode(orc):
    B, H, G, D, T_cap = 3, 8, 2, 16, 29
    lens = np.array([29, 1, 13], dtype=np.int32)
    q = _rand((B, H, D), 7)
    k = _rand((B, G, T_cap, D), 8)
    v = _rand((B, G, T_cap, D), 9)
    for b in range(B):
        k[b, :, lens[b]:] = float("nan")
        v[b, :, lens[b]:] = float("nan")
    scale = 0.3
    got = orc.decode_arrays(q, k, v, lens, scale)
    for b in range(B):
        L = int(lens[b])
        want = F.scaled_dot_product_attention(q[b:b + 1, :, None, :], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                              scale=scale, enable_gqa=True)[0, :, 0]
        _close(got[b], want.numpy(), 1e-12, f"decode vs SDPA b={b} L={L}")
    c = W.DecodeCase("x", q, k, v, torch.tensor(lens), scale, W.F32, W.F32)
    rows = [0, 5, 8, 23]
    _close(orc.decode_rows(c, rows), got.reshape(-1, D)[rows], 0.0, "decode_rows vs decode")


def pin_mha(orc):
    """GQA-H is multi-head attention: each head alone (H=G=1) gives the same row."""
    B, H, D, T = 2, 4, 8, 9
    q, k, v = _rand((B, H, T, D), 11), _rand((B, H, T, D), 12), _rand((B, H, T, D), 13)
    full = orc.prefill_arrays(q, k, v, 0.25, True)
    for b in range(B):
        for h in range(H):
            one = orc.prefill_arrays(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], 0.25, True)
            _close(full[b, h], one[0, 0], 1e-14, f"GQA-H vs single head b={b} h={h}")


def pin_mqa(orc):
    """GQA-1 is multi-query attention: one KV head broadcast to every query head."""
    B, H, D, T = 2, 6, 8, 10
    q, k, v = _rand((B, H, T, D), 21), _rand((B, 1, T, D), 22), _rand((B, 1, T, D), 23)
    one = orc.prefill_arrays(q, k, v, 0.4, True)
    mat = orc.prefill_arrays(q, k.expand(B, H, T, D), v.expand(B, H, T, D), 0.4, True)
    _close(one, mat, 0.0, "GQA-1 vs materialised MQA")


def pin_group_materialise(orc):
    """General G equals G=H with each KV head repeated for its R consecutive query heads."""
    for (H, G) in [(8, 2), (6, 3), (12, 4)]:
        R = H // G
        B, D, T = 2, 8, 7
        q, k, v = _rand((B, H, T, D), 31 + H), _rand((B, G, T, D), 32 + H), _rand((B, G, T, D), 33 + H)
        got = orc.prefill_arrays(q, k, v, 0.35, True)
        want = orc.prefill_arrays(q, k.repeat_interleave(R, dim=1), v.repeat_interleave(R, dim=1), 0.35, True)
        _close(got, want, 0.0, f"prefill H{H} G{G} vs repeat_interleave")
        lens = np.array([T, 3], dtype=np.int32)
        gd = orc.decode_arrays(q[:, :, 0], k, v, lens, 0.35)
        wd = orc.decode_arrays(q[:, :, 0], k.repeat_interleave(R, dim=1), v.repeat_interleave(R, dim=1), lens, 0.35)
        _close(gd, wd, 0.0, f"decode H{H} G{G} vs repeat_interleave")


def pin_identical_keys_mean_v(orc):
    """All key rows equal -> uniform weights -> the mean of the attended value rows."""
    B, H, G, D, T = 2, 4, 2, 8, 12
    q = _rand((B, H, T, D), 41)
    k = _rand((B, G, 1, D), 42).expand(B, G, T, D).contiguous()
    v = _rand((B, G, T, D), 43)
    out = orc.prefill_arrays(q, k, v, 0.5, True)
    vn = v.numpy()
    for h in range(H):
        g = h // (H // G)
        for i in range(T):
            _close(out[:, h, i], vn[:, g, :i + 1].mean(axis=1), 1e-14, f"prefill identical K h={h} i={i}")
    lens = np.array([T, 5], dtype=np.int32)
    od = orc.decode_arrays(q[:, :, 0], k, v, lens, 0.5)
    for b in range(B):
        for h in range(H):
            _close(od[b, h], vn[b, h // 2, :lens[b]].mean(axis=0), 1e-14, "decode identical K")
    # scale 0 makes every score equal as well
    out0 = orc.prefill_arrays(q, _rand((B, G, T, D), 44), v, 0.0, False)
    for h in range(H):
        _close(out0[:, h], np.repeat(vn[:, h // 2].mean(axis=1, keepdims=True), T, axis=1), 1e-14, "scale 0")


def pin_value_constant_per_head(orc):
    """V[b, g] = g + 1 everywhere -> out[b, h] = h // R + 1: pins the head->group map alone."""
    B, H, G, D, T = 2, 12, 3, 4, 6
    q, k = _rand((B, H, T, D), 51), _rand((B, G, T, D), 52)
    v = torch.zeros(B, G, T, D, dtype=torch.float64)
    for g in range(G):
        v[:, g] = g + 1.0
    out = orc.prefill_arrays(q, k, v, 1.0, True)
    for h in range(H):
        assert np.allclose(out[:, h], h // (H // G) + 1.0, atol=1e-13, rtol=0), f"head {h}"
    od = orc.decode_arrays(q[:, :, 0], k, v, np.array([T, 2], dtype=np.int32), 1.0)
    for h in range(H):
        assert np.allclose(od[:, h], h // (H // G) + 1.0, atol=1e-13, rtol=0), f"decode head {h}"


def pin_single_row(orc):
    """L_b = 1 -> the one cached value row, whatever the scores."""
    B, H, G, D, T_cap = 2, 4, 1, 8, 5
    q, k, v = _rand((B, H, D), 61) * 30, _rand((B, G, T_cap, D), 62), _rand((B, G, T_cap, D), 63)
    out = orc.decode_arrays(q, k, v, np.array([1, 1], dtype=np.int32), 1.0)
    for h in range(H):
        _close(out[:, h], v[:, 0, 0].numpy(), 0.0, "L_b = 1")
    # prefill row 0 is value row 0 under the causal mask
    qp, kp, vp = _rand((1, 2, 4, 8), 64), _rand((1, 1, 4, 8), 65), _rand((1, 1, 4, 8), 66)
    op = orc.prefill_arrays(qp, kp, vp, 1.0, True)
    _close(op[0, :, 0], np.repeat(vp[0, :, 0].numpy(), 2, axis=0), 0.0, "causal row 0")


def pin_shift_invariance(orc):
    """Adding one vector to every key row adds q.c to every score: the output is unchanged."""
    B, H, G, D, T = 1, 4, 2, 8, 10
    q, k, v = _rand((B, H, T, D), 71), _rand((B, G, T, D), 72), _rand((B, G, T, D), 73)
    c = _rand((1, 1, 1, D), 74)
    a = orc.prefill_arrays(q, k, v, 0.3, False)
    b = orc.prefill_arrays(q, k + c, v, 0.3, False)
    _close(a, b, 1e-12, "key shift invariance")


def pin_permutation_invariance(orc):
    """Decode: reordering the cached rows leaves the output unchanged."""
    B, H, G, D, T = 1, 8, 2, 16, 33
    q, k, v = _rand((B, H, D), 81), _rand((B, G, T, D), 82), _rand((B, G, T, D), 83)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(5))
    lens = np.array([T], dtype=np.int32)
    a = orc.decode_arrays(q, k, v, lens, 0.25)
    b = orc.decode_arrays(q, k[:, :, perm], v[:, :, perm], lens, 0.25)
    _close(a, b, 1e-13, "cache row permutation")


def pin_linear_and_convex(orc):
    """The output is linear in V and lies inside the box spanned by the attended rows."""
    B, H, G, D, T = 1, 4, 2, 8, 9
    q, k = _rand((B, H, T, D), 91), _rand((B, G, T, D), 92)
    v1, v2 = _rand((B, G, T, D), 93), _rand((B, G, T, D), 94)
    o1 = orc.prefill_arrays(q, k, v1, 0.5, True)
    o2 = orc.prefill_arrays(q, k, v2, 0.5, True)
    o3 = orc.prefill_arrays(q, k, 2.0 * v1 - 3.0 * v2, 0.5, True)
    _close(o3, 2.0 * o1 - 3.0 * o2, 1e-12, "linearity in V")
    v1n = v1.numpy()
    for h in range(H):
        for i in range(T):
            rows = v1n[0, h // 2, :i + 1]
            assert np.all(o1[0, h, i] <= rows.max(axis=0) + 1e-12) and np.all(o1[0, h, i] >= rows.min(axis=0) - 1e-12)


def pin_incremental_decode_equals_prefill(orc):
    """Decoding token t against the cache of tokens 0..t equals causal prefill row t."""
    B, H, G, D, T = 2, 8, 2, 16, 24
    q, k, v = _rand((B, H, T, D), 101), _rand((B, G, T, D), 102), _rand((B, G, T, D), 103)
    full = orc.prefill_arrays(q, k, v, 0.25, True)
    for t in range(T):
        kc = torch.full((B, G, T + 3, D), float("nan"), dtype=torch.float64)
        vc = torch.full((B, G, T + 3, D), float("nan"), dtype=torch.float64)
        kc[:, :, :t + 1] = k[:, :, :t + 1]
        vc[:, :, :t + 1] = v[:, :, :t + 1]
        out = orc.decode_arrays(q[:, :, t], kc, vc, np.full(B, t + 1, dtype=np.int32), 0.25)
        _close(out, full[:, :, t], 1e-13, f"decode step {t} vs prefill row {t}")


def pin_nan_padding(orc):
    """Cache rows beyond L_b are never read (NaN there must not reach the output)."""
    B, H, G, D, T_cap = 2, 4, 2, 8, 16
    q, k, v = _rand((B, H, D), 111), _rand((B, G, T_cap, D), 112), _rand((B, G, T_cap, D), 113)
    lens = np.array([7, 16], dtype=np.int32)
    clean = orc.decode_arrays(q, k, v, lens, 0.5)
    kp, vp = k.clone(), v.clone()
    kp[0, :, 7:] = float("nan")
    vp[0, :, 7:] = float("inf")
    dirty = orc.decode_arrays(q, kp, vp, lens, 0.5)
    _close(dirty, clean, 0.0, "NaN/inf padding")


def pin_length_readings(orc):
    """L_b beyond the capacity is clamped; L_b <= 0 gives a zero row."""
    B, H, G, D, T_cap = 3, 4, 2, 8, 10
    q, k, v = _rand((B, H, D), 121), _rand((B, G, T_cap, D), 122), _rand((B, G, T_cap, D), 123)
    a = orc.decode_arrays(q, k, v, np.array([10, 0, -3], dtype=np.int32), 0.5)
    b = orc.decode_arrays(q, k, v, np.array([50, 0, -3], dtype=np.int32), 0.5)
    _close(a, b, 0.0, "clamp to capacity")
    assert np.all(a[1:] == 0.0)


def pin_e4m3fn_decoder(orc):
    """OCP E4M3FN decoding: every code against torch's float8_e4m3fn conversion, plus
    landmark values of the format (448, 2^-6, 2^-9, NaN)."""
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3fn_value(c) for c in range(256)])
    nan_w = np.isnan(want)
    assert np.array_equal(nan_w, np.isnan(got)), "NaN codes"
    assert np.array_equal(got[~nan_w], want[~nan_w]), "finite codes"
    assert orc.e4m3fn_value(0x7E) == 448.0 and orc.e4m3fn_value(0xFE) == -448.0
    assert orc.e4m3fn_value(0x08) == 2.0 ** -6 and orc.e4m3fn_value(0x01) == 2.0 ** -9
    assert orc.e4m3fn_value(0x38) == 1.0 and math.isnan(orc.e4m3fn_value(0x7F))
    sc = torch.tensor([0.5, 3.0], dtype=torch.float32)
    deq = orc.dequant_e4m3fn(codes.view(2, 128).view(torch.float8_e4m3fn), sc)
    assert np.array_equal(deq[0][~nan_w[:128]], want[:128][~nan_w[:128]] * 0.5)
    assert np.array_equal(deq[1][~nan_w[128:]], want[128:][~nan_w[128:]] * 3.0)


def pin_e4m3fn_encoder(orc):
    """The encoder against the format and a library cast: every finite code round-trips,
    every midpoint between neighbouring codes goes to the even one, values beyond 448
    saturate, and values inside the range match torch's float8_e4m3fn cast (nearest even);
    the quotient x / scale is taken in fp32."""
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for c in finite:
        assert orc.e4m3fn_encode(orc.e4m3fn_value(c)) == c, f"round trip {c:#x}"
    pos = sorted(finite[:127], key=orc.e4m3fn_value)
    for lo, hi in zip(pos, pos[1:]):
        mid = (orc.e4m3fn_value(lo) + orc.e4m3fn_value(hi)) / 2
        even = lo if (lo & 1) == 0 else hi
        assert orc.e4m3fn_encode(mid) == even and orc.e4m3fn_encode(-mid) == even | 0x80, f"midpoint {lo:#x}"
    for big in (449.0, 1e6):
        assert orc.e4m3fn_encode(big) == 0x7E and orc.e4m3fn_encode(-big) == 0xFE, "saturation"
    g = torch.Generator().manual_seed(11)
    x = torch.cat([torch.randn(4000, generator=g) * 60, (torch.rand(1000, generator=g) * 2 - 1) * 448])
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.quant_e4m3fn(x.numpy(), 1.0), want), "library cast"
    q = np.float32(np.float32(1.3) / np.float32(0.37))
    assert orc.quant_e4m3fn([np.float32(1.3)], np.float32(0.37))[0] == orc.e4m3fn_encode(q), "fp32 quotient"


def pin_chunk_special_cases(orc):
    """Chunked prefill reduces to decode (Tq = 1; the decode has its own coding of the softmax,
    so equal up to rounding) and to plain prefill (L = Tq = T_cap; exactly: same rows, same key
    counts, same summation order)."""
    B, H, G, D, T = 2, 8, 2, 16, 20
    q, k, v = _rand((B, H, T, D), 201), _rand((B, G, T, D), 202), _rand((B, G, T, D), 203)
    lens = np.array([T, 7], dtype=np.int32)
    one = orc.prefill_cached_arrays(q[:, :, :1], k, v, lens, 0.3, True)[:, :, 0]
    _close(one, orc.decode_arrays(q[:, :, 0], k, v, lens, 0.3), 1e-13, "Tq = 1 is decode")
    full = np.full(B, T, dtype=np.int32)
    for causal in (True, False):
        got = orc.prefill_cached_arrays(q, k, v, full, 0.3, causal)
        assert np.array_equal(got, orc.prefill_arrays(q, k, v, 0.3, causal)), f"whole chunk, causal={causal}"


def pin_chunks_compose_prefill(orc):
    """Chunks [0,5), [5,17), [17,24) against a growing cache give the causal prefill rows."""
    B, H, G, D, T, T_cap = 2, 8, 2, 16, 24, 30
    q, k, v = _rand((B, H, T, D), 211), _rand((B, G, T, D), 212), _rand((B, G, T, D), 213)
    full = orc.prefill_arrays(q, k, v, 0.25, True)
    for s, e in ((0, 5), (5, 17), (17, 24)):
        kc = torch.full((B, G, T_cap, D), float("nan"), dtype=torch.float64)
        vc = torch.full((B, G, T_cap, D), float("nan"), dtype=torch.float64)
        kc[:, :, :e] = k[:, :, :e]
        vc[:, :, :e] = v[:, :, :e]
        got = orc.prefill_cached_arrays(q[:, :, s:e], kc, vc, np.full(B, e, dtype=np.int32), 0.25, True)
        assert np.array_equal(got, full[:, :, s:e]), f"chunk [{s},{e})"


def pin_chunk_short_cache(orc):
    """L < Tq: rows before position 0 see no key (zero); the row at position 0 sees key 0 only
    (its output is v[0]). Not causal: every row sees all L keys, as a decode at length L."""
    B, H, G, D, Tq, T_cap = 1, 4, 2, 8, 6, 6
    q, k, v = _rand((B, H, Tq, D), 221), _rand((B, G, T_cap, D), 222), _rand((B, G, T_cap, D), 223)
    L = 3
    lens = np.array([L], dtype=np.int32)
    got = orc.prefill_cached_arrays(q, k, v, lens, 0.5, True)
    assert np.all(got[:, :, :Tq - L] == 0), "rows before position 0"
    for h in range(H):
        assert np.array_equal(got[0, h, Tq - L], v[0, h // 2, 0].numpy()), "position 0 sees key 0 only"
    nc = orc.prefill_cached_arrays(q, k, v, lens, 0.5, False)
    for i in range(Tq):
        _close(nc[:, :, i], orc.decode_arrays(q[:, :, i], k, v, lens, 0.5), 1e-13, f"row {i}")


def pin_int4_format(orc):
    """INT4 fields: every field encodes back to itself, midpoints go to the even integer, values
    saturate at -8 and 7, NaN stores zero; a hand-packed byte decodes low field first."""
    for u in range(16):
        assert orc.int4_value(u) == u - 8
        assert orc.int4_encode(float(u - 8)) == u, f"field {u}"
    for k in range(-8, 7):
        even = k if k % 2 == 0 else k + 1
        assert orc.int4_encode(k + 0.5) == even + 8, f"midpoint {k} + 1/2"
        assert orc.int4_encode(np.nextafter(np.float32(k + 0.5), np.float32(-100))) == k + 8
    assert orc.int4_encode(100.0) == 15 and orc.int4_encode(-100.0) == 0
    assert orc.int4_encode(7.5) == 15 and orc.int4_encode(-8.5) == 0
    assert orc.int4_encode(float("nan")) == 8
    vals = orc.dequant_int4(torch.tensor([[0x1F, 0x80]], dtype=torch.uint8), torch.tensor([0.5]))
    assert np.array_equal(vals, [[3.5, -3.5, -4.0, 0.0]]), vals
    assert np.array_equal(orc.quant_int4(np.array([3.4, -3.6, -4.0, 0.2], dtype=np.float32), 0.5),
                          np.array([0x1F, 0x80], dtype=np.uint8))


ALL_PINS = [pin_hand_worked, pin_toy_three_ways, pin_sdpa_prefill, pin_sdpa_decode, pin_mha, pin_mqa,
            pin_group_materialise, pin_identical_keys_mean_v, pin_value_constant_per_head, pin_single_row,
            pin_shift_invariance, pin_permutation_invariance, pin_linear_and_convex,
            pin_incremental_decode_equals_prefill, pin_nan_padding, pin_length_readings, pin_e4m3fn_decoder,
            pin_e4m3fn_encoder, pin_chunk_special_cases, pin_chunks_compose_prefill, pin_chunk_short_cache,
            pin_int4_format]
