"""KV caches whose rows lie more than 4 GiB from their base, through the C ABI (needs a gfx950
GPU with ~18 GB free).

The valid rows of the last KV head sit past 4 GiB (contiguous caches: its slab starts there;
paged caches: the block table points at the pool's last pages), so every byte offset that the
decode, paged-decode and chunked-prefill kernels form has to be 64-bit. Every row that is not
a valid cache row holds NaN (bf16) or a NaN code (fp8). The oracle sees only the valid rows: a
small case with the same values and T_cap = the length.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32
D = 128
L = 3000  # valid rows of every sequence


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_decode_amd as g
    assert torch.cuda.is_available(), "no GPU"
    g.library()
    yield g
    torch.cuda.empty_cache()


def _big_cache(small, row_bytes, poison):
    """small [B, G, L, D] (CPU) -> a device cache [B, G, T_cap, D] whose last slab starts past
    4 GiB, rows past L filled with `poison`."""
    B, G, Ls, Dd = small.shape
    T_cap = FOUR_GIB // (row_bytes * (B * G - 1)) + 64
    assert (B * G - 1) * T_cap * row_bytes > FOUR_GIB
    if small.dtype == torch.float8_e4m3fn:  # filled as bytes: poison is a code
        big = torch.full((B, G, T_cap, Dd), poison, dtype=torch.uint8, device="cuda")
        big[:, :, :Ls] = small.view(torch.uint8).to("cuda")
        return big.view(torch.float8_e4m3fn)
    big = torch.full((B, G, T_cap, Dd), poison, dtype=small.dtype, device="cuda")
    big[:, :, :Ls] = small.to("cuda")
    return big


def _check(got, want, tol, what):
    got = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want)))
    _say(f"    {what}: max abs err {err:.3e}")
    assert err <= tol, f"{what}: {err} > {tol}"


@pytest.mark.parametrize("layout", ["uniform", "flat"])
def test_decode_rows_past_4gib(gqa, layout):
    c = W.make_decode(1, 8, 2, D, L, T_cap=L, seed=11, name="decode_4gib")
    want = oracle.decode(c)
    k = _big_cache(c.k_cache, D * 2, float("nan"))
    v = _big_cache(c.v_cache, D * 2, float("nan"))
    _say(f"[gpu] decode B1 H8 G2 L{L} T_cap {k.shape[2]} (slab of KV head 1 at {k.shape[2] * D * 2 / 2**30:.2f} GiB) "
         f"layout={layout}")
    out = gqa.decode(c.q.cuda(), k, v, c.seq_lens.cuda(), scale=c.scale, layout=layout)
    torch.cuda.synchronize()
    _check(out, want, 2e-2, f"decode {layout}")
    del k, v


def test_paged_decode_pages_past_4gib(gqa):
    c = W.make_decode(1, 8, 2, D, L, T_cap=L, seed=12, name="paged_4gib")
    want = oracle.decode(c)
    ps = 16
    page_bytes = c.G * ps * D * 2
    n_used = (L + ps - 1) // ps
    num_pages = FOUR_GIB // page_bytes + n_used + 8
    # The sequence's pages are the pool's last ones, in reverse order: all past 4 GiB.
    table = torch.tensor([num_pages - 1 - j for j in range(n_used)], dtype=torch.int32).reshape(1, n_used)
    assert int(table.min()) * page_bytes > FOUR_GIB
    pools = []
    for small in (c.k_cache, c.v_cache):
        pool = torch.full((num_pages, c.G, ps, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        padded = torch.full((c.G, n_used * ps, D), float("nan"), dtype=torch.bfloat16)
        padded[:, :L] = small[0]
        pool[table[0].long().cuda()] = padded.reshape(c.G, n_used, ps, D).permute(1, 0, 2, 3).contiguous().cuda()
        pools.append(pool)
    _say(f"[gpu] paged decode B1 H8 G2 L{L} pages {num_pages} x {page_bytes} B, table past 4 GiB")
    out = gqa.decode_paged(c.q.cuda(), pools[0], pools[1], table.cuda(), c.seq_lens.cuda(), scale=c.scale)
    torch.cuda.synchronize()
    _check(out, want, 2e-2, "paged decode")
    del pools


@pytest.mark.parametrize("kv", [W.BF16, W.FP8])
def test_chunk_rows_past_4gib(gqa, kv):
    Tq = 96
    c = W.make_chunk(1, 8, 2, D, Tq, [L], T_cap=L, seed=13, name="chunk_4gib", kv_dtype=kv)
    want = oracle.prefill_cached(c)
    if kv == W.FP8:
        # E4M3FN 0x7F is NaN; the chunk kernel reads rows past the length as zeros anyway.
        k = _big_cache(c.k_cache, D, 0x7F)
        v = _big_cache(c.v_cache, D, 0x7F)
        ks, vs = c.k_scale.cuda(), c.v_scale.cuda()
    else:
        k = _big_cache(c.k_cache, D * 2, float("nan"))
        v = _big_cache(c.v_cache, D * 2, float("nan"))
        ks = vs = None
    _say(f"[gpu] chunk B1 H8 G2 Tq{Tq} L{L} kv={kv} T_cap {k.shape[2]}")
    out = gqa.prefill_cached(c.q.cuda(), k, v, c.seq_lens.cuda(), scale=c.scale, causal=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    _check(out, want, 2e-2 if kv == W.BF16 else 5e-2, f"chunk {kv}")
    del k, v
