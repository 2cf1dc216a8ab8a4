"""Pins for the oracle's paged-cache decode (CPU only).

The paged oracle gathers the logical cache through the block table and runs the contiguous
decode definition. It is pinned by:
  * a hand-built table whose answer follows from which rows the length admits (keys all
    zero, so the output is the mean of the admitted values);
  * equality with the contiguous oracle on cases that workloads.make_paged scattered into
    shuffled pages (independent code: the scatter there, the gather here), for bf16 and fp8
    caches and several page sizes;
  * invariance under a different shuffle of the same pages;
  * a planted mistake (page and in-page offset swapped in a copy of the gather) that the pins
    catch.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _paged(q, k_pages, v_pages, table, lens, scale=1.0):
    return W.PagedDecodeCase(name="hand", q=q, k_pages=k_pages, v_pages=v_pages,
                             block_table=torch.tensor(table, dtype=torch.int32),
                             seq_lens=torch.tensor(lens, dtype=torch.int32), scale=scale, q_dtype=W.F32,
                             kv_dtype=W.F32)


def hand_case(L):
    # One sequence, one KV head, D = 2, pages of 2 rows. Physical row (page p, offset r) holds
    # the value 10 p + r; keys are zero, so every admitted row weighs the same.
    pool_v = torch.zeros(3, 1, 2, 2)
    for p in range(3):
        for r in range(2):
            pool_v[p, 0, r, 0] = 10 * p + r
    pool_k = torch.zeros(3, 1, 2, 2)
    q = torch.tensor([[[1.0, 0.0]]])
    # logical rows 0, 1 -> page 2; rows 2, 3 -> page 0.
    return _paged(q, pool_k, pool_v, [[2, 0]], [L])


@pytest.mark.parametrize("L,admitted", [(1, [20]), (2, [20, 21]), (3, [20, 21, 0]), (4, [20, 21, 0, 1])])
def test_hand_built_table(L, admitted):
    out = oracle.decode_paged(hand_case(L))
    assert out.shape == (1, 1, 2)
    assert out[0, 0, 0] == pytest.approx(sum(admitted) / len(admitted), abs=1e-12)
    assert out[0, 0, 1] == 0.0


@pytest.mark.parametrize("kv,page_size", [(W.BF16, 16), (W.BF16, 64), (W.FP8, 32), (W.BF16, 512), (W.F32, 16)])
def test_paged_equals_contiguous(kv, page_size):
    qd = W.F32 if kv == W.F32 else W.BF16
    c = W.make_decode(4, 16, 2, 64, [300, 1, 0, 129], T_cap=300, q_dtype=qd, kv_dtype=kv, seed=page_size,
                      name="pin")
    p = W.make_paged(c, page_size, seed=7)
    assert p.T_cap >= c.T_cap
    assert np.array_equal(oracle.decode_paged(p), oracle.decode(c))


def test_shuffle_invariance():
    c = W.make_decode(3, 8, 2, 32, [70, 33, 5], T_cap=80, seed=4, name="perm")
    a = oracle.decode_paged(W.make_paged(c, 16, seed=1))
    b = oracle.decode_paged(W.make_paged(c, 16, seed=2, spare_pages=9))
    assert np.array_equal(a, b)


def test_swapped_gather_is_caught(monkeypatch):
    """A copy of the gather with page index and in-page offset swapped fails the pins."""
    o = oracle.load()

    def swapped(case):
        kp, vp, bt = case.k_pages, case.v_pages, case.block_table.to(torch.int64)
        B, pps = bt.shape
        ps = kp.shape[2]
        t = torch.arange(pps * ps)
        page = bt[:, (t % pps)]
        off = (t // pps).expand(B, -1).clamp(max=ps - 1)
        g = lambda pool: pool[page, :, off].permute(0, 2, 1, 3).contiguous()
        return g(kp), g(vp)

    monkeypatch.setattr(o, "paged_kv", swapped)
    caught = 0
    try:
        for L, adm in ((1, [20]), (2, [20, 21]), (3, [20, 21, 0]), (4, [20, 21, 0, 1])):
            test_hand_built_table(L, adm)
    except AssertionError:
        caught += 1
    c = W.make_decode(4, 16, 2, 64, [300, 1, 0, 129], T_cap=300, seed=16, name="pin")
    with np.errstate(invalid="ignore"):
        if not np.array_equal(o.decode_paged(W.make_paged(c, 16, seed=7)), o.decode(c), equal_nan=True):
            caught += 1
    assert caught == 2


@pytest.mark.parametrize("kvd,ps", [(W.BF16, 16), (W.BF16, 64), (W.FP8, 32)])
def test_paged_chunk_is_the_contiguous_chunk(kvd, ps):
    """A chunk against a paged cache gathers the same logical rows: its oracle output equals
    the contiguous chunk's exactly (padding pages and spare pages hold poison)."""
    c = W.make_chunk(3, 16, 4, 128, 40, [300, 40, 0], T_cap=320, seed=5, name="pc", kv_dtype=kvd)
    p = W.make_paged_chunk(c, ps, seed=ps)
    assert p.T_cap >= c.T_cap
    np.testing.assert_array_equal(oracle.prefill_paged(p), oracle.prefill_cached(c))
