"""Seeded synthetic inputs for grouped-query attention (host tensors only).

This module is shared by the tests, the benchmark and the oracle checks. It draws
random numbers and lays them out in the storage formats the kernels read; it holds
none of the attention arithmetic.

Recipe (every workload):
  * generator: ``torch.Generator('cpu').manual_seed(seed)``;
  * draw order: per-sequence cache lengths (ragged decode only), then Q, then K,
    then V, each ``torch.randn`` in float32 over the full allocated shape, then cast
    to the storage dtype (bf16 rounding is round-to-nearest-even);
  * KV-cache rows at or beyond a sequence's valid length are poisoned with NaN, so a
    kernel that reads them produces NaN in its output;
  * fp8 KV (OCP E4M3FN, largest finite value 448): one float32 scale per
    (sequence, KV head) for K and one for V, each the absolute maximum of that
    slab's valid rows divided by 448; codes are ``round_to_nearest_even(x / scale)``
    via torch's cast. The stored value a code stands for is ``fp8(code) * scale``.

Layouts (head-major, head dim innermost: the projections of the page "Hands-on:
implementing GQA in PyTorch", section 1.1, are reshaped to batch, heads, sequence,
head dim in that order):
  decode  q / out    [B, H, D]
          k / v cache [B, G, T_cap, D], seq_lens int32 [B]
  prefill q / out    [B, H, T, D]
          k / v      [B, G, T, D]
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8_e4m3fn"
INT4 = "int4"   # packed: [..., D/2] uint8, low four bits = even head dim, field u = code + 8

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.float8_e4m3fn}
FP8_MAX = 448.0


@dataclass
class DecodeCase:
    """One single-token decode step over a KV cache."""

    name: str
    q: torch.Tensor            # [B, H, D] q_dtype
    k_cache: torch.Tensor      # [B, G, T_cap, D] kv_dtype
    v_cache: torch.Tensor      # [B, G, T_cap, D] kv_dtype
    seq_lens: torch.Tensor     # [B] int32, valid rows per sequence (current token included)
    scale: float
    q_dtype: str
    kv_dtype: str
    k_scale: Optional[torch.Tensor] = None   # [B*G] float32, fp8 only
    v_scale: Optional[torch.Tensor] = None   # [B*G] float32, fp8 only

    @property
    def B(self): return self.q.shape[0]
    @property
    def H(self): return self.q.shape[1]
    @property
    def D(self): return self.q.shape[2]
    @property
    def G(self): return self.k_cache.shape[1]
    @property
    def T_cap(self): return self.k_cache.shape[2]


@dataclass
class PrefillCase:
    """Full-sequence (prefill) attention, causal or not."""

    name: str
    q: torch.Tensor   # [B, H, T, D]
    k: torch.Tensor   # [B, G, T, D]
    v: torch.Tensor   # [B, G, T, D]
    scale: float
    causal: bool
    dtype: str

    @property
    def B(self): return self.q.shape[0]
    @property
    def H(self): return self.q.shape[1]
    @property
    def T(self): return self.q.shape[2]
    @property
    def D(self): return self.q.shape[3]
    @property
    def G(self): return self.k.shape[1]


def _gen(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(seed)


def _randn(shape, g):
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def quantize_fp8_slabs(x: torch.Tensor, seq_lens: torch.Tensor):
    """Store float32 ``x`` [B, G, T_cap, D] as E4M3FN codes with one scale per (b, g).

    The scale is the slab's absolute maximum over its valid rows divided by 448; the
    codes of padding rows are NaN. Returns (codes as float8_e4m3fn tensor, scales
    float32 [B*G]).
    """
    B, G, T_cap, D = x.shape
    codes = torch.empty(x.shape, dtype=torch.float8_e4m3fn)
    scales = torch.empty(B * G, dtype=torch.float32)
    for b in range(B):
        L = int(min(max(int(seq_lens[b]), 0), T_cap))
        for g in range(G):
            slab = x[b, g, :L]
            amax = float(slab.abs().max()) if L > 0 else 0.0
            s = amax / FP8_MAX if amax > 0 else 1.0
            s = float(torch.tensor(s, dtype=torch.float32))
            scales[b * G + g] = s
            q = torch.full((T_cap, D), float("nan"), dtype=torch.float32)
            q[:L] = slab / s
            codes[b, g] = q.to(torch.float8_e4m3fn)
    return codes, scales


INT4_MAX = 7.0


def quantize_int4_slabs(x: torch.Tensor, seq_lens: torch.Tensor):
    """Store float32 ``x`` [B, G, T_cap, D] as packed INT4 fields with one scale per (b, g):
    scale = absmax of the slab's valid rows / 7, code = round-half-even(x / scale) clamped to
    -8 .. 7, field = code + 8, two fields per byte (low four bits = even head dim). Padding
    rows hold 0xFF (the largest value, 7 * scale: a kernel that reads them is off). Returns
    (packed uint8 [B, G, T_cap, D/2], scales float32 [B*G])."""
    B, G, T_cap, D = x.shape
    assert D % 2 == 0
    packed = torch.full((B, G, T_cap, D // 2), 0xFF, dtype=torch.uint8)
    scales = torch.empty(B * G, dtype=torch.float32)
    for b in range(B):
        L = int(min(max(int(seq_lens[b]), 0), T_cap))
        for g in range(G):
            slab = x[b, g, :L]
            amax = float(slab.abs().max()) if L > 0 else 0.0
            s = float(torch.tensor(amax / INT4_MAX if amax > 0 else 1.0, dtype=torch.float32))
            scales[b * G + g] = s
            code = torch.round(slab / s).clamp(-8, 7).to(torch.int32) + 8
            packed[b, g, :L] = (code[:, 0::2] | (code[:, 1::2] << 4)).to(torch.uint8)
    return packed, scales


def make_decode(B, H, G, D, seq_lens, T_cap=None, q_dtype=BF16, kv_dtype=BF16, seed=0,
                name="decode", scale=None, poison=True) -> DecodeCase:
    """Decode inputs. ``seq_lens`` is an int (same length for every sequence), a
    list, or the string ``"uniform:lo:hi"`` for lengths drawn uniformly from
    [lo, hi] inclusive (drawn first, before Q, K and V)."""
    g = _gen(seed)
    if isinstance(seq_lens, str) and seq_lens.startswith("uniform:"):
        _, lo, hi = seq_lens.split(":")
        lens = torch.randint(int(lo), int(hi) + 1, (B,), generator=g).to(torch.int32)
    elif isinstance(seq_lens, int):
        lens = torch.full((B,), seq_lens, dtype=torch.int32)
    else:
        lens = torch.tensor(list(seq_lens), dtype=torch.int32)
        assert lens.numel() == B
    if T_cap is None:
        T_cap = max(int(lens.max()), 1)
    q = _randn((B, H, D), g)
    k = _randn((B, G, T_cap, D), g)
    v = _randn((B, G, T_cap, D), g)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    k_scale = v_scale = None
    if kv_dtype == FP8:
        k_st, k_scale = quantize_fp8_slabs(k, lens)
        v_st, v_scale = quantize_fp8_slabs(v, lens)
    elif kv_dtype == INT4:
        k_st, k_scale = quantize_int4_slabs(k, lens)
        v_st, v_scale = quantize_int4_slabs(v, lens)
    else:
        if poison:
            for b in range(B):
                L = int(min(max(int(lens[b]), 0), T_cap))
                k[b, :, L:] = float("nan")
                v[b, :, L:] = float("nan")
        k_st = k.to(_TORCH_DTYPE[kv_dtype])
        v_st = v.to(_TORCH_DTYPE[kv_dtype])
    return DecodeCase(name=name, q=q.to(_TORCH_DTYPE[q_dtype]), k_cache=k_st, v_cache=v_st,
                      seq_lens=lens, scale=float(scale), q_dtype=q_dtype, kv_dtype=kv_dtype,
                      k_scale=k_scale, v_scale=v_scale)


@dataclass
class PagedDecodeCase:
    """A decode case whose cache rows live in pages: row t of (b, g) is row t % page_size of
    page block_table[b, t // page_size] of the pools [num_pages, G, page_size, D]."""

    name: str
    q: torch.Tensor            # [B, H, D]
    k_pages: torch.Tensor      # [num_pages, G, page_size, D] kv_dtype
    v_pages: torch.Tensor
    block_table: torch.Tensor  # [B, pages_per_seq] int32
    seq_lens: torch.Tensor     # [B] int32
    scale: float
    q_dtype: str
    kv_dtype: str
    k_scale: Optional[torch.Tensor] = None   # [B*G] float32, fp8 only
    v_scale: Optional[torch.Tensor] = None

    @property
    def B(self): return self.q.shape[0]
    @property
    def H(self): return self.q.shape[1]
    @property
    def D(self): return self.q.shape[2]
    @property
    def G(self): return self.k_pages.shape[1]
    @property
    def page_size(self): return self.k_pages.shape[2]
    @property
    def num_pages(self): return self.k_pages.shape[0]
    @property
    def pages_per_seq(self): return self.block_table.shape[1]
    @property
    def T_cap(self): return self.pages_per_seq * self.page_size


def _page_pools(k_cache, v_cache, page_size: int, seed: int, spare_pages: Optional[int]):
    """Scatter caches [B, G, T_cap, D] into shuffled pages: returns (k_pool, v_pool, table)."""
    B, G, T_cap, D = k_cache.shape
    pps = -(-T_cap // page_size)
    spare = B if spare_pages is None else spare_pages
    num_pages = B * pps + spare
    perm = torch.randperm(num_pages, generator=_gen(seed))
    table = perm[:B * pps].reshape(B, pps).to(torch.int32)

    def scatter(cache):
        raw = cache.view(torch.uint8) if cache.dtype == torch.float8_e4m3fn else cache
        pool = torch.empty((num_pages, G, page_size, D), dtype=raw.dtype)
        if raw.dtype == torch.uint8:
            pool.fill_(0x7F)
        else:
            pool.fill_(float("nan"))
        for b in range(B):
            for p in range(pps):
                rows = raw[b, :, p * page_size:(p + 1) * page_size]
                pool[int(table[b, p]), :, :rows.shape[1]] = rows
        return pool.view(torch.float8_e4m3fn) if cache.dtype == torch.float8_e4m3fn else pool

    return scatter(k_cache), scatter(v_cache), table


def make_paged(case: DecodeCase, page_size: int, seed: int = 0, spare_pages: Optional[int] = None,
               name: Optional[str] = None) -> PagedDecodeCase:
    """Scatter a contiguous decode case into shuffled pages of ``page_size`` rows.

    pages_per_seq = ceil(T_cap / page_size); the logical cache is padded to that many whole
    pages with poison (NaN, or the fp8 NaN code); ``spare_pages`` (default B) extra pages, all
    poison, join the pool. A ``torch.randperm`` of the pool (generator seeded with ``seed``)
    gives the physical page of each (sequence, logical page). Scales are unchanged."""
    kp, vp, table = _page_pools(case.k_cache, case.v_cache, page_size, seed, spare_pages)
    return PagedDecodeCase(name=name or f"{case.name}_paged{page_size}", q=case.q, k_pages=kp, v_pages=vp,
                           block_table=table, seq_lens=case.seq_lens, scale=case.scale, q_dtype=case.q_dtype,
                           kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)


@dataclass
class ChunkCase:
    """Prefill of a chunk of Tq query positions against a cache: query i of sequence b sits at
    position seq_lens[b] - Tq + i; the cache already holds the chunk's own keys and values."""

    name: str
    q: torch.Tensor          # [B, H, Tq, D]
    k_cache: torch.Tensor    # [B, G, T_cap, D]
    v_cache: torch.Tensor
    seq_lens: torch.Tensor   # [B] int32, valid cache rows (chunk included)
    scale: float
    causal: bool
    dtype: str                                # q's dtype
    kv_dtype: str = BF16
    k_scale: Optional[torch.Tensor] = None    # [B*G] float32, fp8 only
    v_scale: Optional[torch.Tensor] = None

    @property
    def B(self): return self.q.shape[0]
    @property
    def H(self): return self.q.shape[1]
    @property
    def Tq(self): return self.q.shape[2]
    @property
    def D(self): return self.q.shape[3]
    @property
    def G(self): return self.k_cache.shape[1]
    @property
    def T_cap(self): return self.k_cache.shape[2]


@dataclass
class PagedChunkCase:
    """A chunk case whose cache rows live in pages (layout as for PagedDecodeCase)."""

    name: str
    q: torch.Tensor            # [B, H, Tq, D]
    k_pages: torch.Tensor      # [num_pages, G, page_size, D]
    v_pages: torch.Tensor
    block_table: torch.Tensor  # [B, pages_per_seq] int32
    seq_lens: torch.Tensor     # [B] int32
    scale: float
    causal: bool
    dtype: str
    kv_dtype: str
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    @property
    def B(self): return self.q.shape[0]
    @property
    def H(self): return self.q.shape[1]
    @property
    def Tq(self): return self.q.shape[2]
    @property
    def D(self): return self.q.shape[3]
    @property
    def G(self): return self.k_pages.shape[1]
    @property
    def page_size(self): return self.k_pages.shape[2]
    @property
    def pages_per_seq(self): return self.block_table.shape[1]
    @property
    def T_cap(self): return self.pages_per_seq * self.page_size


def make_paged_chunk(case, page_size: int, seed: int = 0, spare_pages: Optional[int] = None,
                     name: Optional[str] = None) -> PagedChunkCase:
    """Scatter a contiguous ChunkCase's caches into shuffled pages, as make_paged does."""
    kp, vp, table = _page_pools(case.k_cache, case.v_cache, page_size, seed, spare_pages)
    return PagedChunkCase(name=name or f"{case.name}_paged{page_size}", q=case.q, k_pages=kp, v_pages=vp,
                          block_table=table, seq_lens=case.seq_lens, scale=case.scale, causal=case.causal,
                          dtype=case.dtype, kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)


def make_chunk(B, H, G, D, Tq, seq_lens, T_cap=None, dtype=BF16, causal=True, seed=0, name="chunk",
               scale=None, kv_dtype=None) -> ChunkCase:
    """Chunked-prefill inputs. Draw order: Q [B,H,Tq,D], then K and V over the whole cache
    [B,G,T_cap,D]; cache rows at or beyond seq_lens[b] are NaN. kv_dtype FP8 (with bf16 q)
    stores the caches as E4M3FN codes with per-(b, g) scales, as in make_decode."""
    g = _gen(seed)
    lens = torch.tensor(list(seq_lens) if not isinstance(seq_lens, int) else [seq_lens] * B, dtype=torch.int32)
    if T_cap is None:
        T_cap = max(int(lens.max()), 1)
    q = _randn((B, H, Tq, D), g)
    k = _randn((B, G, T_cap, D), g)
    v = _randn((B, G, T_cap, D), g)
    for b in range(B):
        L = int(min(max(int(lens[b]), 0), T_cap))
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("nan")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    td = _TORCH_DTYPE[dtype]
    if kv_dtype == FP8:
        kc, ks = quantize_fp8_slabs(k, lens)
        vc, vs = quantize_fp8_slabs(v, lens)
        return ChunkCase(name=name, q=q.to(td), k_cache=kc, v_cache=vc, seq_lens=lens, scale=float(scale),
                         causal=causal, dtype=dtype, kv_dtype=FP8, k_scale=ks, v_scale=vs)
    return ChunkCase(name=name, q=q.to(td), k_cache=k.to(td), v_cache=v.to(td), seq_lens=lens, scale=float(scale),
                     causal=causal, dtype=dtype, kv_dtype=dtype)


def make_prefill(B, H, G, D, T, dtype=BF16, causal=True, seed=0, name="prefill",
                 scale=None) -> PrefillCase:
    g = _gen(seed)
    q = _randn((B, H, T, D), g)
    k = _randn((B, G, T, D), g)
    v = _randn((B, G, T, D), g)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    td = _TORCH_DTYPE[dtype]
    return PrefillCase(name=name, q=q.to(td), k=k.to(td), v=v.to(td), scale=float(scale),
                       causal=causal, dtype=dtype)


# --------------------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------------------

TOY_PREFILL_T = 5
TOY_DECODE_LENS = (6, 7)


def toy_tokens(seed=0):
    """The 12-dim, 4-head toy of the tutorial pages: H=4, G=2, head dim 3, batch 1.

    Seven tokens are drawn at once (q [1,4,7,3], k/v [1,2,7,3], fp32): the prefill
    uses the first five, the two decode steps then append tokens 6 and 7.
    """
    g = _gen(seed)
    q = _randn((1, 4, 7, 3), g)
    k = _randn((1, 2, 7, 3), g)
    v = _randn((1, 2, 7, 3), g)
    return q, k, v


def toy_prefill(seed=0) -> PrefillCase:
    q, k, v = toy_tokens(seed)
    T = TOY_PREFILL_T
    return PrefillCase(name="toy_prefill", q=q[:, :, :T].contiguous(), k=k[:, :, :T].contiguous(),
                       v=v[:, :, :T].contiguous(), scale=1.0 / math.sqrt(3.0), causal=True, dtype=F32)


def toy_decode_steps(seed=0, T_cap=8):
    """The two decode steps after the toy prefill: cache lengths 6 and 7."""
    q, k, v = toy_tokens(seed)
    steps = []
    for L in TOY_DECODE_LENS:
        kc = torch.full((1, 2, T_cap, 3), float("nan"))
        vc = torch.full((1, 2, T_cap, 3), float("nan"))
        kc[:, :, :L] = k[:, :, :L]
        vc[:, :, :L] = v[:, :, :L]
        steps.append(DecodeCase(name=f"toy_decode_L{L}", q=q[:, :, L - 1].contiguous(), k_cache=kc,
                                v_cache=vc, seq_lens=torch.tensor([L], dtype=torch.int32),
                                scale=1.0 / math.sqrt(3.0), q_dtype=F32, kv_dtype=F32))
    return steps


def llama7b_gqa8_decode(seed=0) -> DecodeCase:
    """Llama-2-7B-shaped GQA-8 decode: B1 H32 G8 D128, cache of 2048 tokens, bf16."""
    return make_decode(1, 32, 8, 128, 2048, T_cap=2048, seed=seed, name="llama7b_gqa8_decode_L2048")


def llama70b_ragged_decode(seed=0) -> DecodeCase:
    """Llama-2-70B-shaped decode: B16 H64 G8 D128, lengths ~ U[1024, 4096], T_cap 4096."""
    return make_decode(16, 64, 8, 128, "uniform:1024:4096", T_cap=4096, seed=seed,
                       name="llama70b_gqa8_decode_B16_ragged")


def causal_prefill_2048(seed=0) -> PrefillCase:
    """Causal GQA prefill: B4 H32 G8 D128 T2048, bf16."""
    return make_prefill(4, 32, 8, 128, 2048, seed=seed, name="gqa8_causal_prefill_B4_T2048")


def mqa_fp8_long_decode(seed=0) -> DecodeCase:
    """Long-context MQA decode: B8 H32 G1 D128, 32768 cached tokens, fp8-E4M3FN KV."""
    return make_decode(8, 32, 1, 128, 32768, T_cap=32768, kv_dtype=FP8, seed=seed,
                       name="mqa_fp8_decode_B8_L32768")


def mqa_int4_long_decode(seed=0) -> DecodeCase:
    """The long-context MQA decode with an INT4 cache: B8 H32 G1 D128, 32768 tokens."""
    return make_decode(8, 32, 1, 128, 32768, T_cap=32768, kv_dtype=INT4, seed=seed, name="mqa_int4_decode_B8_L32768")


def llama70b_ragged_decode_int4(seed=0) -> DecodeCase:
    """The ragged Llama-2-70B-shaped decode with an INT4 cache."""
    return make_decode(16, 64, 8, 128, "uniform:1024:4096", T_cap=4096, kv_dtype=INT4, seed=seed,
                       name="llama70b_gqa8_decode_B16_ragged_int4")


def chunked_prefill_512_of_4096(seed=0) -> ChunkCase:
    """Chunked prefill: B4 H32 G8 D128, the last 512 positions of 4096-token sequences against
    the cache holding the first 3584 (and the chunk's own rows), causal, bf16."""
    return make_chunk(4, 32, 8, 128, 512, 4096, T_cap=4096, seed=seed, name="gqa8_chunked_prefill_B4_Tq512_L4096")


def chunked_prefill_512_of_4096_fp8(seed=0) -> ChunkCase:
    """The chunked prefill against an fp8-E4M3FN cache (per-(sequence, KV head) scales)."""
    return make_chunk(4, 32, 8, 128, 512, 4096, T_cap=4096, seed=seed, name="gqa8_chunked_prefill_B4_Tq512_L4096_fp8",
                      kv_dtype=FP8)


def narrow_group_decode(H: int, seed=0) -> DecodeCase:
    """The Llama-2-7B-shaped decode with H query heads over its 8 KV heads (R = H / 8 query heads
    per KV head): B1 D128, 2048 cached tokens, bf16. For the comparison of the vector-ALU and
    matrix-core decode kernels at narrow groups (R = 2, 4, 8)."""
    return make_decode(1, H, 8, 128, 2048, T_cap=2048, seed=seed, name=f"gqa_decode_B1_H{H}_G8_L2048")


WORKLOADS = {
    "toy": None,  # prefill + two decode steps; see toy_prefill / toy_decode_steps
    "llama7b_gqa8_decode_L2048": llama7b_gqa8_decode,
    "llama70b_gqa8_decode_B16_ragged": llama70b_ragged_decode,
    "gqa8_causal_prefill_B4_T2048": causal_prefill_2048,
    "mqa_fp8_decode_B8_L32768": mqa_fp8_long_decode,
}
