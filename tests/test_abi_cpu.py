"""The C ABI of libgqa.so on the host (no GPU): exported symbols, the options struct,
status strings, the split/workspace queries, and argument validation, which runs
before any HIP call and so can be exercised without a device."""

import ctypes
import os
import re

import pytest

import grouped_query_attention_decode_amd as gqa

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
FAKE = 0x10000  # never dereferenced: every case below is rejected on the host


@pytest.fixture(scope="module")
def lib():
    return gqa.library()


def declared_functions():
    """Every function that a header under include/ declares."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names.update(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gqa_decode", "gqa_prefill", "gqa_decode_workspace_size", "gqa_status_string",
            "gqa_opts_init", "gqa_decode_num_splits", "gqa_decode_noalloc", "gqa_hbm_stream_read"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libgqa.so does not export {n}"


def test_opts_layout_matches_header(lib):
    o = gqa.GqaOpts()
    lib.gqa_opts_init(ctypes.byref(o))
    assert o.struct_size == ctypes.sizeof(gqa.GqaOpts) == 80
    assert (o.q_dtype, o.kv_dtype, o.kv_capacity, o.num_splits, o.path) == (1, 1, 0, 0, 0)
    assert not o.k_scale and not o.v_scale and not o.workspace and o.workspace_bytes == 0
    assert not o.k_new and not o.v_new


def test_status_strings():
    assert gqa.status_string(0) == "GQA_OK"
    assert gqa.status_string(1) == "GQA_ERR_INVALID_ARG"
    assert gqa.status_string(2) == "GQA_ERR_UNSUPPORTED"
    assert gqa.status_string(3) == "GQA_ERR_WORKSPACE"
    assert gqa.status_string(4) == "GQA_ERR_HIP"
    assert gqa.status_string(99) == "GQA_ERR_UNKNOWN"


def _decode(lib, B=2, H=8, G=2, D=128, scale=0.1, ptrs=(FAKE,) * 5, **opt):
    fields = dict(kv_capacity=64)
    fields.update(opt)
    o = gqa.new_opts(**fields)
    return lib.gqa_decode(*ptrs, B, H, G, D, scale, None, ctypes.byref(o))


def _prefill(lib, B=1, T=16, H=8, G=2, D=128, scale=0.1, causal=1, ptrs=(FAKE,) * 4, opts=True, **opt):
    o = gqa.new_opts(**opt)
    return lib.gqa_prefill(*ptrs, B, T, H, G, D, scale, causal, None, ctypes.byref(o) if opts else None)


INV, UNS, WSP = 1, 2, 3


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=(0, FAKE, FAKE, FAKE, FAKE)), INV),
    (dict(ptrs=(FAKE, 0, FAKE, FAKE, FAKE)), INV),
    (dict(ptrs=(FAKE, FAKE, 0, FAKE, FAKE)), INV),
    (dict(ptrs=(FAKE, FAKE, FAKE, 0, FAKE)), INV),
    (dict(ptrs=(FAKE, FAKE, FAKE, FAKE, 0)), INV),
    (dict(B=0), INV), (dict(H=0), INV), (dict(G=0), INV), (dict(D=0), INV),
    (dict(H=8, G=3), INV),
    (dict(D=257), INV),
    (dict(kv_capacity=0), INV),
    (dict(scale=float("nan")), INV), (dict(scale=float("inf")), INV),
    (dict(num_splits=-1), INV), (dict(num_splits=1025), INV),
    (dict(path=4), INV), (dict(path=-1), INV),
    (dict(layout=3), INV), (dict(layout=-1), INV),
    (dict(layout=2, num_splits=4), INV),                 # flat layout chooses its own ranges
    (dict(layout=2, path=1), UNS),                       # flat layout: matrix-core path only
    (dict(layout=2, q_dtype=0, kv_dtype=0), UNS),
    (dict(q_dtype=7), INV), (dict(kv_dtype=9), INV),
    (dict(q_dtype=0, kv_dtype=1), UNS),        # f32 q with bf16 cache
    (dict(q_dtype=1, kv_dtype=0), UNS),
    (dict(q_dtype=2, kv_dtype=2), UNS),        # fp8 q
    (dict(q_dtype=0, kv_dtype=2, k_scale=FAKE, v_scale=FAKE), UNS),
    (dict(kv_dtype=2), INV),                   # fp8 without scales
    (dict(kv_dtype=2, k_scale=FAKE), INV),
    (dict(q_dtype=0, kv_dtype=0, D=3, path=3), UNS),   # matrix-core path needs bf16 q and D=128
    (dict(q_dtype=0, kv_dtype=0, D=3, path=2), UNS),   # vector path needs bf16 and D=128
    (dict(k_new=FAKE), INV), (dict(v_new=FAKE), INV),  # cache append needs both rows
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=16), WSP),
    (dict(num_splits=4, workspace=FAKE + 4, workspace_bytes=1 << 30), INV),  # misaligned workspace
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def _decode_noalloc(lib, B=2, H=8, G=2, D=128, scale=0.1, ptrs=(FAKE,) * 5, **opt):
    fields = dict(kv_capacity=64)
    fields.update(opt)
    o = gqa.new_opts(**fields)
    return lib.gqa_decode_noalloc(*ptrs, B, H, G, D, scale, None, ctypes.byref(o))


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=(0, FAKE, FAKE, FAKE, FAKE)), INV),
    (dict(H=8, G=3), INV),
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=1 << 30), INV),   # the variant takes no workspace
    (dict(B=70000, H=1, G=1, num_splits=2), WSP),                         # more counters than the scratch holds
    (dict(B=64, H=64, G=8, kv_capacity=32768, num_splits=64), WSP),       # split partials beyond 32 MiB
])
def test_decode_noalloc_rejects(lib, kw, code):
    """The allocation-free variant checks its limits on the host, before any HIP call."""
    assert _decode_noalloc(lib, **kw) == code


def test_decode_requires_opts(lib):
    assert lib.gqa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 128, 0.1, None, None) == INV


def test_decode_short_struct_keeps_defaults(lib):
    # A caller built against the layout without the append fields passes a shorter struct:
    # the fields past struct_size are not read (here they hold an invalid lone k_new). The
    # undersized workspace makes both calls fail on the host, at different checks.
    o = gqa.new_opts(kv_capacity=64, k_new=FAKE, num_splits=4, workspace=FAKE, workspace_bytes=16)
    o.struct_size = gqa.GqaOpts.k_new.offset
    assert lib.gqa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 128, 0.1, None, ctypes.byref(o)) == WSP
    o.struct_size = ctypes.sizeof(gqa.GqaOpts)
    assert lib.gqa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 128, 0.1, None, ctypes.byref(o)) == INV


def test_decode_short_struct(lib):
    o = gqa.new_opts(kv_capacity=64)
    o.struct_size = 8
    assert lib.gqa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 128, 0.1, None, ctypes.byref(o)) == INV


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=(0, FAKE, FAKE, FAKE)), INV),
    (dict(ptrs=(FAKE, FAKE, FAKE, 0)), INV),
    (dict(B=0), INV), (dict(T=0), INV), (dict(H=6, G=4), INV), (dict(D=300), INV),
    (dict(causal=2), INV), (dict(causal=-1), INV),
    (dict(scale=float("nan")), INV),
    (dict(q_dtype=1, kv_dtype=0), UNS),
    (dict(q_dtype=2, kv_dtype=2), UNS),
    (dict(path=2), UNS),                        # no vector-ALU prefill
    (dict(q_dtype=0, kv_dtype=0, path=3), UNS), # matrix-core prefill is bf16 only
    (dict(path=5), INV),
])
def test_prefill_rejects(lib, kw, code):
    assert _prefill(lib, **kw) == code


def test_split_queries(lib):
    # one split needs no workspace
    assert gqa.decode_workspace_size(1, 4, 2, 3, 8, "f32", 1) == 0
    assert gqa.decode_num_splits(1, 4, 2, 3, 8, "f32", 1) == 1
    # forced split counts are honoured, even beyond the number of keys (empty splits)
    assert gqa.decode_num_splits(2, 8, 2, 64, 10, "bf16", 7) == 7
    assert gqa.decode_num_splits(2, 8, 2, 64, 10, "bf16", 64) == 64
    S = 5
    up = lambda x: ((x + 255) // 256) * 256
    counters = up(2 * 2 * 4)            # one int per (sequence, KV head)
    acc = up(2 * 8 * S * 64 * 4)        # [B*H][S][D] fp32
    assert gqa.decode_workspace_size(2, 8, 2, 64, 100, "bf16", S) == counters + acc + 2 * 8 * S * 2 * 4
    # automatic choice: between 1 and the number of keys, deterministic
    for args in [(1, 32, 8, 128, 2048, "bf16"), (16, 64, 8, 128, 4096, "bf16"), (8, 32, 1, 128, 32768, "fp8_e4m3fn"),
                 (1, 4, 2, 3, 7, "f32")]:
        s = gqa.decode_num_splits(*args)
        assert 1 <= s <= args[4] and s == gqa.decode_num_splits(*args)
    # small INT4 rows: the ranges still give every one of the 256 CUs a workgroup (8 x 32)
    assert gqa.decode_num_splits(8, 32, 1, 128, 32768, "int4") == 32
    # ... but no range shorter than one 64-key tile
    assert gqa.decode_num_splits(1, 32, 1, 128, 640, "int4") == 10
    # invalid sizes
    assert gqa.decode_num_splits(0, 8, 2, 64, 10) == 0
    assert gqa.decode_workspace_size(1, 6, 4, 64, 10) == 2 ** 64 - 1


def _paged(lib, B=2, H=8, G=2, D=128, scale=0.1, page_size=16, pps=4, num_pages=8,
           ptrs=(FAKE,) * 6, **opt):
    o = gqa.new_opts(**opt)
    return lib.gqa_decode_paged(*ptrs, B, H, G, D, scale, page_size, pps, num_pages, None, ctypes.byref(o))


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=(FAKE, FAKE, FAKE, 0, FAKE, FAKE)), INV),     # no block table
    (dict(ptrs=(FAKE, FAKE, FAKE, FAKE, 0, FAKE)), INV),
    (dict(page_size=8), INV), (dict(page_size=48), INV), (dict(page_size=0), INV), (dict(page_size=1 << 21), INV),
    (dict(pps=0), INV), (dict(num_pages=0), INV),
    (dict(page_size=1 << 20, pps=1 << 12), INV),              # capacity beyond 2^31 rows
    (dict(path=1), UNS), (dict(path=2), UNS),                 # matrix-core family only
    (dict(q_dtype=0, kv_dtype=0), UNS), (dict(D=64), UNS),
    (dict(k_new=FAKE), INV),
    (dict(kv_dtype=2), INV),                                  # fp8 without scales
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=16), WSP),
])
def test_decode_paged_rejects(lib, kw, code):
    assert _paged(lib, **kw) == code


def test_decode_paged_ignores_kv_capacity(lib):
    # kv_capacity comes from the page geometry: an unset opts.kv_capacity (0) is fine, and the
    # call proceeds to the workspace check.
    assert _paged(lib, kv_capacity=0, num_splits=4, workspace=FAKE, workspace_bytes=16) == WSP


def _pchunk(lib, B=2, Tq=16, H=8, G=2, D=128, scale=0.1, causal=1, page_size=16, pps=4, num_pages=8,
            ptrs=(FAKE,) * 6, **opt):
    o = gqa.new_opts(**opt)
    return lib.gqa_prefill_paged(*ptrs, B, Tq, H, G, D, scale, causal, page_size, pps, num_pages, None,
                                 ctypes.byref(o))


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=(FAKE, FAKE, FAKE, 0, FAKE, FAKE)), INV),     # no block table
    (dict(ptrs=(FAKE, FAKE, FAKE, FAKE, 0, FAKE)), INV),     # no seq_lens
    (dict(page_size=8), INV), (dict(page_size=48), INV), (dict(page_size=1 << 21), INV),
    (dict(pps=0), INV), (dict(num_pages=0), INV), (dict(Tq=0), INV), (dict(causal=3), INV),
    (dict(page_size=1 << 20, pps=1 << 12), INV),              # capacity beyond 2^31 rows
    (dict(path=1), UNS), (dict(path=2), UNS),                 # matrix-core family only
    (dict(q_dtype=0, kv_dtype=0), UNS), (dict(D=64), UNS), (dict(H=130, G=2), UNS),
    (dict(kv_dtype=2), INV),                                  # fp8 without scales
    (dict(kv_dtype=3), UNS),                                  # no INT4 chunks
])
def test_prefill_paged_rejects(lib, kw, code):
    assert _pchunk(lib, **kw) == code


def _chunk(lib, B=2, Tq=16, H=8, G=2, D=128, scale=0.1, causal=1, ptrs=(FAKE,) * 5, opts=True, **opt):
    fields = dict(kv_capacity=64)
    fields.update(opt)
    o = gqa.new_opts(**fields)
    return lib.gqa_prefill_cached(*ptrs, B, Tq, H, G, D, scale, causal, None, ctypes.byref(o) if opts else None)


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=(FAKE, FAKE, FAKE, 0, FAKE)), INV),      # seq_lens required
    (dict(ptrs=(0, FAKE, FAKE, FAKE, FAKE)), INV),
    (dict(opts=False), INV),                            # opts carries kv_capacity
    (dict(kv_capacity=0), INV), (dict(Tq=0), INV), (dict(B=0), INV),
    (dict(H=6, G=4), INV), (dict(D=300), INV),
    (dict(causal=2), INV), (dict(scale=float("nan")), INV),
    (dict(q_dtype=0, kv_dtype=1), UNS), (dict(q_dtype=2, kv_dtype=2), UNS),
    (dict(kv_dtype=2), INV),                            # fp8 without scales
    (dict(path=2), UNS),                                # no vector-ALU prefill
    (dict(q_dtype=0, kv_dtype=0, path=3), UNS),         # matrix cores: bf16 only
    (dict(H=130, G=2, path=3), UNS),                    # matrix cores: R up to 64
    (dict(D=64, path=3), UNS),                          # matrix cores: D = 128
    (dict(path=7), INV),
])
def test_prefill_cached_rejects(lib, kw, code):
    assert _chunk(lib, **kw) == code


@pytest.mark.parametrize("buf,nbytes,sink", [
    (0, 1 << 20, FAKE), (FAKE, 1 << 20, 0), (FAKE, 0, FAKE), (FAKE, 1000, FAKE), (FAKE + 8, 1 << 20, FAKE),
])
def test_stream_read_rejects(lib, buf, nbytes, sink):
    """The streaming-read measurement call checks its arguments before any HIP call."""
    assert lib.gqa_hbm_stream_read(buf, nbytes, sink, None) == INV


def test_timeline_calls_in_the_library_proper(lib):
    """The per-workgroup timeline exists only in the diagnostic build: the library proper says so
    (and refuses a null destination first), without touching the device."""
    import ctypes
    buf = ctypes.create_string_buffer(64)
    assert lib.gqa_timeline_read(None, 64) == INV
    assert lib.gqa_timeline_read(ctypes.addressof(buf), 64) == UNS
    assert lib.gqa_timeline_clear() == UNS
