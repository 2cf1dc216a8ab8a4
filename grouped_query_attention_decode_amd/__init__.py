"""Python binding of libgqa.so: grouped-query attention decode and prefill on MI355X.

Argument marshalling only. Every step of the computation runs in the HIP kernels of
libgqa.so, reached through its C ABI (include/gqa.h); torch supplies device memory and
the current stream. There is no fallback: if the library is not built, or the device is
not gfx950, calls raise.

    decode(q, k_cache, v_cache, seq_lens, ...)   q [B,H,D], caches [B,G,T_cap,D]
    decode_paged(q, k_pages, v_pages, block_table, seq_lens, ...)
                                                 pools [num_pages,G,page_size,D], table [B,pages_per_seq]
    prefill(q, k, v, causal=True, ...)           q [B,H,T,D], k/v [B,G,T,D]
    prefill_cached(q, k_cache, v_cache, seq_lens, causal=True, ...)
                                                 q [B,H,Tq,D] against caches [B,G,T_cap,D]
"""

from __future__ import annotations

import ctypes
import math
import os

import torch  # loads torch's HIP runtime first, so libgqa.so binds to that same runtime

__all__ = ["decode", "decode_noalloc", "decode_paged", "prefill", "prefill_cached", "prefill_paged", "decode_num_splits", "decode_workspace_size", "hbm_stream_read", "status_string",
           "GqaError", "library", "LIBRARY_PATH", "GqaOpts", "PATHS", "DTYPES", "LAYOUTS"]

# The library built in this package; GQA_LIBRARY_PATH may name another build of the same sources
# (the host-sanitized one for the CPU tests of the C ABI).
LIBRARY_PATH = os.environ.get("GQA_LIBRARY_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                                  "libgqa.so")

GQA_OK = 0
DTYPES = {"f32": 0, "bf16": 1, "fp8_e4m3fn": 2, "int4": 3}
PATHS = {"auto": 0, "generic": 1, "valu": 2, "mfma": 3}
LAYOUTS = {"auto": 0, "uniform": 1, "flat": 2}
_TORCH_TO_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2, torch.uint8: 3}  # uint8 = packed INT4


class GqaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} ({status})")


class GqaOpts(ctypes.Structure):
    """Mirror of gqa_opts in include/gqa.h."""

    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
    ]


_lib = None


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def library() -> ctypes.CDLL:
    """Load libgqa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(f"{LIBRARY_PATH} is not built: run "
                           "`python -m grouped_query_attention_decode_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.gqa_opts_init.argtypes = [ctypes.POINTER(GqaOpts)]
    lib.gqa_opts_init.restype = None
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp, ctypes.POINTER(GqaOpts)]
    lib.gqa_decode.restype = i
    lib.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp, ctypes.POINTER(GqaOpts)]
    lib.gqa_decode_noalloc.restype = i
    lib.gqa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp, ctypes.POINTER(GqaOpts)]
    lib.gqa_decode_paged.restype = i
    lib.gqa_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, vp, ctypes.POINTER(GqaOpts)]
    lib.gqa_prefill_cached.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, ctypes.POINTER(GqaOpts)]
    lib.gqa_prefill_cached.restype = i
    lib.gqa_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp,
                                      ctypes.POINTER(GqaOpts)]
    lib.gqa_prefill_paged.restype = i
    lib.gqa_prefill.restype = i
    lib.gqa_decode_num_splits.argtypes = [i] * 7
    lib.gqa_decode_num_splits.restype = i
    lib.gqa_decode_workspace_size.argtypes = [i] * 7
    lib.gqa_decode_workspace_size.restype = ctypes.c_size_t
    lib.gqa_hbm_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.gqa_hbm_stream_read.restype = i
    lib.gqa_timeline_read.argtypes = [vp, ctypes.c_size_t]
    lib.gqa_timeline_read.restype = i
    lib.gqa_timeline_clear.argtypes = []
    lib.gqa_timeline_clear.restype = i
    lib.gqa_status_string.argtypes = [i]
    lib.gqa_status_string.restype = ctypes.c_char_p
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped ({sorted(runtimes)}); streams would not be shared")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().gqa_status_string(int(status)).decode()


def new_opts(**fields) -> GqaOpts:
    o = GqaOpts()
    library().gqa_opts_init(ctypes.byref(o))
    for k, v in fields.items():
        setattr(o, k, v)
    return o


def _kv_code(kv_dtype) -> int:
    return kv_dtype if isinstance(kv_dtype, int) else DTYPES[kv_dtype]


def hbm_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of the device tensor ``buf`` once (gqa_hbm_stream_read, a measurement
    aid: the plain streaming-read rate, and the pass that evicts the Infinity Cache). ``sink`` is
    a device int32 tensor of at least 1024 elements."""
    _need_cuda(buf, "buf")
    _need_cuda(sink, "sink", buf.device)
    if sink.dtype != torch.int32 or sink.numel() < 1024:
        raise ValueError("sink must be a device int32 tensor of at least 1024 elements")
    st = library().gqa_hbm_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                       _stream_handle(stream, buf.device))
    if st != GQA_OK:
        raise GqaError(st, "gqa_hbm_stream_read")


TIMELINE_WORKGROUPS, TIMELINE_SLOTS = 4096, 32


def timeline_clear() -> None:
    """Zero the per-workgroup timeline (gqa_timeline_clear; the timeline build only)."""
    st = library().gqa_timeline_clear()
    if st != GQA_OK:
        raise GqaError(st, "gqa_timeline_clear")


def timeline_read():
    """The per-workgroup timeline of the decode kernels since the last clear, as a numpy uint64
    array [4096 workgroups, 32 slots] (gqa_timeline_read; the timeline build only; the slots are
    described in include/gqa_measure.h)."""
    import numpy as np
    buf = np.zeros((TIMELINE_WORKGROUPS, TIMELINE_SLOTS), dtype=np.uint64)
    st = library().gqa_timeline_read(buf.ctypes.data, buf.nbytes)
    if st != GQA_OK:
        raise GqaError(st, "gqa_timeline_read")
    return buf


def decode_num_splits(B, H, G, D, kv_capacity, kv_dtype="bf16", num_splits=0) -> int:
    """KV splits gqa_decode uses for these sizes (0 for invalid sizes)."""
    return int(library().gqa_decode_num_splits(B, H, G, D, kv_capacity, _kv_code(kv_dtype), num_splits))


def decode_workspace_size(B, H, G, D, kv_capacity, kv_dtype="bf16", num_splits=0) -> int:
    """Device workspace bytes gqa_decode needs for these sizes (0: none)."""
    return int(library().gqa_decode_workspace_size(B, H, G, D, kv_capacity, _kv_code(kv_dtype), num_splits))


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype not in _TORCH_TO_CODE:
        raise TypeError(f"{what}: unsupported dtype {t.dtype}")
    return _TORCH_TO_CODE[t.dtype]


def _need_cuda(t: torch.Tensor, what: str, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, not on q's device {device}")


def _check_out(out, q, what="out"):
    """A caller's output must have q's device, dtype and shape: the kernels write q.numel()
    elements of q's type to it."""
    _need_cuda(out, what, q.device)
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"{what} must be {tuple(q.shape)} {q.dtype} like q, got {tuple(out.shape)} {out.dtype}")
    if out.data_ptr() == q.data_ptr():
        raise ValueError(f"{what} must not alias q")


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _on_stream(stream, make):
    """Run make() with `stream` current, so that memory it allocates belongs to that stream (the
    caching allocator then never hands it to other work while the call's kernels use it) and the
    work it enqueues (a zero fill) is ordered before those kernels."""
    if stream is None:
        return make()
    with torch.cuda.stream(stream):
        return make()


def _new_out(q, stream):
    return _on_stream(stream, lambda: torch.empty_like(q))


def _scales(o, B, G, k_scale, v_scale, device, what):
    if k_scale is None or v_scale is None:
        raise ValueError(f"{what} need k_scale and v_scale")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _need_cuda(t, n, device)
        if t.dtype != torch.float32 or t.numel() != B * G:
            raise ValueError(f"{n} must be float32 [B*G]")
    o.k_scale, o.v_scale = k_scale.data_ptr(), v_scale.data_ptr()


def _decode_opts(q, cache, B, G, D, T_cap, k_scale, v_scale, num_splits, path, layout, k_new, v_new, workspace,
                 stream):
    if path not in PATHS or layout not in LAYOUTS:
        raise ValueError(f"path must be one of {sorted(PATHS)}, layout one of {sorted(LAYOUTS)}")
    kv_code = _dtype_code(cache, "k_cache")
    o = new_opts(q_dtype=_dtype_code(q, "q"), kv_dtype=kv_code, kv_capacity=T_cap,
                 num_splits=int(num_splits), path=PATHS[path], layout=LAYOUTS[layout])
    if kv_code in (DTYPES["fp8_e4m3fn"], DTYPES["int4"]):
        _scales(o, B, G, k_scale, v_scale, q.device, "fp8 and INT4 caches")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _need_cuda(t, n, q.device)
            if t.dtype != q.dtype or tuple(t.shape) != (B, G, D):
                raise ValueError(f"{n} must be [B, G, D] = {(B, G, D)} in q's dtype")
        o.k_new, o.v_new = k_new.data_ptr(), v_new.data_ptr()
    need = decode_workspace_size(B, q.shape[1], G, D, T_cap, kv_code, int(num_splits))
    if need == (1 << 64) - 1:
        raise ValueError("decode sizes out of range")
    if workspace is not None:
        _need_cuda(workspace, "workspace", q.device)
        have = workspace.numel() * workspace.element_size()
        if have < need:
            raise ValueError(f"workspace holds {have} bytes, these sizes need {need}")
    if need > 0:
        if workspace is None:
            # Allocated and zero-filled on the call's stream: ordered before its kernels.
            workspace = _on_stream(stream, lambda: torch.zeros(need, dtype=torch.uint8, device=q.device))
        o.workspace, o.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return o, workspace


def decode(q, k_cache, v_cache, seq_lens, out=None, scale=None, k_scale=None, v_scale=None,
           num_splits=0, path="auto", workspace=None, stream=None, layout="auto", k_new=None, v_new=None):
    """Single-token GQA decode. Returns ``out`` [B, H, D] (q's dtype).

    ``layout`` ("auto", "uniform" or "flat") chooses how the key rows are spread over the
    workgroups; "flat" balances batches of unequal lengths (matrix-core path only).

    ``k_new``/``v_new`` ([B, G, D], q's dtype; both or neither) append the current token to the
    caches first: row seq_lens[b]-1 of every (b, g) with 1 <= seq_lens[b] <= T_cap receives them
    (E4M3FN codes of k_new / k_scale for fp8 caches), and the attention includes that row.

    ``workspace`` (uint8 device tensor of at least ``decode_workspace_size`` bytes) must be
    zero-filled before its first use; each completed call leaves it ready for the next.
    Without one, a zeroed workspace is allocated for this call."""
    _need_cuda(q, "q")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _need_cuda(t, n, q.device)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected q [B,H,D] and k_cache, v_cache [B,G,T_cap,D]")
    B, H, D = q.shape
    Bk, G, T_cap, Dk = k_cache.shape
    if k_cache.dtype == torch.uint8:  # packed INT4: two head dims per byte
        Dk *= 2
    if Bk != B or Dk != D or seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, caches and seq_lens (int32 [B])")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must share a dtype")
    if out is None:
        out = _new_out(q, stream)
    _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o, workspace = _decode_opts(q, k_cache, B, G, D, T_cap, k_scale, v_scale, num_splits, path, layout,
                                k_new, v_new, workspace, stream)
    st = library().gqa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                              out.data_ptr(), B, H, G, D, float(scale), _stream_handle(stream, q.device),
                              ctypes.byref(o))
    if st != GQA_OK:
        raise GqaError(st, "gqa_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, seq_lens, out, scale=None, k_scale=None, v_scale=None, num_splits=0,
                   path="auto", stream=None, layout="auto", k_new=None, v_new=None):
    """``decode`` through gqa_decode_noalloc: split partials in the library's static device
    scratch instead of a workspace, so nothing is allocated (``out`` must be given). Calls that
    overlap in time on one GPU race on that scratch; calls ordered on one stream do not."""
    _need_cuda(q, "q")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _need_cuda(t, n, q.device)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected q [B,H,D] and k_cache, v_cache [B,G,T_cap,D]")
    B, H, D = q.shape
    Bk, G, T_cap, Dk = k_cache.shape
    if k_cache.dtype == torch.uint8:
        Dk *= 2
    if Bk != B or Dk != D or seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, caches and seq_lens (int32 [B])")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must share a dtype")
    _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if path not in PATHS or layout not in LAYOUTS:
        raise ValueError(f"path must be one of {sorted(PATHS)}, layout one of {sorted(LAYOUTS)}")
    kv_code = _dtype_code(k_cache, "k_cache")
    o = new_opts(q_dtype=_dtype_code(q, "q"), kv_dtype=kv_code, kv_capacity=T_cap,
                 num_splits=int(num_splits), path=PATHS[path], layout=LAYOUTS[layout])
    if kv_code in (DTYPES["fp8_e4m3fn"], DTYPES["int4"]):
        _scales(o, B, G, k_scale, v_scale, q.device, "fp8 and INT4 caches")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _need_cuda(t, n, q.device)
            if t.dtype != q.dtype or tuple(t.shape) != (B, G, D):
                raise ValueError(f"{n} must be [B, G, D] = {(B, G, D)} in q's dtype")
        o.k_new, o.v_new = k_new.data_ptr(), v_new.data_ptr()
    st = library().gqa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                      out.data_ptr(), B, H, G, D, float(scale), _stream_handle(stream, q.device),
                                      ctypes.byref(o))
    if st != GQA_OK:
        raise GqaError(st, "gqa_decode_noalloc")
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, out=None, scale=None, k_scale=None, v_scale=None,
                 num_splits=0, path="auto", workspace=None, stream=None, layout="auto", k_new=None, v_new=None):
    """Single-token GQA decode over a paged cache. Returns ``out`` [B, H, D] (q's dtype).

    ``k_pages``/``v_pages`` [num_pages, G, page_size, D]; ``block_table`` int32 [B, pages_per_seq]:
    row t of sequence b is row t % page_size of page block_table[b, t // page_size]. The other
    arguments are those of ``decode`` (the workspace size is that of a cache of
    pages_per_seq * page_size rows)."""
    _need_cuda(q, "q")
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _need_cuda(t, n, q.device)
    if q.dim() != 3 or k_pages.dim() != 4 or k_pages.shape != v_pages.shape or block_table.dim() != 2:
        raise ValueError("expected q [B,H,D], pools [num_pages,G,page_size,D] and block_table [B,pages_per_seq]")
    B, H, D = q.shape
    num_pages, G, page_size, Dk = k_pages.shape
    if k_pages.dtype == torch.uint8:  # packed INT4
        Dk *= 2
    Bt, pages_per_seq = block_table.shape
    if Bt != B or Dk != D or block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, pools, block_table (int32) and seq_lens (int32 [B])")
    if k_pages.dtype != v_pages.dtype:
        raise TypeError("k_pages and v_pages must share a dtype")
    if out is None:
        out = _new_out(q, stream)
    _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o, workspace = _decode_opts(q, k_pages, B, G, D, pages_per_seq * page_size, k_scale, v_scale, num_splits,
                                path, layout, k_new, v_new, workspace, stream)
    st = library().gqa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                    seq_lens.data_ptr(), out.data_ptr(), B, H, G, D, float(scale), page_size,
                                    pages_per_seq, num_pages, _stream_handle(stream, q.device), ctypes.byref(o))
    if st != GQA_OK:
        raise GqaError(st, "gqa_decode_paged")
    return out


def prefill(q, k, v, out=None, scale=None, causal=True, path="auto", stream=None):
    """GQA prefill (causal by default). Returns ``out`` [B, H, T, D] (q's dtype)."""
    _need_cuda(q, "q")
    for t, n in ((k, "k"), (v, "v")):
        _need_cuda(t, n, q.device)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,H,T,D] and k, v [B,G,T,D]")
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    B, H, T, D = q.shape
    Bk, G, Tk, Dk = k.shape
    if (Bk, Tk, Dk) != (B, T, D):
        raise ValueError("shape mismatch between q and k/v")
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    if out is None:
        out = _new_out(q, stream)
    _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = new_opts(q_dtype=_dtype_code(q, "q"), kv_dtype=_dtype_code(k, "k"), path=PATHS[path])
    st = library().gqa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, T, H, G, D,
                               float(scale), int(bool(causal)), _stream_handle(stream, q.device),
                               ctypes.byref(o))
    if st != GQA_OK:
        raise GqaError(st, "gqa_prefill")
    return out


def _chunk_opts(q, cache, B, G, T_cap, k_scale, v_scale, path):
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    kv_code = _dtype_code(cache, "cache")
    o = new_opts(q_dtype=_dtype_code(q, "q"), kv_dtype=kv_code, kv_capacity=T_cap, path=PATHS[path])
    if kv_code == DTYPES["fp8_e4m3fn"]:
        _scales(o, B, G, k_scale, v_scale, q.device, "fp8 caches")
    return o


def prefill_cached(q, k_cache, v_cache, seq_lens, out=None, scale=None, causal=True, k_scale=None, v_scale=None,
                   path="auto", stream=None):
    """Prefill of a chunk of Tq positions against a cache. Returns ``out`` [B, H, Tq, D].

    q [B, H, Tq, D]; caches [B, G, T_cap, D] already holding the chunk's keys and values at rows
    seq_lens[b]-Tq .. seq_lens[b]-1; query i of sequence b sits at position seq_lens[b]-Tq+i."""
    _need_cuda(q, "q")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _need_cuda(t, n, q.device)
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected q [B,H,Tq,D] and k_cache, v_cache [B,G,T_cap,D]")
    B, H, Tq, D = q.shape
    Bk, G, T_cap, Dk = k_cache.shape
    if Bk != B or Dk != D or seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, caches and seq_lens (int32 [B])")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must share a dtype")
    if out is None:
        out = _new_out(q, stream)
    _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = _chunk_opts(q, k_cache, B, G, T_cap, k_scale, v_scale, path)
    st = library().gqa_prefill_cached(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                      out.data_ptr(), B, Tq, H, G, D, float(scale), int(bool(causal)),
                                      _stream_handle(stream, q.device), ctypes.byref(o))
    if st != GQA_OK:
        raise GqaError(st, "gqa_prefill_cached")
    return out


def prefill_paged(q, k_pages, v_pages, block_table, seq_lens, out=None, scale=None, causal=True, k_scale=None,
                  v_scale=None, path="auto", stream=None):
    """Prefill of a chunk of Tq positions against a paged cache. Returns ``out`` [B, H, Tq, D].

    ``k_pages``/``v_pages`` [num_pages, G, page_size, D] and ``block_table`` int32 [B, pages_per_seq]
    as for ``decode_paged``; the other arguments are those of ``prefill_cached``."""
    _need_cuda(q, "q")
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _need_cuda(t, n, q.device)
    if q.dim() != 4 or k_pages.dim() != 4 or k_pages.shape != v_pages.shape or block_table.dim() != 2:
        raise ValueError("expected q [B,H,Tq,D], pools [num_pages,G,page_size,D] and block_table [B,pages_per_seq]")
    B, H, Tq, D = q.shape
    num_pages, G, page_size, Dk = k_pages.shape
    Bt, pages_per_seq = block_table.shape
    if Bt != B or Dk != D or block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, pools, block_table (int32) and seq_lens (int32 [B])")
    if k_pages.dtype != v_pages.dtype:
        raise TypeError("k_pages and v_pages must share a dtype")
    if out is None:
        out = _new_out(q, stream)
    _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = _chunk_opts(q, k_pages, B, G, pages_per_seq * page_size, k_scale, v_scale, path)
    st = library().gqa_prefill_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                     seq_lens.data_ptr(), out.data_ptr(), B, Tq, H, G, D, float(scale),
                                     int(bool(causal)), page_size, pages_per_seq, num_pages,
                                     _stream_handle(stream, q.device), ctypes.byref(o))
    if st != GQA_OK:
        raise GqaError(st, "gqa_prefill_paged")
    return out
