"""fp64 CPU oracle for grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP path: the C source
``gqa_oracle.c`` (built with gcc into ``liboracle.so``) computes attention from its
definition in double precision, and ``brute.py`` repeats it in pure Python for tiny
inputs. Inputs come from ``workloads.py``; bf16 and fp32 values convert exactly to
float64, fp8 codes are decoded by the C oracle's own E4M3FN decoder.

Which passage each function follows is stated in ``gqa_oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gqa_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_fp = ctypes.POINTER(ctypes.c_float)


# A sanitized build (AddressSanitizer + UndefinedBehaviorSanitizer, gcc) of the same source, for
# the CPU test suite run under those checkers: build it with build(sanitize=True) and point
# GQA_ORACLE_LIBRARY at it (the process must preload gcc's libasan and libubsan; see README).
SANITIZED_LIBRARY = os.path.join(_HERE, "liboracle_sanitized.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def compile_c(src: str, out: str, sanitize: bool = False) -> str:
    """gcc -O2 -fopenmp (no fast-math) of one oracle source into a shared library."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
           *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(sanitize: bool = False) -> str:
    """Compile liboracle.so (or, with sanitize, liboracle_sanitized.so) from gqa_oracle.c."""
    return compile_c(SOURCE, SANITIZED_LIBRARY if sanitize else LIBRARY, sanitize)


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu()
        if x.dtype == torch.float8_e4m3fn:
            raise TypeError("fp8 tensors need their scales: use dequant_e4m3fn")
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class Oracle:
    """ctypes view of one build of the C oracle."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.gqa_oracle_decode.argtypes = [_dp, _dp, _dp, _ip, _dp] + [ctypes.c_int] * 5 + [ctypes.c_double]
        lib.gqa_oracle_decode.restype = ctypes.c_int
        lib.gqa_oracle_decode_rows.argtypes = ([_dp, _dp, _dp, _ip] + [ctypes.c_int] * 5 +
                                               [ctypes.c_double, _lp, ctypes.c_long, _dp])
        lib.gqa_oracle_decode_rows.restype = ctypes.c_int
        lib.gqa_oracle_prefill.argtypes = ([_dp, _dp, _dp, _dp] + [ctypes.c_int] * 5 +
                                           [ctypes.c_double, ctypes.c_int])
        lib.gqa_oracle_prefill.restype = ctypes.c_int
        lib.gqa_oracle_prefill_rows.argtypes = ([_dp, _dp, _dp] + [ctypes.c_int] * 5 +
                                                [ctypes.c_double, ctypes.c_int, _lp, ctypes.c_long, _dp])
        lib.gqa_oracle_prefill_rows.restype = ctypes.c_int
        lib.gqa_oracle_prefill_cached.argtypes = ([_dp, _dp, _dp, _ip, _dp] + [ctypes.c_int] * 5 +
                                                  [ctypes.c_long, ctypes.c_double, ctypes.c_int])
        lib.gqa_oracle_prefill_cached.restype = ctypes.c_int
        lib.gqa_oracle_int4_value.argtypes = [ctypes.c_int]
        lib.gqa_oracle_int4_value.restype = ctypes.c_int
        lib.gqa_oracle_int4_encode.argtypes = [ctypes.c_float]
        lib.gqa_oracle_int4_encode.restype = ctypes.c_int
        lib.gqa_oracle_quant_int4.argtypes = [_fp, ctypes.c_float, ctypes.c_long, _u8p]
        lib.gqa_oracle_quant_int4.restype = None
        lib.gqa_oracle_dequant_int4.argtypes = [_u8p, _fp, ctypes.c_long, ctypes.c_long, _dp]
        lib.gqa_oracle_dequant_int4.restype = None
        lib.gqa_oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.gqa_oracle_e4m3fn_value.restype = ctypes.c_double
        lib.gqa_oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
        lib.gqa_oracle_e4m3fn_encode.restype = ctypes.c_uint8
        lib.gqa_oracle_quant_e4m3fn.argtypes = [_fp, ctypes.c_float, ctypes.c_long, _u8p]
        lib.gqa_oracle_quant_e4m3fn.restype = None
        lib.gqa_oracle_dequant_e4m3fn.argtypes = [_u8p, _fp, ctypes.c_long, ctypes.c_long, _dp]
        lib.gqa_oracle_dequant_e4m3fn.restype = None
        lib.gqa_oracle_num_threads.restype = ctypes.c_int
        lib.gqa_oracle_set_num_threads.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = path

    # ---- threads -------------------------------------------------------------------
    def num_threads(self) -> int:
        return int(self.lib.gqa_oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.gqa_oracle_set_num_threads(int(n))

    # ---- fp8 -----------------------------------------------------------------------
    def e4m3fn_value(self, code: int) -> float:
        return float(self.lib.gqa_oracle_e4m3fn_value(int(code) & 0xFF))

    def e4m3fn_encode(self, q: float) -> int:
        return int(self.lib.gqa_oracle_e4m3fn_encode(float(q)))

    def quant_e4m3fn(self, x, scale: float) -> np.ndarray:
        """Codes (uint8) of x / scale, the quotient in fp32, nearest-even, saturating at 448."""
        xn = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        codes = np.empty(xn.shape, dtype=np.uint8)
        self.lib.gqa_oracle_quant_e4m3fn(_ptr(xn, _fp), ctypes.c_float(float(np.float32(scale))), xn.size,
                                         _ptr(codes, _u8p))
        return codes

    def int4_value(self, u: int) -> int:
        return int(self.lib.gqa_oracle_int4_value(int(u)))

    def int4_encode(self, q: float) -> int:
        return int(self.lib.gqa_oracle_int4_encode(float(q)))

    def quant_int4(self, x, scale: float) -> np.ndarray:
        """Packed INT4 fields (uint8, half the length) of x / scale, the quotient in fp32."""
        xn = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        packed = np.empty(xn.shape[:-1] + (xn.shape[-1] // 2,), dtype=np.uint8)
        self.lib.gqa_oracle_quant_int4(_ptr(xn, _fp), ctypes.c_float(float(np.float32(scale))), xn.size,
                                       _ptr(packed, _u8p))
        return packed

    def dequant_int4(self, packed: torch.Tensor, scales: torch.Tensor) -> np.ndarray:
        """packed [S, ..., D/2] uint8, scales [S] float32 -> float64 [S, ..., D]."""
        c = np.ascontiguousarray(packed.detach().cpu().numpy(), dtype=np.uint8)
        sn = np.ascontiguousarray(scales.detach().cpu().to(torch.float32).numpy(), dtype=np.float32)
        nslab = sn.shape[0]
        slab_len = 2 * c.size // nslab
        out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.float64)
        self.lib.gqa_oracle_dequant_int4(_ptr(c, _u8p), _ptr(sn, _fp), nslab, slab_len, _ptr(out, _dp))
        return out

    # ---- cache append ---------------------------------------------------------------
    def append(self, case, k_new, v_new):
        """The caches of a decode case after storing the new token's key and value [B, G, D]
        (q's dtype) at row L_b - 1 of every (b, g) with 1 <= L_b <= T_cap: copied for fp32 and
        bf16 caches, quantised with the slab's fixed scale for fp8 ones. Returns new cache
        tensors (same dtype as the case's); the case is not modified."""
        kc, vc = case.k_cache.clone(), case.v_cache.clone()
        B, G, T_cap, D = kc.shape
        kn = k_new.detach().cpu().to(torch.float32).numpy()
        vn = v_new.detach().cpu().to(torch.float32).numpy()
        for b in range(B):
            L = int(case.seq_lens[b])
            if not 1 <= L <= T_cap:
                continue
            for g in range(G):
                if case.kv_dtype == "fp8_e4m3fn":
                    i = b * G + g
                    kc.view(torch.uint8)[b, g, L - 1] = torch.from_numpy(self.quant_e4m3fn(kn[b, g], case.k_scale[i]))
                    vc.view(torch.uint8)[b, g, L - 1] = torch.from_numpy(self.quant_e4m3fn(vn[b, g], case.v_scale[i]))
                elif case.kv_dtype == "int4":
                    i = b * G + g
                    kc[b, g, L - 1] = torch.from_numpy(self.quant_int4(kn[b, g], case.k_scale[i]))
                    vc[b, g, L - 1] = torch.from_numpy(self.quant_int4(vn[b, g], case.v_scale[i]))
                else:
                    kc[b, g, L - 1] = k_new[b, g].to(kc.dtype)
                    vc[b, g, L - 1] = v_new[b, g].to(vc.dtype)
        return kc, vc

    def dequant_e4m3fn(self, codes: torch.Tensor, scales: torch.Tensor) -> np.ndarray:
        """codes [S, ...] float8_e4m3fn (or uint8), scales [S] float32 -> float64 code*scale."""
        c = codes.detach().cpu().contiguous()
        if c.dtype == torch.float8_e4m3fn:
            c = c.view(torch.uint8)
        cn = np.ascontiguousarray(c.numpy(), dtype=np.uint8)
        sn = np.ascontiguousarray(scales.detach().cpu().to(torch.float32).numpy(), dtype=np.float32)
        nslab = sn.shape[0]
        slab_len = cn.size // nslab
        assert nslab * slab_len == cn.size
        out = np.empty(cn.shape, dtype=np.float64)
        self.lib.gqa_oracle_dequant_e4m3fn(_ptr(cn, _u8p), _ptr(sn, _fp), nslab, slab_len, _ptr(out, _dp))
        return out

    # ---- decode --------------------------------------------------------------------
    def decode_kv_f64(self, case):
        """The K and V cache values a decode case stands for, as float64 arrays."""
        if case.kv_dtype == "fp8_e4m3fn":
            return (self.dequant_e4m3fn(case.k_cache, case.k_scale),
                    self.dequant_e4m3fn(case.v_cache, case.v_scale))
        if case.kv_dtype == "int4":
            return self.dequant_int4(case.k_cache, case.k_scale), self.dequant_int4(case.v_cache, case.v_scale)
        return _f64(case.k_cache), _f64(case.v_cache)

    def decode_arrays(self, q, k_cache, v_cache, seq_lens, scale) -> np.ndarray:
        q, k, v = _f64(q), _f64(k_cache), _f64(v_cache)
        B, H, D = q.shape
        _, G, T_cap, _ = k.shape
        sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        out = np.empty((B, H, D), dtype=np.float64)
        rc = self.lib.gqa_oracle_decode(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(sl, _ip),
                                        _ptr(out, _dp), B, H, G, D, T_cap, float(scale))
        if rc != 0:
            raise ValueError(f"oracle decode rejected its arguments (code {rc})")
        return out

    def decode(self, case) -> np.ndarray:
        """Oracle output [B, H, D] (float64) for a workloads.DecodeCase."""
        k, v = self.decode_kv_f64(case)
        return self.decode_arrays(case.q, k, v, case.seq_lens.numpy(), case.scale)

    def paged_kv(self, case):
        """The logical caches [B, G, pages_per_seq * page_size, D] of a paged case: row t of
        (b, g) is row t mod page_size of page block_table[b, t div page_size]. Returns tensors of
        the case's cache dtype, so decode_kv_f64 and append read them as a contiguous case."""
        kp, vp, bt = case.k_pages, case.v_pages, case.block_table.to(torch.int64)
        B, pps = bt.shape
        ps = kp.shape[2]
        t = torch.arange(pps * ps)
        page = bt[:, t // ps]                       # [B, T]
        off = (t % ps).expand(B, -1)                # [B, T]
        # pool[page, :, off] for every (b, t) -> [B, T, G, D] -> [B, G, T, D]
        gather = lambda pool: pool[page, :, off].permute(0, 2, 1, 3).contiguous()
        return gather(kp), gather(vp)

    def contiguous_case(self, case):
        """A workloads.DecodeCase-like view of a paged case, with the logical caches."""
        import types
        k, v = self.paged_kv(case)
        return types.SimpleNamespace(q=case.q, k_cache=k, v_cache=v, seq_lens=case.seq_lens, scale=case.scale,
                                     q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                                     v_scale=case.v_scale, name=case.name)

    def decode_paged(self, case) -> np.ndarray:
        """Oracle output [B, H, D] (float64) for a paged case: the decode of its logical caches."""
        return self.decode(self.contiguous_case(case))

    def decode_rows(self, case, rows, kv=None) -> np.ndarray:
        """Oracle output for selected rows (b*H + h) -> [len(rows), D]."""
        k, v = kv if kv is not None else self.decode_kv_f64(case)
        q = _f64(case.q)
        B, H, D = q.shape
        _, G, T_cap, _ = k.shape
        sl = np.ascontiguousarray(case.seq_lens.numpy().astype(np.int32))
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rc = self.lib.gqa_oracle_decode_rows(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(sl, _ip),
                                             B, H, G, D, T_cap, float(case.scale), _ptr(r, _lp),
                                             r.shape[0], _ptr(out, _dp))
        if rc != 0:
            raise ValueError(f"oracle decode_rows rejected its arguments (code {rc})")
        return out

    # ---- prefill -------------------------------------------------------------------
    def prefill_arrays(self, q, k, v, scale, causal) -> np.ndarray:
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, T, D = q.shape
        G = k.shape[1]
        out = np.empty((B, H, T, D), dtype=np.float64)
        rc = self.lib.gqa_oracle_prefill(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(out, _dp),
                                         B, T, H, G, D, float(scale), int(bool(causal)))
        if rc != 0:
            raise ValueError(f"oracle prefill rejected its arguments (code {rc})")
        return out

    def prefill(self, case) -> np.ndarray:
        """Oracle output [B, H, T, D] (float64) for a workloads.PrefillCase."""
        return self.prefill_arrays(case.q, case.k, case.v, case.scale, case.causal)

    def prefill_cached_arrays(self, q, k_cache, v_cache, seq_lens, scale, causal) -> np.ndarray:
        """Chunk of Tq queries [B,H,Tq,D] against caches [B,G,T_cap,D] holding seq_lens[b] rows."""
        q, k, v = _f64(q), _f64(k_cache), _f64(v_cache)
        B, H, Tq, D = q.shape
        _, G, T_cap, _ = k.shape
        sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        out = np.empty((B, H, Tq, D), dtype=np.float64)
        rc = self.lib.gqa_oracle_prefill_cached(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(sl, _ip),
                                                _ptr(out, _dp), B, Tq, H, G, D, T_cap, float(scale),
                                                int(bool(causal)))
        if rc != 0:
            raise ValueError(f"oracle prefill_cached rejected its arguments (code {rc})")
        return out

    def prefill_cached(self, case) -> np.ndarray:
        """Oracle output [B, H, Tq, D] (float64) for a workloads.ChunkCase (fp8 caches dequantised
        with their scales first)."""
        if case.kv_dtype == "fp8_e4m3fn":
            k, v = self.dequant_e4m3fn(case.k_cache, case.k_scale), self.dequant_e4m3fn(case.v_cache, case.v_scale)
        else:
            k, v = case.k_cache, case.v_cache
        return self.prefill_cached_arrays(case.q, k, v, case.seq_lens.numpy(), case.scale, case.causal)

    def prefill_paged(self, case) -> np.ndarray:
        """Oracle output [B, H, Tq, D] for a paged chunk case: prefill_cached over the logical
        caches gathered from its pages."""
        import types
        k, v = self.paged_kv(case)
        return self.prefill_cached(types.SimpleNamespace(q=case.q, k_cache=k, v_cache=v, seq_lens=case.seq_lens,
                                                         scale=case.scale, causal=case.causal, kv_dtype=case.kv_dtype,
                                                         k_scale=case.k_scale, v_scale=case.v_scale))

    def prefill_rows(self, case, rows, f64=None) -> np.ndarray:
        """Oracle output for selected rows ((b*H + h)*T + i) -> [len(rows), D]."""
        q, k, v = f64 if f64 is not None else (_f64(case.q), _f64(case.k), _f64(case.v))
        B, H, T, D = q.shape
        G = k.shape[1]
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rc = self.lib.gqa_oracle_prefill_rows(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), B, T, H, G, D,
                                              float(case.scale), int(bool(case.causal)), _ptr(r, _lp),
                                              r.shape[0], _ptr(out, _dp))
        if rc != 0:
            raise ValueError(f"oracle prefill_rows rejected its arguments (code {rc})")
        return out


_default = None


def load() -> Oracle:
    """The oracle built from gqa_oracle.c (compiled here if missing or stale), or the build that
    GQA_ORACLE_LIBRARY names (the sanitized one)."""
    global _default
    if _default is None:
        path = os.environ.get("GQA_ORACLE_LIBRARY")
        if path is None:
            path = LIBRARY
            if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
                build()
        _default = Oracle(path)
    return _default


def from_library(path: str) -> Oracle:
    return Oracle(path)


def to_f64(x) -> np.ndarray:
    """Exact float64 copy of an fp32/bf16 tensor or array."""
    return _f64(x)


# Module-level shortcuts onto the default build.
def decode(case): return load().decode(case)
def decode_rows(case, rows, kv=None): return load().decode_rows(case, rows, kv)
def decode_paged(case): return load().decode_paged(case)
def paged_kv(case): return load().paged_kv(case)
def contiguous_case(case): return load().contiguous_case(case)
def decode_arrays(*a): return load().decode_arrays(*a)
def decode_kv_f64(case): return load().decode_kv_f64(case)
def prefill(case): return load().prefill(case)
def prefill_rows(case, rows, f64=None): return load().prefill_rows(case, rows, f64)
def prefill_arrays(*a): return load().prefill_arrays(*a)
def prefill_cached(case): return load().prefill_cached(case)
def prefill_paged(case): return load().prefill_paged(case)
def prefill_cached_arrays(*a): return load().prefill_cached_arrays(*a)
def dequant_e4m3fn(codes, scales): return load().dequant_e4m3fn(codes, scales)
def e4m3fn_value(code): return load().e4m3fn_value(code)
def e4m3fn_encode(q): return load().e4m3fn_encode(q)
def quant_e4m3fn(x, scale): return load().quant_e4m3fn(x, scale)
def append(case, k_new, v_new): return load().append(case, k_new, v_new)
def int4_value(u): return load().int4_value(u)
def int4_encode(q): return load().int4_encode(q)
def quant_int4(x, scale): return load().quant_int4(x, scale)
def dequant_int4(packed, scales): return load().dequant_int4(packed, scales)
def num_threads(): return load().num_threads()
def set_num_threads(n): return load().set_num_threads(n)
