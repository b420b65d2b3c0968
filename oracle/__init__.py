"""CPU oracle for ragged paged attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. The product path (``ragged_paged_attention_rpa_amd``
and its HIP library) never imports it, and this package imports nothing from
the product path: the two share no code.

The arithmetic lives in ``rpa_oracle.c`` (plain C, fp64, OpenMP over output
rows); this module only builds it with gcc and marshals numpy arrays through
ctypes. Inputs are the raw stored arrays (fp32, bf16 bit patterns as uint16,
fp8 e4m3fn bit patterns as uint8); outputs are fp64.

Pages cited by short name: "RPA v2 page" (tpu-inference ragged_paged_attention
v2 kernel), "MLA v1 page" (tpu-inference MLA v1 kernel), "Sparse page"
(sglang-jax sparse MLA prefill kernel).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rpa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8_E4M3, INT8, INT4 = 0, 1, 2, 3, 4
LAYOUT_COMBINED_GQA, LAYOUT_MLA_SPLIT, LAYOUT_MLA_FUSED = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compiles rpa_oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # RPA_ORACLE_LIB names another build of this oracle (the mutation test
        # loads deliberately broken copies through it); default: the in-tree one.
        path = os.environ.get("RPA_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        c_void_p, c_int, c_double = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.oracle_rpa.restype = c_int
        lib.oracle_rpa.argtypes = [c_void_p, c_int, c_int, c_int, c_int,
                                   c_void_p, c_int, c_int, c_int, c_int,
                                   c_void_p, c_void_p, c_int, c_void_p, c_int,
                                   c_double, c_int, c_double, c_double, c_double, c_double,
                                   c_void_p, c_int, c_void_p]
        lib.oracle_mla.restype = c_int
        lib.oracle_mla.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                   c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_int,
                                   c_void_p, c_void_p, c_int, c_void_p, c_int,
                                   c_double, c_int, c_double, c_double, c_double, c_double,
                                   c_void_p, c_int, c_void_p]
        lib.oracle_sparse_mla.restype = c_int
        lib.oracle_sparse_mla.argtypes = [c_void_p, c_int, c_int, c_int, c_int, c_int,
                                          c_void_p, c_int, c_int, c_int,
                                          c_void_p, c_int, c_void_p, c_int, c_int,
                                          c_void_p, c_int, c_double,
                                          c_void_p, c_void_p, c_void_p, c_int,
                                          c_void_p, c_int, c_void_p]
        lib.oracle_kv_update.restype = c_int
        lib.oracle_kv_update.argtypes = [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                         c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                         c_void_p, c_void_p, c_int, c_void_p, c_int,
                                         c_void_p, c_int]
        lib.oracle_num_threads.restype = c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_decode_bf16.restype = c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_e4m3fn.restype = c_double
        lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _storage(a, dtype):
    """Raw storage array for one of the oracle's dtype codes."""
    want = {F32: np.float32, BF16: np.uint16, FP8_E4M3: np.uint8, INT8: np.int8,
            INT4: np.uint8}[dtype]
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"expected storage dtype {want} for code {dtype}, got {a.dtype}")
    return a


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle rejected the input (code {rc})")


def rpa(q, q_dtype, kv_pages, kv_dtype, kv_lens, page_indices, cu_q_lens, num_seqs, *,
        sm_scale=1.0, sliding_window=None, soft_cap=None, k_scale=None, v_scale=None,
        q_scale=None, tokens=None):
    """GQA ragged paged attention [RPA v2 page: ref_ragged_paged_attention].
    Stored K, V and Q are dequantised exactly by k_scale, v_scale, q_scale.

    q [T, Hq, D]; kv_pages [P, ps, 2*Hkv, D]; page_indices [max_num_seqs, pps]
    (or flat). Returns fp64 [T, Hq, D]; rows outside ``tokens`` (when given)
    are NaN.
    """
    q = _storage(q, q_dtype)
    kv_pages = _storage(kv_pages, kv_dtype)
    T, Hq, D = q.shape
    P, ps, ch, D2 = kv_pages.shape
    # INT4 storage: two values per byte along the last index.
    assert (2 * D2 if kv_dtype == INT4 else D2) == D and ch % 2 == 0
    kv_lens = _c(kv_lens, np.int32)
    cu_q_lens = _c(cu_q_lens, np.int32)
    pi = _c(page_indices, np.int32)
    max_num_seqs = kv_lens.shape[0]
    pps = pi.size // max_num_seqs
    tl = None if tokens is None else _c(tokens, np.int32)
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    rc = _load().oracle_rpa(
        _ptr(q), q_dtype, T, Hq, D, _ptr(kv_pages), kv_dtype, P, ps, ch // 2,
        _ptr(kv_lens), _ptr(pi), pps, _ptr(cu_q_lens), int(num_seqs),
        float(sm_scale), int(sliding_window or 0), float(soft_cap or 0.0),
        float(1.0 if k_scale is None else k_scale), float(1.0 if v_scale is None else v_scale),
        float(1.0 if q_scale is None else q_scale),
        _ptr(tl), 0 if tl is None else tl.size, _ptr(out))
    _check(rc, "rpa")
    return out


def mla(ql_nope, q_pe, dtype, cache_kv_c, cache_k_pe, kv_lens, page_indices, cu_q_lens,
        num_seqs, *, sm_scale=1.0, sliding_window=None, soft_cap=None, tokens=None,
        fused=False, q_scale=None, k_scale=None, v_scale=None):
    """MLA latent attention over an updated cache
    [MLA v1 page: ref_mla_ragged_paged_attention].

    ql_nope [T, H, Dl], q_pe [T, H, Dr]; cache_kv_c [P, ps, >=Dl] and
    cache_k_pe [P, ps, >=Dr] (split layout) or, with ``fused``, one array
    [P, ps, >=Dl+Dr] passed as cache_kv_c (cache_k_pe ignored).
    Scores are multiplied by sm_scale, k_scale and q_scale, the value sum by
    v_scale (the page's kernel scales). Returns fp64 [T, H, Dl].
    """
    ql_nope = _storage(ql_nope, dtype)
    q_pe = _storage(q_pe, dtype)
    T, H, Dl = ql_nope.shape
    Dr = q_pe.shape[2]
    cache_kv_c = _storage(cache_kv_c, dtype)
    P, ps, kvc_stride = cache_kv_c.shape
    if fused:
        cache_k_pe, kpe_stride, kpe_col = cache_kv_c, kvc_stride, Dl
    else:
        cache_k_pe = _storage(cache_k_pe, dtype)
        kpe_stride, kpe_col = cache_k_pe.shape[2], 0
    kv_lens = _c(kv_lens, np.int32)
    cu_q_lens = _c(cu_q_lens, np.int32)
    pi = _c(page_indices, np.int32)
    pps = pi.size // kv_lens.shape[0]
    tl = None if tokens is None else _c(tokens, np.int32)
    out = np.full((T, H, Dl), np.nan, dtype=np.float64)
    rc = _load().oracle_mla(
        _ptr(ql_nope), _ptr(q_pe), dtype, T, H, Dl, Dr, _ptr(cache_kv_c), kvc_stride,
        _ptr(cache_k_pe), kpe_stride, kpe_col, P, ps, _ptr(kv_lens), _ptr(pi), pps,
        _ptr(cu_q_lens), int(num_seqs), float(sm_scale), int(sliding_window or 0),
        float(soft_cap or 0.0), float(1.0 if q_scale is None else q_scale),
        float(1.0 if k_scale is None else k_scale), float(1.0 if v_scale is None else v_scale),
        _ptr(tl), 0 if tl is None else tl.size, _ptr(out))
    _check(rc, "mla")
    return out


def sparse_mla(q, dtype, kv_cache, page_table, indices, positions, *, seq_len=0, read_block,
               sm_scale, dv=512, queries=None, cu_q_lens=None, seq_lens=None, cu_kv_lens=None):
    """Sparse MLA-latent attention, paged single-sequence or packed-ragged mode
    [Sparse page: sparse_mla_attention / _sparse_mla_kernel_chunked_hminor;
    prefill_write_and_attend_ragged].

    q [S, H, Dk]; kv_cache [P, ps, C] fused latent pool; page_table [PTW];
    indices [S, K] unit ids (-1 = padding); positions [S].
    Single-sequence mode: causal bound seq_len, page_table indexed from 0.
    Ragged mode (cu_q_lens [R+1], seq_lens [R], cu_kv_lens [R+1] given): token s
    belongs to request rid = min(searchsorted(cu_q_lens[1:], s, 'right'), R-1),
    is bounded by seq_lens[rid], and its unit ids index page_table from
    cu_kv_lens[rid] // page_size.
    Returns fp64 [S, H, dv]; an empty key set gives zeros.
    """
    q = _storage(q, dtype)
    kv_cache = _storage(kv_cache, dtype)
    S, H, Dk = q.shape
    P, ps, C = kv_cache.shape
    pt = _c(page_table, np.int32)
    idx = _c(indices, np.int32)
    pos = _c(positions, np.int32)
    ql = None if queries is None else _c(queries, np.int32)
    ragged = cu_q_lens is not None
    if ragged and (seq_lens is None or cu_kv_lens is None):
        raise ValueError("ragged mode needs cu_q_lens, seq_lens and cu_kv_lens")
    cq = _c(cu_q_lens, np.int32) if ragged else None
    sl = _c(seq_lens, np.int32) if ragged else None
    ck = _c(cu_kv_lens, np.int32) if ragged else None
    out = np.full((S, H, dv), np.nan, dtype=np.float64)
    rc = _load().oracle_sparse_mla(
        _ptr(q), dtype, S, H, Dk, dv, _ptr(kv_cache), P, ps, C, _ptr(pt), pt.size,
        _ptr(idx), idx.shape[1], int(read_block), _ptr(pos), int(seq_len), float(sm_scale),
        _ptr(cq), _ptr(sl), _ptr(ck), 0 if not ragged else sl.size,
        _ptr(ql), 0 if ql is None else ql.size, _ptr(out))
    _check(rc, "sparse_mla")
    return out


def kv_update(layout, new_a, new_b, cache_a, cache_b, dtype, *, kv_lens=None,
              page_indices=None, cu_q_lens=None, num_seqs=0, slot_loc=None):
    """Scatter new tokens into the caches IN PLACE (numpy arrays)
    [MLA v1 page: update_kv_cache; Sparse page: prefill_write_and_attend].

    COMBINED_GQA: new_a = K [T, Hkv, D], new_b = V [T, Hkv, D], cache_a [P, ps, 2Hkv, D]
                  (INT4: packed bytes, last dimension D / 2).
    MLA_SPLIT: new_a = kv_c [T, Dl], new_b = k_pe [T, Dr], cache_a [P, ps, >=Dl],
               cache_b [P, ps, >=Dr] (pad columns written as 0).
    MLA_FUSED: cache_a [P, ps, >=Dl+Dr] receives [kv_c || k_pe || 0].
    """
    new_a = _storage(new_a, dtype)
    new_b = _storage(new_b, dtype)
    assert cache_a.flags["C_CONTIGUOUS"]
    _storage(cache_a, dtype)
    P, ps = cache_a.shape[0], cache_a.shape[1]
    T = new_a.shape[0]
    if layout == LAYOUT_COMBINED_GQA:
        heads, dim_a = new_a.shape[1], new_a.shape[2] * (2 if dtype == INT4 else 1)
        dim_b, stride_a, stride_b = dim_a, 0, 0
    else:
        heads = 0
        dim_a, dim_b = new_a.shape[1], new_b.shape[1]
        stride_a = cache_a.shape[2]
        stride_b = cache_b.shape[2] if cache_b is not None else 0
    if cache_b is not None:
        assert cache_b.flags["C_CONTIGUOUS"]
        _storage(cache_b, dtype)
    kv_lens = _c(kv_lens, np.int32)
    cu_q_lens = _c(cu_q_lens, np.int32)
    pi = _c(page_indices, np.int32)
    sl = _c(slot_loc, np.int32)
    pps = 0 if pi is None else pi.size // kv_lens.shape[0]
    rc = _load().oracle_kv_update(
        layout, _ptr(new_a), _ptr(new_b), _ptr(cache_a), _ptr(cache_b), dtype, P, ps, heads,
        dim_a, dim_b, stride_a, stride_b, _ptr(kv_lens), _ptr(pi), pps, _ptr(cu_q_lens),
        int(num_seqs), _ptr(sl), T)
    _check(rc, "kv_update")


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(bits)


def decode_e4m3fn(bits: int) -> float:
    return _load().oracle_decode_e4m3fn(bits)
