"""MI355X-native ragged paged attention: Python binding of librpa.so.

Thin ctypes marshalling over the C ABI declared in ``include/rpa.h``; every
step of the computation runs in the library's HIP kernels. PyTorch supplies
device memory and the current stream. The functions carry the C names:

* :func:`rpa_forward`        GQA attention over a packed ragged batch and a paged K/V pool
* :func:`kv_cache_update`    scatter new tokens into page/row slots
* :func:`mla_rpa_forward`    MLA latent variant (scatter + attention)
* :func:`sparse_mla_forward` sparse top-k MLA over a fused latent pool

The library is loaded on first use; if it has not been built
(``python -m ragged_paged_attention_rpa_amd.build``) the call raises
:class:`RpaLibraryMissing`. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["rpa_forward", "kv_cache_update", "mla_rpa_forward", "sparse_mla_forward",
           "sparse_mla_forward_ragged",
           "rpa_workspace_size", "mla_rpa_workspace_size",
           "RpaError", "RpaLibraryMissing", "library_path", "load_library",
           "LAYOUT_COMBINED_GQA", "LAYOUT_MLA_SPLIT", "LAYOUT_MLA_FUSED", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# RPA_LIBRARY names another build of the library (e.g. the host-sanitized one
# the CPU tests make); by default the in-tree librpa.so.
LIB_PATH = os.environ.get("RPA_LIBRARY") or os.path.join(_HERE, "librpa.so")

LAYOUT_COMBINED_GQA, LAYOUT_MLA_SPLIT, LAYOUT_MLA_FUSED = 0, 1, 2
EXPORTED_SYMBOLS = ("rpa_opts_init", "rpa_last_error", "rpa_last_path", "rpa_set_profile_events",
                    "rpa_set_profile_events_split",
                    "rpa_tile_config", "rpa_workspace_size", "rpa_forward", "rpa_forward_noalloc",
                    "rpa_noalloc_scratch_bytes",
                    "kv_cache_update", "mla_rpa_workspace_size", "mla_rpa_forward",
                    "sparse_mla_forward",
                    "sparse_mla_forward_ragged")


class RpaLibraryMissing(RuntimeError):
    pass


class RpaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"rpa status {status}: {message}")
        self.status = status


class _Meta(ctypes.Structure):
    _fields_ = [("cu_q_lens", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("page_indices", ctypes.c_void_p), ("num_seqs", ctypes.c_void_p),
                ("max_num_seqs", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32),
                ("max_num_tokens", ctypes.c_int32)]


class _Opts(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("sliding_window", ctypes.c_int32),
                ("soft_cap", ctypes.c_float), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("debug_validate", ctypes.c_int32),
                ("split_keys", ctypes.c_int32), ("q_scale", ctypes.c_float)]


class _TileParams(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("table_row", ctypes.c_int32)]


TILE_DECODE_SPLIT, TILE_MLA_SHARE = 0, 1


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Loads librpa.so (once) and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RpaLibraryMissing(
            f"{LIB_PATH} is missing; build it with `python -m ragged_paged_attention_rpa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    MP, OP = ctypes.POINTER(_Meta), ctypes.POINTER(_Opts)
    lib.rpa_opts_init.argtypes = [OP]
    lib.rpa_opts_init.restype = None
    lib.rpa_last_error.argtypes = []
    lib.rpa_last_error.restype = ctypes.c_char_p
    lib.rpa_tile_config.argtypes = [I32, I32, I32, I32, I32, I32, MP, OP,
                                    ctypes.POINTER(_TileParams)]
    lib.rpa_tile_config.restype = I32
    lib.rpa_last_path.argtypes = []
    lib.rpa_last_path.restype = ctypes.c_char_p
    lib.rpa_set_profile_events.argtypes = [P, P]
    lib.rpa_set_profile_events.restype = None
    lib.rpa_set_profile_events_split.argtypes = [P, P, P, P]
    lib.rpa_set_profile_events_split.restype = None
    lib.rpa_workspace_size.argtypes = [MP, I32, I32, I32]
    lib.rpa_workspace_size.restype = SZ
    lib.rpa_forward.argtypes = [P, I32, I32, I32, P, I32, I32, I32, I32, P, MP, OP, P, P, SZ, P]
    lib.rpa_forward.restype = I32
    lib.rpa_forward_noalloc.argtypes = [P, I32, I32, I32, P, I32, I32, I32, I32, P, MP, OP, P, P]
    lib.rpa_forward_noalloc.restype = I32
    lib.rpa_noalloc_scratch_bytes.argtypes = []
    lib.rpa_noalloc_scratch_bytes.restype = SZ
    lib.kv_cache_update.argtypes = [I32, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32,
                                    MP, P, I32, P]
    lib.kv_cache_update.restype = I32
    lib.mla_rpa_workspace_size.argtypes = [MP, I32, I32]
    lib.mla_rpa_workspace_size.restype = SZ
    lib.mla_rpa_forward.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, MP,
                                    OP, P, P, SZ, P]
    lib.mla_rpa_forward.restype = I32
    lib.sparse_mla_forward.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32,
                                       I32, I32, F32, P, P]
    lib.sparse_mla_forward.restype = I32
    lib.sparse_mla_forward_ragged.argtypes = [P, P, P, I32, P, P, P, P, P, I32, I32, I32, I32, I32,
                                              I32, I32, I32, I32, I32, F32, P, P]
    lib.sparse_mla_forward_ragged.restype = I32
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype == torch.float8_e4m3fn:
        return 2
    if t.dtype == torch.int8:
        return 3
    if t.dtype == torch.uint8:
        return 4  # a packed INT4 pool: two values per byte, element 2i in the low nibble
    raise TypeError(f"unsupported dtype {t.dtype}")


def _pool_head_dim(kv_pages):
    """head_dim of a [P, ps, 2*Hkv, D] pool (a packed INT4 pool stores D / 2 bytes)."""
    return kv_pages.shape[3] * (2 if kv_pages.dtype == _torch().uint8 else 1)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def _check_new_kv(new_kv, kv_pages, T):
    if new_kv is None:
        return
    if new_kv.dtype != kv_pages.dtype or tuple(new_kv.shape[1:]) != tuple(kv_pages.shape[2:]) \
            or new_kv.shape[0] < T:
        raise ValueError("new_kv must be [T, 2*Hkv, D] in the pool's dtype")


def _i32(t):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError("metadata tensors must be int32")
    return t


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _raise(lib, st):
    if st != 0:
        raise RpaError(st, lib.rpa_last_error().decode())


def _meta(kv_lens, page_indices, cu_q_lens, num_seqs, max_num_tokens):
    _i32(kv_lens), _i32(page_indices), _i32(cu_q_lens), _i32(num_seqs)
    m = _Meta()
    m.cu_q_lens = cu_q_lens.data_ptr()
    m.kv_lens = kv_lens.data_ptr()
    m.page_indices = page_indices.data_ptr()
    m.num_seqs = num_seqs.data_ptr()
    m.max_num_seqs = kv_lens.numel()
    m.pages_per_seq = page_indices.numel() // max(1, kv_lens.numel())
    m.max_num_tokens = max_num_tokens
    return m


def _opts(lib, sm_scale, sliding_window, soft_cap, k_scale, v_scale, debug_validate,
          split_keys=None, q_scale=None):
    o = _Opts()
    lib.rpa_opts_init(ctypes.byref(o))
    o.sm_scale = float(sm_scale)
    o.sliding_window = int(sliding_window or 0)
    o.soft_cap = float(soft_cap or 0.0)
    o.k_scale = float(1.0 if k_scale is None else k_scale)
    o.v_scale = float(1.0 if v_scale is None else v_scale)
    o.debug_validate = 1 if debug_validate else 0
    o.split_keys = int(split_keys or 0)
    o.q_scale = float(1.0 if q_scale is None else q_scale)
    return o


def tile_config(path, kv_dtype, num_q_heads, num_kv_heads, head_dim, page_size, pages_per_seq,
                split_keys=None):
    """Tile sizes a call would use (see rpa_tile_config in include/rpa.h):
    returns (keys, max_splits, table_row). ``kv_dtype`` is a torch dtype or an
    RPA dtype code; ``path`` is TILE_DECODE_SPLIT or TILE_MLA_SHARE."""
    lib = load_library()
    code = kv_dtype if isinstance(kv_dtype, int) else _dtype_code(_torch().empty(0, dtype=kv_dtype))
    m = _Meta()
    m.max_num_seqs = 1
    m.pages_per_seq = pages_per_seq
    m.max_num_tokens = 1
    o = _opts(lib, 1.0, None, None, None, None, False, split_keys)
    p = _TileParams()
    st = lib.rpa_tile_config(path, code, num_q_heads, num_kv_heads, head_dim, page_size,
                             ctypes.byref(m), ctypes.byref(o), ctypes.byref(p))
    _raise(lib, st)
    return p.keys, p.max_splits, p.table_row


def last_path() -> str:
    """Kernel path of this thread's last successful rpa_forward call
    ("gqa_mfma", "gqa_mfma_prefill" or "gqa_generic")."""
    return load_library().rpa_last_path().decode()


def set_profile_events(start, stop):
    """Records the hipEvent_t handles ``start``/``stop`` (ints or c_void_p, created
    with hipEventCreate) around the main kernel of the following calls on this
    thread; ``None, None`` turns the hook off."""
    lib = load_library()
    if start is None or stop is None:
        lib.rpa_set_profile_events(None, None)
    else:
        lib.rpa_set_profile_events(ctypes.c_void_p(int(getattr(start, "value", start))),
                                   ctypes.c_void_p(int(getattr(stop, "value", stop))))


def rpa_workspace_size(kv_lens, page_indices, max_num_tokens, num_q_heads, num_kv_heads,
                       head_dim):
    lib = load_library()
    m = _Meta()
    m.max_num_seqs = kv_lens.numel()
    m.pages_per_seq = page_indices.numel() // max(1, kv_lens.numel())
    m.max_num_tokens = max_num_tokens
    return int(lib.rpa_workspace_size(ctypes.byref(m), num_q_heads, num_kv_heads, head_dim))


def rpa_forward(q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, *, sm_scale=1.0,
                sliding_window=None, soft_cap=None, k_scale=None, v_scale=None, out=None,
                workspace=None, debug_validate=False, split_keys=None, q_scale=None,
                new_kv=None, stream=None):
    """GQA ragged paged attention (see ``rpa_forward`` in include/rpa.h).

    With ``new_kv`` [T, 2*Hkv, D] (the step's new tokens as pool rows, in the
    pool's dtype) the call also writes those rows into ``kv_pages``.

    q [T, Hq, D] (fp32/bf16, or fp8 e4m3fn with q_scale); kv_pages
    [P, ps, 2*Hkv, D] (fp32/bf16/fp8 e4m3fn/int8 with k_scale, v_scale), or
    uint8 [P, ps, 2*Hkv, D/2] holding packed int4 values (two per byte, element
    2i in the low nibble);
    kv_lens [S], page_indices [S, pps] or [S*pps], cu_q_lens [S+1], num_seqs [1]
    (int32, on the GPU). Returns ``out`` [T, Hq, D] in q's dtype (bf16 for fp8 q).
    """
    torch = _torch()
    lib = load_library()
    _check_dev(q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, out, workspace, new_kv)
    T, Hq, D = q.shape
    P, ps, ch, _ = kv_pages.shape
    if _pool_head_dim(kv_pages) != D or ch % 2:
        raise ValueError("kv_pages must be [P, ps, 2*Hkv, head_dim] (head_dim / 2 bytes for int4)")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn
                          else q.dtype, device=q.device)
    meta = _meta(kv_lens, page_indices, cu_q_lens, num_seqs, T)
    opts = _opts(lib, sm_scale, sliding_window, soft_cap, k_scale, v_scale, debug_validate,
                 split_keys, q_scale)
    need = int(lib.rpa_workspace_size(ctypes.byref(meta), Hq, ch // 2, D))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_new_kv(new_kv, kv_pages, T)
    st = lib.rpa_forward(_ptr(q), _dtype_code(q), Hq, D, _ptr(kv_pages), _dtype_code(kv_pages), P,
                         ps, ch // 2, _ptr(new_kv), ctypes.byref(meta), ctypes.byref(opts),
                         _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _raise(lib, st)
    return out


def rpa_forward_noalloc(q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, *, out,
                        sm_scale=1.0, sliding_window=None, soft_cap=None, k_scale=None,
                        v_scale=None, debug_validate=False, split_keys=None, q_scale=None,
                        new_kv=None, stream=None):
    """rpa_forward on the library's static scratch (see ``rpa_forward_noalloc``
    in include/rpa.h): no workspace and no allocation; ``out`` must be given."""
    lib = load_library()
    _check_dev(q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, out, new_kv)
    T, Hq, D = q.shape
    P, ps, ch, _ = kv_pages.shape
    if _pool_head_dim(kv_pages) != D or ch % 2:
        raise ValueError("kv_pages must be [P, ps, 2*Hkv, head_dim] (head_dim / 2 bytes for int4)")
    meta = _meta(kv_lens, page_indices, cu_q_lens, num_seqs, T)
    opts = _opts(lib, sm_scale, sliding_window, soft_cap, k_scale, v_scale, debug_validate,
                 split_keys, q_scale)
    _check_new_kv(new_kv, kv_pages, T)
    st = lib.rpa_forward_noalloc(_ptr(q), _dtype_code(q), Hq, D, _ptr(kv_pages),
                                 _dtype_code(kv_pages), P, ps, ch // 2, _ptr(new_kv),
                                 ctypes.byref(meta), ctypes.byref(opts), _ptr(out),
                                 _stream(stream))
    _raise(lib, st)
    return out


def noalloc_scratch_bytes() -> int:
    return int(load_library().rpa_noalloc_scratch_bytes())


def kv_cache_update(layout, new_a, new_b, cache_a, cache_b=None, *, kv_lens=None,
                    page_indices=None, cu_q_lens=None, num_seqs=None, slot_loc=None,
                    debug_validate=False, stream=None):
    """Scatter new tokens into a paged cache in place (see include/rpa.h).

    COMBINED_GQA: new_a = K [T, Hkv, D], new_b = V [T, Hkv, D], cache_a [P, ps, 2Hkv, D].
    MLA_SPLIT: new_a = kv_c [T, Dl], new_b = k_pe [T, Dr], cache_a [P, ps, >=Dl],
               cache_b [P, ps, >=Dr].
    MLA_FUSED: cache_a [P, ps, >=Dl+Dr] receives [kv_c || k_pe || 0].
    Addressing: the ragged metadata (page-table mode) or ``slot_loc`` [T].
    """
    lib = load_library()
    _check_dev(new_a, new_b, cache_a, cache_b, kv_lens, page_indices, cu_q_lens, num_seqs,
               slot_loc)
    if new_a.dtype != cache_a.dtype or new_b.dtype != cache_a.dtype:
        raise TypeError("cache dtype must equal the new tokens' dtype")
    P, ps = cache_a.shape[0], cache_a.shape[1]
    T = new_a.shape[0]
    if layout == LAYOUT_COMBINED_GQA:
        heads, dim_a, dim_b, stride_a, stride_b = new_a.shape[1], new_a.shape[2], 0, 0, 0
    else:
        heads, dim_a, dim_b = 0, new_a.shape[1], new_b.shape[1]
        stride_a = cache_a.shape[2]
        stride_b = cache_b.shape[2] if cache_b is not None else 0
    meta = None
    if slot_loc is None:
        meta = _meta(kv_lens, page_indices, cu_q_lens, num_seqs, T)
    else:
        _i32(slot_loc)
    st = lib.kv_cache_update(layout, _ptr(new_a), _ptr(new_b), _ptr(cache_a), _ptr(cache_b),
                             _dtype_code(cache_a), P, ps, heads, dim_a, dim_b, stride_a, stride_b,
                             T, ctypes.byref(meta) if meta is not None else None, _ptr(slot_loc),
                             1 if debug_validate else 0, _stream(stream))
    _raise(lib, st)


def mla_rpa_workspace_size(kv_lens, page_indices, max_num_tokens, num_heads, lkv_dim):
    lib = load_library()
    m = _Meta()
    m.max_num_seqs = kv_lens.numel()
    m.pages_per_seq = page_indices.numel() // max(1, kv_lens.numel())
    m.max_num_tokens = max_num_tokens
    return int(lib.mla_rpa_workspace_size(ctypes.byref(m), num_heads, lkv_dim))


def mla_rpa_forward(ql_nope, q_pe, new_kv_c, new_k_pe, cache_kv_c, cache_k_pe, kv_lens,
                    page_indices, cu_q_lens, num_seqs, *, sm_scale=1.0, sliding_window=None,
                    soft_cap=None, out=None, workspace=None, debug_validate=False, split_keys=None,
                    q_scale=None, k_scale=None, v_scale=None, stream=None):
    """MLA ragged paged attention: scatter (unless new_* are None) then attend.

    ql_nope [T, H, 512], q_pe [T, H, 64], new_kv_c [T, 512], new_k_pe [T, 64],
    cache_kv_c [P, ps, 512], cache_k_pe [P, ps, 128] (bf16). Scores are scaled by
    sm_scale, k_scale and q_scale, the value sum by v_scale. Returns out [T, H, 512].
    """
    torch = _torch()
    lib = load_library()
    _check_dev(ql_nope, q_pe, new_kv_c, new_k_pe, cache_kv_c, cache_k_pe, kv_lens, page_indices,
               cu_q_lens, num_seqs, out, workspace)
    T, H, Dl = ql_nope.shape
    Dr = q_pe.shape[2]
    P, ps, kvc_stride = cache_kv_c.shape
    kpe_stride = cache_k_pe.shape[2]
    if out is None:
        out = torch.empty_like(ql_nope)
    meta = _meta(kv_lens, page_indices, cu_q_lens, num_seqs, T)
    opts = _opts(lib, sm_scale, sliding_window, soft_cap, k_scale, v_scale, debug_validate,
                 split_keys, q_scale)
    need = int(lib.mla_rpa_workspace_size(ctypes.byref(meta), H, Dl))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ql_nope.device)
    st = lib.mla_rpa_forward(_ptr(ql_nope), _ptr(q_pe), _ptr(new_kv_c), _ptr(new_k_pe),
                             _ptr(cache_kv_c), _ptr(cache_k_pe), _dtype_code(ql_nope), H, Dl, Dr,
                             kvc_stride, kpe_stride, P, ps, ctypes.byref(meta), ctypes.byref(opts),
                             _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _raise(lib, st)
    return out


def sparse_mla_forward(q, kv_cache, page_table, indices, positions, *, seq_len, read_block,
                       sm_scale, kv_lora_rank=512, rope_dim=64, out=None, stream=None):
    """Sparse MLA-latent attention over a fused paged latent pool.

    q [S, H, 576] bf16; kv_cache [P, ps, C] bf16; page_table [PTW]; indices [S, K]
    (-1 = padding); positions [S] (int32). Returns out [S, H, 512] fp32.
    """
    torch = _torch()
    lib = load_library()
    _check_dev(q, kv_cache, page_table, indices, positions, out)
    S, H, Dk = q.shape
    if Dk != kv_lora_rank + rope_dim:
        raise ValueError("q last dim must be kv_lora_rank + rope_dim")
    P, ps, C = kv_cache.shape
    K = indices.shape[1]
    if out is None:
        out = torch.empty((S, H, kv_lora_rank), dtype=torch.float32, device=q.device)
    st = lib.sparse_mla_forward(_ptr(q), _ptr(kv_cache), _ptr(_i32(page_table)),
                                _ptr(_i32(indices)), _ptr(_i32(positions)), int(seq_len), S, H, K,
                                int(read_block), ps, P, C, page_table.numel(), kv_lora_rank,
                                rope_dim, float(sm_scale), _ptr(out), _stream(stream))
    _raise(lib, st)
    return out


def sparse_mla_forward_ragged(q, kv_cache, page_indices, indices, positions, cu_q_lens, seq_lens,
                              cu_kv_lens, *, read_block, sm_scale, kv_lora_rank=512, rope_dim=64,
                              out=None, stream=None):
    """Sparse MLA-latent attention over packed tokens of several requests.

    q [T, H, 576] bf16; kv_cache [P, ps, C] bf16; page_indices [PTW] packed page
    list; indices [T, K] request-local unit ids (-1 = padding); positions [T];
    cu_q_lens [R+1]; seq_lens [R]; cu_kv_lens [R+1] (all int32, on the device).
    Returns out [T, H, 512] fp32.
    """
    torch = _torch()
    lib = load_library()
    _check_dev(q, kv_cache, page_indices, indices, positions, cu_q_lens, seq_lens, cu_kv_lens, out)
    T, H, Dk = q.shape
    if Dk != kv_lora_rank + rope_dim:
        raise ValueError("q last dim must be kv_lora_rank + rope_dim")
    P, ps, C = kv_cache.shape
    K = indices.shape[1]
    R = seq_lens.numel()
    if cu_q_lens.numel() != R + 1 or cu_kv_lens.numel() != R + 1:
        raise ValueError("cu_q_lens and cu_kv_lens need len(seq_lens) + 1 entries")
    if out is None:
        out = torch.empty((T, H, kv_lora_rank), dtype=torch.float32, device=q.device)
    st = lib.sparse_mla_forward_ragged(
        _ptr(q), _ptr(kv_cache), _ptr(_i32(page_indices)), page_indices.numel(), _ptr(_i32(indices)),
        _ptr(_i32(positions)), _ptr(_i32(cu_q_lens)), _ptr(_i32(seq_lens)), _ptr(_i32(cu_kv_lens)), R,
        T, H, K, int(read_block), ps, P, C, kv_lora_rank, rope_dim, float(sm_scale), _ptr(out),
        _stream(stream))
    _raise(lib, st)
    return out
