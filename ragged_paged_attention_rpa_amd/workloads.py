"""Seeded synthetic inputs for ragged paged attention.

This module only draws random numbers and lays them out (pools, page tables,
ragged metadata); it holds none of the attention arithmetic, and it imports
neither the HIP binding nor the oracle, so both sides can use it.

Shapes follow the five workloads the pages' kernels are built for:

* ``tiny_gqa``      3 sequences, q_lens {1,1,8}, kv_lens {5,17,40}, 8/2 heads,
                    head_dim 128, page 16, 16-page pool, fp32.
* ``decode_gqa``    128 decodes, kv_len U[512,8192], 32/8 heads, head_dim 128,
                    page 16, bf16, combined interleaved K/V pool, shuffled pages.
* ``mixed_gqa``     120 decodes (kv U[256,8192]) then 8 prefill chunks
                    (q_len U[512,2048], kv_len U[q_len,8192]); fp8 e4m3fn KV
                    stored as N(0,1)/0.5 with k_scale = v_scale = 0.5,
                    window 4096, soft cap 50, bf16 queries.
* ``mla_decode``    64 decodes, kv_len U[4096,32768] after the update,
                    128 heads, latent 512 + rope 64 (padded to 128), page 64.
* ``sparse_mla``    one 65536-token latent sequence, 4096 queries at the last
                    positions, 32 distinct causal page units of 64 tokens each.

Integer metadata comes from ``numpy.random.default_rng(seed)``; tensors from a
seeded ``torch.Generator`` on the requested device (values N(0,1) in fp32,
rounded to the storage dtype by torch's own cast).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype, gen, device, scale=1.0):
    """N(0,1)*scale drawn in fp32 and cast to ``dtype`` (bf16/fp8/fp32); for
    int8, the integers round(32 * N(0,1) * scale) clipped to [-128, 127] (a pool
    quantised at 1/32 per step, dequantised by a scale of 1/32); for uint8, a
    packed int4 array: the integers round(2 * N(0,1) * scale) clipped to
    [-8, 7], two per byte along the last index (element 2i in the low nibble),
    so the result's last dimension is half of ``shape``'s."""
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    if dtype == torch.int8:
        return x.mul_(32.0).round_().clamp_(-128, 127).to(torch.int8)
    if dtype == torch.uint8:
        return pack_int4(x.mul_(2.0).round_().clamp_(-8, 7).to(torch.int16))
    return x.to(dtype)


def pack_int4(v):
    """Integers in [-8, 7] (last dimension even) as packed int4 bytes: element
    2i in the low nibble of byte i, each a two's-complement nibble."""
    n = v.to(torch.int16) & 15
    return (n[..., 0::2] | (n[..., 1::2] << 4)).to(torch.uint8)


def deal_pages(rng, kv_lens, page_size, pages_per_seq, spare_pages=0):
    """Gives each sequence cdiv(kv_len, ps) pages from one shuffled pool.

    Table entries past a sequence's last page are filled with random (valid)
    page ids, like stale entries left by an earlier step.
    Returns (total_num_pages, page_indices int32 [S, pages_per_seq]).
    """
    need = [cdiv(int(L), page_size) for L in kv_lens]
    if max(need, default=0) > pages_per_seq:
        raise ValueError("pages_per_seq too small for kv_lens")
    total = int(sum(need)) + int(spare_pages)
    total = max(total, 1)
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((len(kv_lens), pages_per_seq), dtype=np.int32)
    off = 0
    for i, n in enumerate(need):
        table[i, :n] = perm[off:off + n]
        off += n
        table[i, n:] = rng.integers(0, total, pages_per_seq - n, dtype=np.int32)
    return total, table


@dataclass
class GqaCase:
    """One ragged paged GQA batch (all tensors on ``device``)."""
    name: str
    q: torch.Tensor                # [T, Hq, D]
    kv_pages: torch.Tensor         # [P, ps, 2*Hkv, D]
    kv_lens: np.ndarray            # int32 [max_num_seqs]
    page_indices: np.ndarray       # int32 [max_num_seqs, pages_per_seq]
    cu_q_lens: np.ndarray          # int32 [max_num_seqs + 1]
    num_seqs: int
    sm_scale: float
    sliding_window: int | None = None
    soft_cap: float | None = None
    k_scale: float | None = None
    v_scale: float | None = None
    extra: dict = field(default_factory=dict)

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def num_kv_heads(self):
        return self.kv_pages.shape[2] // 2

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def page_size(self):
        return self.kv_pages.shape[1]


def ragged_meta(q_lens, kv_lens, max_num_seqs=None):
    """cu_q_lens / kv_lens padded to max_num_seqs (padding: q_len 0, kv_len 0)."""
    S = len(q_lens)
    m = max_num_seqs or S
    cu = np.zeros(m + 1, dtype=np.int32)
    cu[1:S + 1] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    cu[S + 1:] = cu[S]
    kl = np.zeros(m, dtype=np.int32)
    kl[:S] = kv_lens
    return cu, kl


def make_gqa(seqs, *, num_q_heads, num_kv_heads, head_dim, page_size, q_dtype, kv_dtype,
             seed, device="cpu", pages_per_seq=None, spare_pages=2, kv_value_scale=1.0,
             q_value_scale=1.0, sm_scale=None, sliding_window=None, soft_cap=None,
             k_scale=None, v_scale=None, max_num_seqs=None, extra_tokens=0, name="gqa"):
    """Random ragged GQA batch. ``seqs`` is a list of (q_len, kv_len)."""
    rng = np.random.default_rng(seed)
    gen = _gen(device, seed)
    q_lens = [s[0] for s in seqs]
    kv_lens = [s[1] for s in seqs]
    pps = pages_per_seq or max(1, max(cdiv(L, page_size) for L in kv_lens) if seqs else 1)
    P, table = deal_pages(rng, kv_lens, page_size, pps, spare_pages)
    m = max_num_seqs or len(seqs)
    full_table = np.zeros((m, pps), dtype=np.int32)
    full_table[:len(seqs)] = table
    cu, kl = ragged_meta(q_lens, kv_lens, m)
    T = int(cu[-1]) + int(extra_tokens)
    q = randn((max(T, 1), num_q_heads, head_dim), q_dtype, gen, device, q_value_scale)
    kv = randn((P, page_size, 2 * num_kv_heads, head_dim), kv_dtype, gen, device,
               kv_value_scale)
    return GqaCase(name=name, q=q, kv_pages=kv, kv_lens=kl, page_indices=full_table,
                   cu_q_lens=cu, num_seqs=len(seqs),
                   sm_scale=sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim),
                   sliding_window=sliding_window, soft_cap=soft_cap, k_scale=k_scale,
                   v_scale=v_scale)


def tiny_gqa(device="cpu", seed=1001):
    """3 seqs, q_lens {1,1,8}, kv_lens {5,17,40}; 8/2 heads, d 128, page 16,
    16-page pool with page_indices = first 9 entries of a random permutation."""
    rng = np.random.default_rng(seed)
    gen = _gen(device, seed)
    perm = rng.permutation(16).astype(np.int32)
    table = perm[:9].reshape(3, 3).copy()
    cu = np.array([0, 1, 2, 10], dtype=np.int32)
    kl = np.array([5, 17, 40], dtype=np.int32)
    q = randn((10, 8, 128), torch.float32, gen, device)
    kv = randn((16, 16, 4, 128), torch.float32, gen, device)
    return GqaCase(name="tiny_gqa", q=q, kv_pages=kv, kv_lens=kl, page_indices=table,
                   cu_q_lens=cu, num_seqs=3, sm_scale=1.0 / math.sqrt(128))


def decode_gqa(device="cpu", seed=1002, num_seqs=128):
    """128 decodes, kv_len U[512,8192], 32/8 heads, d 128, page 16, bf16."""
    rng = np.random.default_rng(seed)
    kv_lens = rng.integers(512, 8192 + 1, num_seqs)
    seqs = [(1, int(L)) for L in kv_lens]
    return make_gqa(seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=seed + 7,
                    device=device, pages_per_seq=512, spare_pages=0, name="decode_gqa")


def mixed_gqa(device="cpu", seed=1003, shuffle_order=False, q_value_scale=1.0):
    """120 decodes (kv U[256,8192]) then 8 prefill chunks (q U[512,2048],
    kv U[q,8192]); fp8 KV (N(0,1)/0.5), scales 0.5, window 4096, cap 50."""
    rng = np.random.default_rng(seed)
    dec = [(1, int(L)) for L in rng.integers(256, 8192 + 1, 120)]
    pre = []
    for _ in range(8):
        ql = int(rng.integers(512, 2048 + 1))
        pre.append((ql, int(rng.integers(ql, 8192 + 1))))
    seqs = dec + pre
    if shuffle_order:
        order = rng.permutation(len(seqs))
        seqs = [seqs[i] for i in order]
    return make_gqa(seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.float8_e4m3fn, seed=seed + 7,
                    device=device, pages_per_seq=512, spare_pages=0, kv_value_scale=2.0,
                    q_value_scale=q_value_scale, sm_scale=1.0 / math.sqrt(128),
                    sliding_window=4096, soft_cap=50.0, k_scale=0.5, v_scale=0.5,
                    name="mixed_gqa")


@dataclass
class MlaCase:
    """One MLA latent batch: queries, new tokens and the split paged caches."""
    name: str
    ql_nope: torch.Tensor     # [T, H, Dl]
    q_pe: torch.Tensor        # [T, H, Dr]
    new_kv_c: torch.Tensor    # [T, Dl]
    new_k_pe: torch.Tensor    # [T, Dr]
    cache_kv_c: torch.Tensor  # [P, ps, Dl_pad]
    cache_k_pe: torch.Tensor  # [P, ps, Dr_pad]  (pad columns 0)
    kv_lens: np.ndarray
    page_indices: np.ndarray
    cu_q_lens: np.ndarray
    num_seqs: int
    sm_scale: float
    sliding_window: int | None = None
    soft_cap: float | None = None

    @property
    def page_size(self):
        return self.cache_kv_c.shape[1]


def make_mla(seqs, *, num_heads, lkv_dim=512, r_dim=64, page_size=64, dtype=torch.bfloat16,
             seed=0, device="cpu", pages_per_seq=None, spare_pages=1, sm_scale=None,
             sliding_window=None, soft_cap=None, name="mla"):
    """Random MLA batch; ``seqs`` = [(q_len, kv_len_after_update)]."""
    rng = np.random.default_rng(seed)
    gen = _gen(device, seed)
    q_lens = [s[0] for s in seqs]
    kv_lens = [s[1] for s in seqs]
    pps = pages_per_seq or max(cdiv(L, page_size) for L in kv_lens)
    P, table = deal_pages(rng, kv_lens, page_size, pps, spare_pages)
    cu, kl = ragged_meta(q_lens, kv_lens)
    T = int(cu[-1])
    lkv_pad = cdiv(lkv_dim, 128) * 128
    r_pad = cdiv(r_dim, 128) * 128
    ql_nope = randn((T, num_heads, lkv_dim), dtype, gen, device)
    q_pe = randn((T, num_heads, r_dim), dtype, gen, device)
    new_kv_c = randn((T, lkv_dim), dtype, gen, device)
    new_k_pe = randn((T, r_dim), dtype, gen, device)
    cache_kv_c = torch.zeros((P, page_size, lkv_pad), dtype=dtype, device=device)
    cache_kv_c[:, :, :lkv_dim] = randn((P, page_size, lkv_dim), dtype, gen, device)
    cache_k_pe = torch.zeros((P, page_size, r_pad), dtype=dtype, device=device)
    cache_k_pe[:, :, :r_dim] = randn((P, page_size, r_dim), dtype, gen, device)
    return MlaCase(name=name, ql_nope=ql_nope, q_pe=q_pe, new_kv_c=new_kv_c,
                   new_k_pe=new_k_pe, cache_kv_c=cache_kv_c, cache_k_pe=cache_k_pe,
                   kv_lens=kl, page_indices=table, cu_q_lens=cu, num_seqs=len(seqs),
                   sm_scale=sm_scale if sm_scale is not None else 1.0 / math.sqrt(192),
                   sliding_window=sliding_window, soft_cap=soft_cap)


def mla_decode(device="cpu", seed=1004, num_seqs=64):
    """64 decodes, kv_len U[4096,32768] after the update, 128 heads, page 64."""
    rng = np.random.default_rng(seed)
    seqs = [(1, int(L)) for L in rng.integers(4096, 32768 + 1, num_seqs)]
    return make_mla(seqs, num_heads=128, page_size=64, seed=seed + 7, device=device,
                    pages_per_seq=512, spare_pages=0, name="mla_decode")


@dataclass
class SparseCase:
    """One sparse MLA batch over a fused paged latent pool."""
    name: str
    q: torch.Tensor            # [S, H, Dk]
    kv_cache: torch.Tensor     # [P, ps, 640]  (cols >= Dk are 0)
    page_table: np.ndarray     # int32 [PTW]
    indices: np.ndarray        # int32 [S, K]
    positions: np.ndarray      # int32 [S]
    seq_len: int
    read_block: int
    sm_scale: float
    kv_lora_rank: int = 512
    rope_dim: int = 64

    @property
    def page_size(self):
        return self.kv_cache.shape[1]


def sample_units(rng, positions, K, read_block, pad_frac=0.0):
    """For each query position p: K distinct unit ids drawn uniformly without
    replacement from {0..p//RB}, sorted (fewer available -> -1 padding)."""
    S = len(positions)
    out = np.full((S, K), -1, dtype=np.int32)
    for s, p in enumerate(positions):
        n_units = int(p) // read_block + 1
        k = min(K, n_units)
        if pad_frac > 0.0:
            k = max(0, k - int(rng.integers(0, int(K * pad_frac) + 1)))
        sel = np.sort(rng.choice(n_units, size=k, replace=False)).astype(np.int32)
        out[s, :k] = sel
    return out


def make_sparse(*, T, S, H, K, page_size=64, read_block=64, dtype=torch.bfloat16, seed=0,
                device="cpu", kv_lora_rank=512, rope_dim=64, pad_cols=640, positions=None,
                pad_frac=0.0, name="sparse"):
    rng = np.random.default_rng(seed)
    gen = _gen(device, seed)
    dk = kv_lora_rank + rope_dim
    n_pages = cdiv(T, page_size)
    page_table = rng.permutation(n_pages).astype(np.int32)
    if positions is None:
        positions = np.arange(T - S, T, dtype=np.int32)
    positions = np.asarray(positions, dtype=np.int32)
    indices = sample_units(rng, positions, K, read_block, pad_frac)
    q = randn((S, H, dk), dtype, gen, device)
    kv = torch.zeros((n_pages, page_size, pad_cols), dtype=dtype, device=device)
    kv[:, :, :dk] = randn((n_pages, page_size, dk), dtype, gen, device)
    return SparseCase(name=name, q=q, kv_cache=kv, page_table=page_table, indices=indices,
                      positions=positions, seq_len=T, read_block=read_block,
                      sm_scale=1.0 / math.sqrt(192), kv_lora_rank=kv_lora_rank,
                      rope_dim=rope_dim)


@dataclass
class SparseRaggedCase:
    """Packed tokens of several requests over one fused paged latent pool
    (the sparse page's packed-ragged mode)."""
    name: str
    q: torch.Tensor            # [T, H, Dk] packed tokens (T may exceed cu_q_lens[-1]: padding)
    kv_cache: torch.Tensor     # [P, ps, pad_cols]
    page_indices: np.ndarray   # int32 [PTW] packed physical pages, request r's from cu_kv_lens[r]//ps
    indices: np.ndarray        # int32 [T, K] request-local unit ids (-1 = padding)
    positions: np.ndarray      # int32 [T]
    cu_q_lens: np.ndarray      # int32 [R+1]
    seq_lens: np.ndarray       # int32 [R]
    cu_kv_lens: np.ndarray     # int32 [R+1] page-aligned
    read_block: int
    sm_scale: float
    kv_lora_rank: int = 512
    rope_dim: int = 64

    @property
    def page_size(self):
        return self.kv_cache.shape[1]


def make_sparse_ragged(*, seq_lens, q_lens, H, K, page_size=64, read_block=64,
                       dtype=torch.bfloat16, seed=0, device="cpu", kv_lora_rank=512, rope_dim=64,
                       pad_cols=640, pad_tokens=0, spare_pages=3, pad_frac=0.0,
                       name="sparse_ragged"):
    """Requests r = 0..R-1 with kv length seq_lens[r] whose last q_lens[r]
    tokens are queries (positions seq_lens[r] - q_lens[r] .. seq_lens[r] - 1),
    packed in request order, then pad_tokens extra tokens (positions of the
    last request's last token). Each request owns ceil(seq_len / ps) pages of
    the packed table, at page-aligned offsets cu_kv_lens; the physical pages
    are a random permutation of the pool (plus spare_pages never referenced)."""
    rng = np.random.default_rng(seed)
    gen = _gen(device, seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    R = len(seq_lens)
    dk = kv_lora_rank + rope_dim
    pages = np.array([cdiv(int(L), page_size) for L in seq_lens], dtype=np.int64)
    cu_kv_lens = np.zeros(R + 1, dtype=np.int32)
    cu_kv_lens[1:] = np.cumsum(pages * page_size)
    n_pages = int(pages.sum()) + spare_pages
    page_indices = rng.permutation(n_pages)[: int(pages.sum())].astype(np.int32)
    cu_q_lens = np.zeros(R + 1, dtype=np.int32)
    cu_q_lens[1:] = np.cumsum(q_lens)
    positions = np.concatenate(
        [np.arange(L - ql, L, dtype=np.int32) for L, ql in zip(seq_lens, q_lens)]
        + [np.full(pad_tokens, seq_lens[-1] - 1, dtype=np.int32)])
    T = len(positions)
    indices = sample_units(rng, positions, K, read_block, pad_frac)
    q = randn((T, H, dk), dtype, gen, device)
    kv = torch.zeros((n_pages, page_size, pad_cols), dtype=dtype, device=device)
    kv[:, :, :dk] = randn((n_pages, page_size, dk), dtype, gen, device)
    return SparseRaggedCase(name=name, q=q, kv_cache=kv, page_indices=page_indices,
                            indices=indices, positions=positions, cu_q_lens=cu_q_lens,
                            seq_lens=seq_lens, cu_kv_lens=cu_kv_lens, read_block=read_block,
                            sm_scale=1.0 / math.sqrt(192), kv_lora_rank=kv_lora_rank,
                            rope_dim=rope_dim)


def sparse_mla(device="cpu", seed=1005):
    """T=65536 latent tokens, 4096 queries at T-4096..T-1, 16 heads,
    K=32 distinct causal units of 64 tokens (page-level selection)."""
    return make_sparse(T=65536, S=4096, H=16, K=32, page_size=64, read_block=64, seed=seed,
                       device=device, name="sparse_mla")
