"""Pins for the CPU oracle (no GPU): each check ties the oracle to something
other than itself — a format definition, a hand-derived worked example, a
library routine on a dense unpaged layout, a closed form or an invariant.

Pages cited by short name: "RPA v2 page" (ragged_paged_attention v2 kernel),
"MLA v1 page" (MLA ragged paged attention v1 kernel), "Sparse page" (sparse
MLA prefill kernel).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from ragged_paged_attention_rpa_amd import workloads as wl
from tests.helpers import storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_derived.json")


# ----------------------------------------------------------------- decoders --

def test_decoders_match_format_definitions():
    # bf16 worked values from the binary32 layout (upper half of a float).
    assert oracle.decode_bf16(0x3F80) == 1.0
    assert oracle.decode_bf16(0xC000) == -2.0
    assert oracle.decode_bf16(0x3FC0) == 1.5
    assert math.isinf(oracle.decode_bf16(0x7F80))
    assert oracle.decode_bf16(0x0001) == 2.0 ** -133
    # OCP e4m3fn worked values: bias 7, no inf, S.1111.111 = NaN.
    assert oracle.decode_e4m3fn(0x38) == 1.0
    assert oracle.decode_e4m3fn(0xB8) == -1.0
    assert oracle.decode_e4m3fn(0x3C) == 1.5
    assert oracle.decode_e4m3fn(0x7E) == 448.0
    assert oracle.decode_e4m3fn(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3fn(0x01) == 2.0 ** -9
    assert math.isnan(oracle.decode_e4m3fn(0x7F))


def test_decoders_match_torch_for_every_fp8_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3fn(int(c)) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_matches_torch_on_random_codes():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 1 << 16, 4000).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ----------------------------------------------------- hand-derived golden --

def _coord(tok):
    ln2, ln3 = math.log(2.0), math.log(3.0)
    table = {"0": 0.0, "ln2": ln2, "ln3": ln3, "2ln2": 2 * ln2, "2ln3": 2 * ln3,
             "3ln3*ln2/2": 3 * ln3 * ln2 / 2}
    return table[tok]


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_rpa_hand_derived(case):
    """One sequence, head_dim 2, page size 2, pages in reverse physical order."""
    kv_len, q_len = case["kv_len"], case["q_len"]
    ps, D = 2, 2
    n_pages = -(-kv_len // ps)
    P = n_pages + 1
    pool = np.full((P, ps, 2, D), np.nan, dtype=np.float32)  # unused rows are NaN
    table = np.array([[P - 1 - lp for lp in range(n_pages)]], dtype=np.int32)
    for t in range(kv_len):
        page, row = table[0, t // ps], t % ps
        pool[page, row, 0] = [_coord(case["key_first_coord"][t]), 0.0]
        pool[page, row, 1] = case["values"][t]
    q = np.zeros((q_len, 1, D), dtype=np.float32)
    q[:, 0, 0] = 1.0
    cap = case["soft_cap"]
    cap = 3 * math.log(3.0) if cap == "3ln3" else float(cap)
    out = oracle.rpa(q, oracle.F32, pool, oracle.F32, [kv_len], table, [0, q_len], 1,
                     sm_scale=1.0, sliding_window=case["window"] or None,
                     soft_cap=cap or None, k_scale=case["k_scale"], v_scale=case["v_scale"])
    np.testing.assert_allclose(out[:, 0, :], np.array(case["expected"], float), rtol=0,
                               atol=2e-6)


def test_gqa_head_mapping():
    """q head h reads kv head h // (Hq/Hkv) [RPA v2 page: jnp.repeat of K/V heads]."""
    Hq, Hkv, D, ps = 4, 2, 8, 4
    pool = np.zeros((1, ps, 2 * Hkv, D), dtype=np.float32)
    pool[0, :, 1, :] = 1.0  # V of kv head 0
    pool[0, :, 3, :] = 2.0  # V of kv head 1
    rng = np.random.default_rng(0)
    pool[0, :, 0, :] = rng.standard_normal((ps, D))
    pool[0, :, 2, :] = rng.standard_normal((ps, D))
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = oracle.rpa(q, oracle.F32, pool, oracle.F32, [3], [[0]], [0, 1], 1)
    np.testing.assert_array_equal(out[0, :, 0], [1.0, 1.0, 2.0, 2.0])


# ------------------------------------------- dense library attention (SDPA) --

def _sdpa(q, k, v, mask, scale):
    """torch SDPA in fp64 on CPU: q [Hq, n_q, D], k/v [Hq, n_k, *], mask [n_q, n_k]."""
    return F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None, None],
                                          scale=scale)[0]


def _dense_gqa_case(rng, seqs, Hq, Hkv, D, ps, window, k_scale, v_scale):
    """Builds per-sequence dense K/V first, then scatters them into a shuffled
    paged pool (written here, independently of the oracle)."""
    S = len(seqs)
    pps = max(-(-kv // ps) for _, kv in seqs) + 1
    need = [-(-kv // ps) for _, kv in seqs]
    P = sum(need) + 3
    perm = rng.permutation(P)
    table = rng.integers(0, P, (S, pps)).astype(np.int32)
    pool = rng.standard_normal((P, ps, 2 * Hkv, D)).astype(np.float32)
    Ks, Vs = [], []
    off = 0
    for i, (ql, kv) in enumerate(seqs):
        table[i, :need[i]] = perm[off:off + need[i]]
        off += need[i]
        K = rng.standard_normal((kv, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((kv, Hkv, D)).astype(np.float32)
        for t in range(kv):
            pg, r = table[i, t // ps], t % ps
            pool[pg, r, 0::2] = K[t]
            pool[pg, r, 1::2] = V[t]
        Ks.append(K)
        Vs.append(V)
    cu = np.concatenate([[0], np.cumsum([s[0] for s in seqs])]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float32)
    G = Hq // Hkv
    want = np.zeros((int(cu[-1]), Hq, D))
    for i, (ql, kv) in enumerate(seqs):
        qpos = kv - ql + np.arange(ql)
        kpos = np.arange(kv)
        mask = kpos[None, :] <= qpos[:, None]
        if window:
            mask &= kpos[None, :] > qpos[:, None] - window
        qi = torch.from_numpy(q[cu[i]:cu[i + 1]].astype(np.float64)).transpose(0, 1)
        ki = torch.from_numpy(Ks[i].astype(np.float64) * k_scale).transpose(0, 1)
        vi = torch.from_numpy(Vs[i].astype(np.float64) * v_scale).transpose(0, 1)
        ki = ki.repeat_interleave(G, dim=0)
        vi = vi.repeat_interleave(G, dim=0)
        o = _sdpa(qi, ki, vi, torch.from_numpy(mask), 1.0 / math.sqrt(D))
        want[cu[i]:cu[i + 1]] = o.transpose(0, 1).numpy()
    return q, pool, table, cu, np.array([s[1] for s in seqs], np.int32), want


@pytest.mark.parametrize("seed,Hq,Hkv,D,ps,window,ks,vs", [
    (1, 8, 2, 16, 4, 0, 1.0, 1.0),
    (2, 4, 4, 8, 2, 3, 1.0, 1.0),
    (3, 6, 1, 32, 8, 5, 0.5, 2.0),
    (4, 16, 4, 64, 16, 0, 0.25, 0.75),
])
def test_rpa_matches_dense_sdpa(seed, Hq, Hkv, D, ps, window, ks, vs):
    rng = np.random.default_rng(seed)
    seqs = [(1, 1), (1, 9), (5, 5), (3, 17), (7, 30), (1, 2 * ps), (4, 4 * ps + 1)]
    q, pool, table, cu, kl, want = _dense_gqa_case(rng, seqs, Hq, Hkv, D, ps, window, ks, vs)
    got = oracle.rpa(q, oracle.F32, pool, oracle.F32, kl, table, cu, len(seqs),
                     sm_scale=1.0 / math.sqrt(D), sliding_window=window or None,
                     k_scale=ks, v_scale=vs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


# ------------------------------------------------------------- invariants --

def _tiny():
    c = wl.tiny_gqa()
    q, qd = storage(c.q)
    kv, kd = storage(c.kv_pages)
    return c, q, qd, kv, kd


def test_kv_len_one_returns_v0_exactly():
    rng = np.random.default_rng(9)
    pool = rng.standard_normal((3, 4, 4, 16)).astype(np.float32)
    q = rng.standard_normal((1, 4, 16)).astype(np.float32)
    out = oracle.rpa(q, oracle.F32, pool, oracle.F32, [1], [[2]], [0, 1], 1, v_scale=0.5)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], pool[2, 0, 2 * (h // 2) + 1].astype(np.float64) * 0.5)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(10)
    c = wl.make_gqa([(3, 20), (1, 7)], num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=4,
                    q_dtype=torch.float32, kv_dtype=torch.float32, seed=10)
    q = np.zeros(tuple(c.q.shape), np.float32)
    kv, _ = storage(c.kv_pages)
    W = 6
    out = oracle.rpa(q, oracle.F32, kv, oracle.F32, c.kv_lens, c.page_indices, c.cu_q_lens,
                     c.num_seqs, sliding_window=W)
    for i in range(c.num_seqs):
        ql = c.cu_q_lens[i + 1] - c.cu_q_lens[i]
        L = c.kv_lens[i]
        logical = np.stack([kv[c.page_indices[i, t // 4], t % 4] for t in range(L)])
        for r in range(ql):
            p = L - ql + r
            vis = [t for t in range(L) if p - W < t <= p]
            for h in range(4):
                want = logical[vis, 2 * (h // 2) + 1].astype(np.float64).mean(0)
                np.testing.assert_allclose(out[c.cu_q_lens[i] + r, h], want, atol=1e-12)


def test_page_permutation_invariance_bit_exact():
    c, q, qd, kv, kd = _tiny()
    base = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale)
    rng = np.random.default_rng(77)
    perm = rng.permutation(kv.shape[0])          # new physical slot of old page p
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    table2 = perm[c.page_indices].astype(np.int32)
    got = oracle.rpa(q, qd, kv2, kd, c.kv_lens, table2, c.cu_q_lens, 3, sm_scale=c.sm_scale)
    assert np.array_equal(got, base)


def test_nan_in_unused_pages_and_tail_rows_is_never_read():
    c, q, qd, kv, kd = _tiny()
    base = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale)
    kv2 = kv.copy()
    used = set()
    for i in range(3):
        L = c.kv_lens[i]
        for t in range(-(-L // 16) * 16):
            pg = c.page_indices[i, t // 16]
            if t >= L:
                kv2[pg, t % 16] = np.nan
            used.add(int(pg))
    for pg in range(kv.shape[0]):
        if pg not in used:
            kv2[pg] = np.nan
    got = oracle.rpa(q, qd, kv2, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale)
    assert np.array_equal(got, base)


def test_window_at_least_kv_len_equals_no_window_and_huge_cap_equals_no_cap():
    c, q, qd, kv, kd = _tiny()
    base = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale)
    win = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale,
                     sliding_window=40)
    assert np.array_equal(win, base)
    cap = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale,
                     soft_cap=1e9)
    np.testing.assert_allclose(cap, base, atol=1e-12)
    small_win = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3,
                           sm_scale=c.sm_scale, sliding_window=4)
    assert not np.allclose(small_win[2:], base[2:])


def test_last_prefill_row_equals_decode_of_same_sequence():
    c, q, qd, kv, kd = _tiny()
    base = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, 3, sm_scale=c.sm_scale)
    # Sequence 2 is an 8-token prefill over 40 keys; a decode of its last token
    # (q_len 1, same kv_len) must give the same row.
    dec = oracle.rpa(q[9:10], qd, kv, kd, c.kv_lens[2:3], c.page_indices[2:3], [0, 1], 1,
                     sm_scale=c.sm_scale)
    assert np.array_equal(dec[0], base[9])


def test_oracle_rejects_q_len_above_kv_len():
    c, q, qd, kv, kd = _tiny()
    with pytest.raises(oracle.OracleError):
        oracle.rpa(q, qd, kv, kd, [5, 17, 7], c.page_indices, c.cu_q_lens, 3)


# ---------------------------------------------------------------------- MLA --

def test_mla_matches_dense_sdpa_mqa():
    """K = [kv_c || k_pe], V = kv_c, shared by all heads [MLA v1 page:
    ref_mla_ragged_paged_attention]."""
    c = wl.make_mla([(1, 70), (3, 3), (5, 129)], num_heads=4, lkv_dim=32, r_dim=8,
                    page_size=16, dtype=torch.float32, seed=11)
    ql, d = storage(c.ql_nope)
    qp, _ = storage(c.q_pe)
    ckv, _ = storage(c.cache_kv_c)
    ckp, _ = storage(c.cache_k_pe)
    got = oracle.mla(ql, qp, d, ckv, ckp, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs,
                     sm_scale=c.sm_scale)
    for i in range(c.num_seqs):
        L, ql_i = int(c.kv_lens[i]), int(c.cu_q_lens[i + 1] - c.cu_q_lens[i])
        rows = [c.page_indices[i, t // 16] * 16 + t % 16 for t in range(L)]
        kvc = ckv.reshape(-1, ckv.shape[2])[rows, :32].astype(np.float64)
        kpe = ckp.reshape(-1, ckp.shape[2])[rows, :8].astype(np.float64)
        K = torch.from_numpy(np.concatenate([kvc, kpe], 1))[None].expand(4, -1, -1)
        V = torch.from_numpy(kvc)[None].expand(4, -1, -1)
        sl = slice(c.cu_q_lens[i], c.cu_q_lens[i + 1])
        Q = torch.from_numpy(np.concatenate([ql[sl], qp[sl]], 2).astype(np.float64)).transpose(0, 1)
        qpos = L - ql_i + np.arange(ql_i)
        mask = torch.from_numpy(np.arange(L)[None, :] <= qpos[:, None])
        want = _sdpa(Q, K, V, mask, c.sm_scale).transpose(0, 1).numpy()
        np.testing.assert_allclose(got[sl], want, atol=1e-10)


def test_mla_fused_pool_equals_split_pool():
    c = wl.make_mla([(2, 40), (1, 65)], num_heads=3, lkv_dim=32, r_dim=8, page_size=16,
                    dtype=torch.float32, seed=12)
    ql, d = storage(c.ql_nope)
    qp, _ = storage(c.q_pe)
    ckv, _ = storage(c.cache_kv_c)
    ckp, _ = storage(c.cache_k_pe)
    fused = np.zeros(ckv.shape[:2] + (64,), np.float32)
    fused[:, :, :32] = ckv[:, :, :32]
    fused[:, :, 32:40] = ckp[:, :, :8]
    a = oracle.mla(ql, qp, d, ckv, ckp, c.kv_lens, c.page_indices, c.cu_q_lens, 2)
    b = oracle.mla(ql, qp, d, fused, None, c.kv_lens, c.page_indices, c.cu_q_lens, 2, fused=True)
    assert np.array_equal(a, b)


# ------------------------------------------------------ scales and int8 KV --

def _gqa_small(seed):
    return wl.make_gqa([(3, 20), (1, 7), (6, 40), (1, 1)], num_q_heads=8, num_kv_heads=2,
                       head_dim=16, page_size=4, q_dtype=torch.float32, kv_dtype=torch.float32,
                       seed=seed)




def test_q_scale_multiplies_the_scores():
    """q_scale dequantises Q, so it enters the scores like sm_scale does and
    leaves the values alone; a power of two keeps the products exact, so the
    two calls agree bit for bit."""
    c = _gqa_small(seed=90)
    q, qd = storage(c.q)
    kv, kd = storage(c.kv_pages)
    args = (q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs)
    a = oracle.rpa(*args, sm_scale=c.sm_scale, q_scale=4.0)
    b = oracle.rpa(*args, sm_scale=4.0 * c.sm_scale)
    assert np.array_equal(a, b)
    assert not np.allclose(a, oracle.rpa(*args, sm_scale=c.sm_scale), atol=1e-6)


def test_mla_scales_follow_the_page_kernel():
    """The MLA page's kernel multiplies the scores by k_scale and q_scale and
    the value sum by v_scale: with powers of two that is sm_scale * k * q on
    the scores and v on the output, exactly."""
    c = wl.make_mla([(2, 70), (1, 33)], num_heads=3, lkv_dim=16, r_dim=8, page_size=8,
                    dtype=torch.float32, seed=91)
    ql, d = storage(c.ql_nope)
    qp, _ = storage(c.q_pe)
    ckv, _ = storage(c.cache_kv_c)
    ckp, _ = storage(c.cache_k_pe)
    args = (ql, qp, d, ckv, ckp, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs)
    a = oracle.mla(*args, sm_scale=0.25, q_scale=2.0, k_scale=4.0, v_scale=0.5)
    b = oracle.mla(*args, sm_scale=2.0)
    assert np.array_equal(a, 0.5 * b)


def test_int8_pool_is_its_integers():
    """An int8 pool holds two's-complement integers (negative bytes included):
    it gives exactly what an fp32 pool of the same integer values gives."""
    c = _gqa_small(seed=92)
    rng = np.random.default_rng(92)
    ints = rng.integers(-128, 128, size=tuple(c.kv_pages.shape)).astype(np.int8)
    q, qd = storage(c.q)
    meta = (c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs)
    a = oracle.rpa(q, qd, ints, oracle.INT8, *meta, sm_scale=c.sm_scale, k_scale=0.02,
                   v_scale=0.03)
    b = oracle.rpa(q, qd, ints.astype(np.float32), oracle.F32, *meta, sm_scale=c.sm_scale,
                   k_scale=0.02, v_scale=0.03)
    assert np.array_equal(a, b)


def _pack_nibbles(ints):
    """Test-side packing of integers in [-8, 7]: element 2i in the low four bits
    of byte i (the RPA_INT4 layout)."""
    n = ints.astype(np.int16) & 15
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def test_int4_pool_is_its_integers():
    """A packed int4 pool holds two's-complement nibbles (negative values
    included) in element order: it gives exactly what an fp32 pool of the same
    integers gives."""
    c = _gqa_small(seed=93)
    rng = np.random.default_rng(93)
    ints = rng.integers(-8, 8, size=tuple(c.kv_pages.shape))
    q, qd = storage(c.q)
    meta = (c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs)
    a = oracle.rpa(q, qd, _pack_nibbles(ints), oracle.INT4, *meta, sm_scale=c.sm_scale,
                   k_scale=0.25, v_scale=0.5)
    b = oracle.rpa(q, qd, ints.astype(np.float32), oracle.F32, *meta, sm_scale=c.sm_scale,
                   k_scale=0.25, v_scale=0.5)
    assert np.array_equal(a, b)


def test_int4_bytes_by_hand():
    """One key, head_dim 2: the output is the key's V row times v_scale. Byte
    0x3F holds (-1, 3) (low nibble first), byte 0x78 holds (-8, 7)."""
    q = np.array([[[1.0, 0.0]]], dtype=np.float32)            # [T=1, Hq=1, D=2]
    meta = (np.array([1], np.int32), np.array([[0]], np.int32), np.array([0, 1], np.int32), 1)
    for vbyte, want in ((0x3F, (-1.0, 3.0)), (0x78, (-8.0, 7.0))):
        kv = np.array([[[[0x21], [vbyte]]]], dtype=np.uint8)   # [P=1, ps=1, 2, D/2=1]
        out = oracle.rpa(q, oracle.F32, kv, oracle.INT4, *meta, v_scale=0.5)
        assert np.array_equal(out[0, 0], 0.5 * np.array(want))


def test_int4_scatter_is_the_packed_int8_scatter():
    """Scattering packed int4 rows gives the packing of the same scatter done
    on int8 rows of the same integers."""
    rng = np.random.default_rng(94)
    P, ps, H, D = 6, 4, 2, 8
    kv_lens = np.array([5, 9], np.int32)
    cu = np.array([0, 2, 5], np.int32)
    table = np.array([[3, 1, 0], [5, 2, 4]], np.int32)
    pool = rng.integers(-8, 8, size=(P, ps, 2 * H, D)).astype(np.int8)
    nk = rng.integers(-8, 8, size=(5, H, D)).astype(np.int8)
    nv = rng.integers(-8, 8, size=(5, H, D)).astype(np.int8)
    meta = dict(kv_lens=kv_lens, page_indices=table, cu_q_lens=cu, num_seqs=2)
    packed = _pack_nibbles(pool)
    oracle.kv_update(oracle.LAYOUT_COMBINED_GQA, _pack_nibbles(nk), _pack_nibbles(nv), packed,
                     None, oracle.INT4, **meta)
    oracle.kv_update(oracle.LAYOUT_COMBINED_GQA, nk, nv, pool, None, oracle.INT8, **meta)
    assert np.array_equal(packed, _pack_nibbles(pool))


# ------------------------------------------------------------------ sparse --

def _sparse_small(seed=13, K=4, RB=16, ps=32, T=256, S=6, H=4, pad_frac=0.0):
    c = wl.make_sparse(T=T, S=S, H=H, K=K, page_size=ps, read_block=RB, dtype=torch.float32,
                       seed=seed, kv_lora_rank=32, rope_dim=8, pad_cols=48,
                       positions=np.sort(np.random.default_rng(seed).integers(0, T, S)),
                       pad_frac=pad_frac)
    return c


def _logical_rows(c, tokens):
    ps = c.page_size
    return [c.page_table[t // ps] * ps + t % ps for t in tokens]


def test_sparse_matches_sdpa_over_expanded_tokens():
    """Unit ids expand to RB consecutive tokens each [Sparse page:
    units_to_token_ids]; the key set is causal and bounded by seq_len, and a
    unit repeated in the selection counts once per occurrence."""
    c = _sparse_small(pad_frac=0.5)
    idx = c.indices.copy()
    idx[0, -1] = idx[0, 0]          # a duplicated unit
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    got = oracle.sparse_mla(q, d, kv, c.page_table, idx, c.positions, seq_len=c.seq_len,
                            read_block=c.read_block, sm_scale=c.sm_scale, dv=32)
    flat = kv.reshape(-1, kv.shape[2]).astype(np.float64)
    for s in range(q.shape[0]):
        toks = [u * c.read_block + r for u in idx[s] if u >= 0 for r in range(c.read_block)]
        toks = [t for t in toks if t <= c.positions[s] and t < c.seq_len]
        if not toks:
            np.testing.assert_array_equal(got[s], 0.0)
            continue
        rows = flat[_logical_rows(c, toks)]
        K = torch.from_numpy(rows[:, :40])[None].expand(4, -1, -1)
        V = torch.from_numpy(rows[:, :32])[None].expand(4, -1, -1)
        Q = torch.from_numpy(q[s].astype(np.float64))[:, None, :]
        mask = torch.ones((1, len(toks)), dtype=torch.bool)
        want = _sdpa(Q, K, V, mask, c.sm_scale)[:, 0, :].numpy()
        np.testing.assert_allclose(got[s], want, atol=1e-10)


def test_sparse_all_causal_units_equals_dense_causal_mla():
    c = _sparse_small(seed=14, K=16, RB=16, ps=32, T=256, S=5)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    S = q.shape[0]
    idx = np.full((S, 16), -1, np.int32)
    for s in range(S):
        n = c.positions[s] // 16 + 1
        idx[s, :n] = np.arange(n)
    got = oracle.sparse_mla(q, d, kv, c.page_table, idx, c.positions, seq_len=c.seq_len,
                            read_block=16, sm_scale=c.sm_scale, dv=32)
    # Same queries as a dense MLA over one sequence (decode of each position).
    for s in range(S):
        L = int(c.positions[s]) + 1
        table = np.zeros((1, 8), np.int32)
        table[0] = c.page_table[:8]
        ql = q[s:s + 1, :, :32].copy()
        qp = q[s:s + 1, :, 32:40].copy()
        dense = oracle.mla(ql, qp, d, kv, None, [L], table, [0, 1], 1, sm_scale=c.sm_scale,
                           fused=True)
        np.testing.assert_allclose(got[s], dense[0], atol=1e-12)


def test_sparse_empty_selection_gives_zero_and_padding_is_ignored():
    c = _sparse_small(seed=15)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    idx = c.indices.copy()
    idx[0] = -1
    got = oracle.sparse_mla(q, d, kv, c.page_table, idx, c.positions, seq_len=c.seq_len,
                            read_block=c.read_block, sm_scale=c.sm_scale, dv=32)
    np.testing.assert_array_equal(got[0], 0.0)
    idx2 = c.indices.copy()
    idx2[1, 1:] = -1
    a = oracle.sparse_mla(q, d, kv, c.page_table, idx2, c.positions, seq_len=c.seq_len,
                          read_block=c.read_block, sm_scale=c.sm_scale, dv=32)
    idx3 = np.full_like(idx2, -1)
    idx3[:, 0] = idx2[:, 0]
    b = oracle.sparse_mla(q, d, kv, c.page_table, idx3, c.positions, seq_len=c.seq_len,
                          read_block=c.read_block, sm_scale=c.sm_scale, dv=32)
    assert np.array_equal(a[1], b[1])


def _sparse_ragged(seed=60, seq_lens=(200, 75, 130), q_lens=(5, 1, 3), K=6, RB=16, ps=32, H=3,
                   pad_tokens=0, pad_frac=0.3):
    return wl.make_sparse_ragged(seq_lens=list(seq_lens), q_lens=list(q_lens), H=H, K=K,
                                 page_size=ps, read_block=RB, dtype=torch.float32, seed=seed,
                                 kv_lora_rank=32, rope_dim=8, pad_cols=48, pad_tokens=pad_tokens,
                                 pad_frac=pad_frac)


def _sparse_one_request(c, q, d, kv, r, rows):
    """The single-sequence call for request r on the given packed rows: its own
    page-table slice, its own kv length as the causal bound."""
    ps = c.page_size
    base = int(c.cu_kv_lens[r]) // ps
    npg = (int(c.cu_kv_lens[r + 1]) - int(c.cu_kv_lens[r])) // ps
    table = c.page_indices[base:base + npg].copy()
    return oracle.sparse_mla(q[rows], d, kv, table, c.indices[rows], c.positions[rows],
                             seq_len=int(c.seq_lens[r]), read_block=c.read_block,
                             sm_scale=c.sm_scale, dv=32)


def test_sparse_ragged_equals_each_request_alone():
    """Packed-ragged mode [Sparse page: prefill_write_and_attend_ragged,
    sparse_mla_attention ragged branch]: every token gives what the
    single-sequence call of its own request gives (its pages, its bound),
    bit for bit; one request has a single token (decode, S == 1)."""
    c = _sparse_ragged()
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    got = oracle.sparse_mla(q, d, kv, c.page_indices, c.indices, c.positions, read_block=c.read_block,
                            sm_scale=c.sm_scale, dv=32, cu_q_lens=c.cu_q_lens, seq_lens=c.seq_lens,
                            cu_kv_lens=c.cu_kv_lens)
    for r in range(len(c.seq_lens)):
        rows = np.arange(c.cu_q_lens[r], c.cu_q_lens[r + 1])
        want = _sparse_one_request(c, q, d, kv, r, rows)
        assert np.array_equal(got[rows], want), r


def test_sparse_ragged_bound_is_per_request():
    """The causal bound of a token is its own request's kv length: with query
    positions pushed past every request's length, keys stop at seq_lens[rid]
    (the single-sequence call with that request's length as seq_len)."""
    c = _sparse_ragged(seed=64, seq_lens=(200, 75, 130), q_lens=(3, 2, 2), K=8, pad_frac=0.0)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    pos = c.positions.copy()
    for r in range(len(c.seq_lens)):
        pos[c.cu_q_lens[r]:c.cu_q_lens[r + 1]] = int(c.seq_lens[r]) + 40
    idx = np.full_like(c.indices, -1)
    for t in range(q.shape[0]):
        r = int(np.searchsorted(c.cu_q_lens[1:], t, side="right"))
        n = -(-int(c.seq_lens[r]) // 16)
        idx[t, :min(8, n)] = np.arange(max(0, n - 8), n)
    got = oracle.sparse_mla(q, d, kv, c.page_indices, idx, pos, read_block=16, sm_scale=c.sm_scale,
                            dv=32, cu_q_lens=c.cu_q_lens, seq_lens=c.seq_lens, cu_kv_lens=c.cu_kv_lens)
    for r in range(len(c.seq_lens)):
        rows = np.arange(c.cu_q_lens[r], c.cu_q_lens[r + 1])
        ps = c.page_size
        base = int(c.cu_kv_lens[r]) // ps
        npg = (int(c.cu_kv_lens[r + 1]) - int(c.cu_kv_lens[r])) // ps
        want = oracle.sparse_mla(q[rows], d, kv, c.page_indices[base:base + npg].copy(), idx[rows],
                                 pos[rows], seq_len=int(c.seq_lens[r]), read_block=16,
                                 sm_scale=c.sm_scale, dv=32)
        assert np.array_equal(got[rows], want), r
        # the last unit is cut at the request's length, so the bound is engaged
        assert int(c.seq_lens[r]) % 16 != 0


def test_sparse_ragged_all_causal_units_equals_dense_causal_mla():
    """Selecting every causal unit of its request turns each token's sparse
    attention into dense causal MLA over that request's first position + 1
    tokens, read through the request's own window of the packed table."""
    c = _sparse_ragged(seed=61, seq_lens=(96, 160, 40), q_lens=(2, 3, 1), K=16, RB=16, pad_frac=0.0)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    T = q.shape[0]
    idx = np.full((T, 16), -1, np.int32)
    for t in range(T):
        n = int(c.positions[t]) // 16 + 1
        idx[t, :n] = np.arange(n)
    got = oracle.sparse_mla(q, d, kv, c.page_indices, idx, c.positions, read_block=16,
                            sm_scale=c.sm_scale, dv=32, cu_q_lens=c.cu_q_lens, seq_lens=c.seq_lens,
                            cu_kv_lens=c.cu_kv_lens)
    ps = c.page_size
    for r in range(len(c.seq_lens)):
        base = int(c.cu_kv_lens[r]) // ps
        npg = (int(c.cu_kv_lens[r + 1]) - int(c.cu_kv_lens[r])) // ps
        table = c.page_indices[base:base + npg].reshape(1, npg).copy()
        for t in range(c.cu_q_lens[r], c.cu_q_lens[r + 1]):
            L = int(c.positions[t]) + 1
            dense = oracle.mla(q[t:t + 1, :, :32].copy(), q[t:t + 1, :, 32:40].copy(), d, kv, None,
                               [L], table, [0, 1], 1, sm_scale=c.sm_scale, fused=True)
            np.testing.assert_allclose(got[t], dense[0], atol=1e-12)


def test_sparse_ragged_padding_tokens_belong_to_the_last_request():
    """Tokens past cu_q_lens[R] map to request R - 1 (the page's right-sided
    search clipped to the last request). The per-request arrays are views of
    longer buffers, so a missing clip would read the sentinel entries."""
    c = _sparse_ragged(seed=62, pad_tokens=3)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    R = len(c.seq_lens)
    sl_buf = np.concatenate([c.seq_lens, [0]]).astype(np.int32)
    got = oracle.sparse_mla(q, d, kv, c.page_indices, c.indices, c.positions, read_block=c.read_block,
                            sm_scale=c.sm_scale, dv=32, cu_q_lens=c.cu_q_lens,
                            seq_lens=sl_buf[:R], cu_kv_lens=c.cu_kv_lens)
    pad_rows = np.arange(c.cu_q_lens[R], q.shape[0])
    assert len(pad_rows) == 3
    want = _sparse_one_request(c, q, d, kv, R - 1, pad_rows)
    assert np.array_equal(got[pad_rows], want)
    assert np.abs(want).sum() > 0


def test_sparse_ragged_single_request_is_the_single_sequence_mode():
    c = _sparse_small(seed=63, pad_frac=0.3)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    S = q.shape[0]
    a = oracle.sparse_mla(q, d, kv, c.page_table, c.indices, c.positions, seq_len=c.seq_len,
                          read_block=c.read_block, sm_scale=c.sm_scale, dv=32)
    b = oracle.sparse_mla(q, d, kv, c.page_table, c.indices, c.positions, read_block=c.read_block,
                          sm_scale=c.sm_scale, dv=32, cu_q_lens=[0, S], seq_lens=[c.seq_len],
                          cu_kv_lens=[0, len(c.page_table) * c.page_size])
    assert np.array_equal(a, b)


# -------------------------------------------------------------- kv update --

def test_kv_update_combined_gqa_by_direct_assignment():
    rng = np.random.default_rng(20)
    Hkv, D, ps = 2, 8, 4
    seqs = [(2, 5), (3, 3), (1, 9)]
    c = wl.make_gqa(seqs, num_q_heads=4, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=20, spare_pages=3)
    pool, d = storage(c.kv_pages)
    T = int(c.cu_q_lens[-1])
    newk = rng.integers(0, 1 << 16, (T, Hkv, D)).astype(np.uint16)
    newv = rng.integers(0, 1 << 16, (T, Hkv, D)).astype(np.uint16)
    got = pool.copy()
    oracle.kv_update(oracle.LAYOUT_COMBINED_GQA, newk, newv, got, None, d, kv_lens=c.kv_lens,
                     page_indices=c.page_indices, cu_q_lens=c.cu_q_lens, num_seqs=3)
    want = pool.copy()
    for i, (ql, kv) in enumerate(seqs):
        for j in range(ql):
            pos = kv - ql + j
            pg = c.page_indices[i, pos // ps]
            for h in range(Hkv):
                want[pg, pos % ps, 2 * h] = newk[c.cu_q_lens[i] + j, h]
                want[pg, pos % ps, 2 * h + 1] = newv[c.cu_q_lens[i] + j, h]
    assert np.array_equal(got, want)
    assert (got != pool).any()


def test_kv_update_mla_split_and_fused_slot_list():
    rng = np.random.default_rng(21)
    P, ps, Dl, Dr = 5, 4, 16, 4
    ckv = rng.integers(0, 1 << 16, (P, ps, 16)).astype(np.uint16)
    ckp = rng.integers(0, 1 << 16, (P, ps, 8)).astype(np.uint16)
    T = 6
    kvc = rng.integers(0, 1 << 16, (T, Dl)).astype(np.uint16)
    kpe = rng.integers(0, 1 << 16, (T, Dr)).astype(np.uint16)
    kv_lens = np.array([6, 2], np.int32)
    cu = np.array([0, 4, 6], np.int32)
    table = np.array([[3, 1], [0, 4]], np.int32)
    a, b = ckv.copy(), ckp.copy()
    oracle.kv_update(oracle.LAYOUT_MLA_SPLIT, kvc, kpe, a, b, oracle.BF16, kv_lens=kv_lens,
                     page_indices=table, cu_q_lens=cu, num_seqs=2)
    wa, wb = ckv.copy(), ckp.copy()
    dest = {0: (3, 2), 1: (3, 3), 2: (1, 0), 3: (1, 1), 4: (0, 0), 5: (0, 1)}
    for t, (pg, r) in dest.items():
        wa[pg, r] = kvc[t]
        wb[pg, r, :Dr] = kpe[t]
        wb[pg, r, Dr:] = 0
    assert np.array_equal(a, wa) and np.array_equal(b, wb)
    # Fused pool in slot-list mode: row [kv_c || k_pe || 0], -1 slots dropped.
    fused = rng.integers(0, 1 << 16, (P, ps, 24)).astype(np.uint16)
    loc = np.array([7, -1, 0, 19, -1, 12], np.int32)
    f = fused.copy()
    oracle.kv_update(oracle.LAYOUT_MLA_FUSED, kvc, kpe, f, None, oracle.BF16, slot_loc=loc)
    wf = fused.copy().reshape(P * ps, 24)
    for t, s in enumerate(loc):
        if s < 0:
            continue
        wf[s, :Dl] = kvc[t]
        wf[s, Dl:Dl + Dr] = kpe[t]
        wf[s, Dl + Dr:] = 0
    assert np.array_equal(f.reshape(P * ps, 24), wf)


def test_sparse_seq_len_bound_cuts_keys():
    """Keys at or past seq_len are excluded even when causal [Sparse page:
    validity bias kp < kv_len]."""
    c = _sparse_small(seed=16, K=8, RB=16, ps=32, T=256, S=4)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    pos = np.array([200, 210, 220, 255], np.int32)
    idx = np.tile(np.arange(8, 16, dtype=np.int32), (4, 1))   # tokens 128..255
    seq_len = 150
    got = oracle.sparse_mla(q, d, kv, c.page_table, idx, pos, seq_len=seq_len, read_block=16,
                            sm_scale=c.sm_scale, dv=32)
    flat = kv.reshape(-1, kv.shape[2]).astype(np.float64)
    rows = flat[_logical_rows(c, list(range(128, 150)))]
    for s in range(4):
        K = torch.from_numpy(rows[:, :40])[None].expand(4, -1, -1)
        V = torch.from_numpy(rows[:, :32])[None].expand(4, -1, -1)
        Q = torch.from_numpy(q[s].astype(np.float64))[:, None, :]
        want = _sdpa(Q, K, V, torch.ones((1, 22), dtype=torch.bool), c.sm_scale)[:, 0, :].numpy()
        np.testing.assert_allclose(got[s], want, atol=1e-10)


# ---------------------------------------------- MLA window and soft cap --

GOLDEN_MLA = os.path.join(os.path.dirname(__file__), "golden", "hand_derived_mla.json")


def _mla_expr(tok):
    if isinstance(tok, (int, float)):
        return float(tok)
    if tok == "(2ln2+3ln3)/6":
        return (2 * math.log(2.0) + 3 * math.log(3.0)) / 6
    return _coord(tok)


def _mla_golden_cases():
    with open(GOLDEN_MLA) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _mla_golden_cases(), ids=lambda c: c["name"])
def test_mla_hand_derived(case):
    """One sequence, latent width 2 (the value), rope width 1, page size 2,
    pages in reverse physical order, unused rows NaN [MLA v1 page:
    ref_mla_ragged_paged_attention]."""
    kv_len, q_len = case["kv_len"], case["q_len"]
    ps, Dl, Dr = 2, 2, 1
    n_pages = -(-kv_len // ps)
    P = n_pages + 1
    ckv = np.full((P, ps, Dl), np.nan, dtype=np.float32)
    ckp = np.full((P, ps, Dr), np.nan, dtype=np.float32)
    table = np.array([[P - 1 - lp for lp in range(n_pages)]], dtype=np.int32)
    for t in range(kv_len):
        page, row = table[0, t // ps], t % ps
        score = _coord(case["key_score"][t])
        vals = case["values"][t]
        if case["score_from"] == "rope":
            ckv[page, row] = vals
            ckp[page, row, 0] = score
        else:
            ckv[page, row] = [score, vals[1]]
            ckp[page, row, 0] = 0.0
    ql = np.zeros((q_len, 1, Dl), dtype=np.float32)
    qp = np.zeros((q_len, 1, Dr), dtype=np.float32)
    if case["score_from"] == "rope":
        qp[:, 0, 0] = 1.0
    else:
        ql[:, 0, 0] = 1.0
    cap = case["soft_cap"]
    cap = 3 * math.log(3.0) if cap == "3ln3" else float(cap)
    out = oracle.mla(ql, qp, oracle.F32, ckv, ckp, [kv_len], table, [0, q_len], 1, sm_scale=1.0,
                     sliding_window=case["window"] or None, soft_cap=cap or None)
    want = np.array([[_mla_expr(x) for x in row] for row in case["expected"]])
    np.testing.assert_allclose(out[:, 0, :], want, rtol=0, atol=2e-6)


def _mla_dense(c, ql, qp, ckv, ckp, window, scale_q=1.0):
    """fp64 SDPA over each sequence's unpaged latent with an explicit
    causal + window mask."""
    H, Dl, Dr = ql.shape[1], ql.shape[2], qp.shape[2]
    ps = ckv.shape[1]
    want = np.zeros(ql.shape, np.float64)
    for i in range(c.num_seqs):
        L, ql_i = int(c.kv_lens[i]), int(c.cu_q_lens[i + 1] - c.cu_q_lens[i])
        rows = [c.page_indices[i, t // ps] * ps + t % ps for t in range(L)]
        kvc = ckv.reshape(-1, ckv.shape[2])[rows, :Dl].astype(np.float64)
        kpe = ckp.reshape(-1, ckp.shape[2])[rows, :Dr].astype(np.float64)
        K = torch.from_numpy(np.concatenate([kvc, kpe], 1))[None].expand(H, -1, -1)
        V = torch.from_numpy(kvc)[None].expand(H, -1, -1)
        sl = slice(c.cu_q_lens[i], c.cu_q_lens[i + 1])
        Q = torch.from_numpy(np.concatenate([ql[sl], qp[sl]], 2).astype(np.float64) * scale_q)
        qpos = L - ql_i + np.arange(ql_i)
        kpos = np.arange(L)
        mask = kpos[None, :] <= qpos[:, None]
        if window:
            mask &= kpos[None, :] > qpos[:, None] - window
        want[sl] = _sdpa(Q.transpose(0, 1), K, V, torch.from_numpy(mask),
                         c.sm_scale).transpose(0, 1).numpy()
    return want


@pytest.mark.parametrize("window", [1, 5, 33])
def test_mla_window_matches_dense_sdpa(window):
    c = wl.make_mla([(1, 70), (3, 3), (5, 129), (2, 40)], num_heads=4, lkv_dim=32, r_dim=8,
                    page_size=16, dtype=torch.float32, seed=30 + window)
    ql, d = storage(c.ql_nope)
    qp, _ = storage(c.q_pe)
    ckv, _ = storage(c.cache_kv_c)
    ckp, _ = storage(c.cache_k_pe)
    got = oracle.mla(ql, qp, d, ckv, ckp, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs,
                     sm_scale=c.sm_scale, sliding_window=window)
    np.testing.assert_allclose(got, _mla_dense(c, ql, qp, ckv, ckp, window), atol=1e-10)


def test_mla_huge_cap_is_no_cap_and_engaged_cap_moves_output():
    c = wl.make_mla([(1, 70), (4, 90)], num_heads=4, lkv_dim=32, r_dim=8, page_size=16,
                    dtype=torch.float32, seed=40)
    ql, d = storage(c.ql_nope)
    qp, _ = storage(c.q_pe)
    ckv, _ = storage(c.cache_kv_c)
    ckp, _ = storage(c.cache_k_pe)
    args = (d, ckv, ckp, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs)
    base = oracle.mla(ql, qp, *args, sm_scale=c.sm_scale)
    np.testing.assert_allclose(oracle.mla(ql, qp, *args, sm_scale=c.sm_scale, soft_cap=1e9), base,
                               atol=1e-12)
    # Queries x16 push |score| well past a cap of 2: the capped output differs.
    ql16, qp16 = ql * 16, qp * 16
    capped = oracle.mla(ql16, qp16, *args, sm_scale=c.sm_scale, soft_cap=2.0)
    uncapped = oracle.mla(ql16, qp16, *args, sm_scale=c.sm_scale)
    assert np.abs(capped - uncapped).max() > 0.1


# ------------------------------------------------------ row-subset paths --

def test_rpa_token_subset_equals_full_rows():
    c = wl.make_gqa([(3, 20), (1, 7), (6, 40), (1, 1)], num_q_heads=8, num_kv_heads=2,
                    head_dim=16, page_size=4, q_dtype=torch.float32, kv_dtype=torch.float32,
                    seed=50)
    q, qd = storage(c.q)
    kv, kd = storage(c.kv_pages)
    kw = dict(sm_scale=0.3, sliding_window=5, soft_cap=3.0)
    full = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs, **kw)
    toks = np.array([10, 0, 4, 9, 5], np.int32)
    sub = oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs,
                     tokens=toks, **kw)
    assert np.array_equal(sub[toks], full[toks])
    rest = np.setdiff1d(np.arange(q.shape[0]), toks)
    assert np.isnan(sub[rest]).all()


def test_mla_token_subset_equals_full_rows():
    c = wl.make_mla([(1, 70), (3, 3), (5, 129)], num_heads=4, lkv_dim=32, r_dim=8,
                    page_size=16, dtype=torch.float32, seed=51)
    ql, d = storage(c.ql_nope)
    qp, _ = storage(c.q_pe)
    ckv, _ = storage(c.cache_kv_c)
    ckp, _ = storage(c.cache_k_pe)
    args = (ql, qp, d, ckv, ckp, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs)
    kw = dict(sm_scale=c.sm_scale, sliding_window=7, soft_cap=4.0)
    full = oracle.mla(*args, **kw)
    toks = np.array([8, 1, 0, 3], np.int32)
    sub = oracle.mla(*args, tokens=toks, **kw)
    assert np.array_equal(sub[toks], full[toks])
    rest = np.setdiff1d(np.arange(ql.shape[0]), toks)
    assert np.isnan(sub[rest]).all()


def test_sparse_query_subset_equals_full_rows():
    c = _sparse_small(seed=52, pad_frac=0.3)
    q, d = storage(c.q)
    kv, _ = storage(c.kv_cache)
    kw = dict(seq_len=c.seq_len, read_block=c.read_block, sm_scale=c.sm_scale, dv=32)
    full = oracle.sparse_mla(q, d, kv, c.page_table, c.indices, c.positions, **kw)
    qs = np.array([5, 2, 0], np.int32)
    sub = oracle.sparse_mla(q, d, kv, c.page_table, c.indices, c.positions, queries=qs, **kw)
    assert np.array_equal(sub[qs], full[qs])
    rest = np.setdiff1d(np.arange(q.shape[0]), qs)
    assert np.isnan(sub[rest]).all()
