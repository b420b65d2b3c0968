"""GPU parity of mla_rpa_forward (scatter + attention) and sparse_mla_forward
against the CPU oracle. bf16 tolerances: max-abs 2e-2, mean-abs 2e-3."""
import math

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_rpa_amd as rpa
from ragged_paged_attention_rpa_amd import workloads as wl
from tests.helpers import as_f64, assert_close, storage

pytestmark = pytest.mark.gpu
TOL = (2e-2, 2e-3)


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _meta(c):
    d = "cuda"
    return (torch.from_numpy(c.kv_lens).to(d), torch.from_numpy(c.page_indices).to(d),
            torch.from_numpy(c.cu_q_lens).to(d),
            torch.tensor([c.num_seqs], dtype=torch.int32, device=d))


def _mla_gpu(c, update=True):
    kl, pi, cu, ns = _meta(c)
    out = rpa.mla_rpa_forward(c.ql_nope, c.q_pe, c.new_kv_c if update else None,
                              c.new_k_pe if update else None, c.cache_kv_c, c.cache_k_pe, kl, pi,
                              cu, ns, sm_scale=c.sm_scale, sliding_window=c.sliding_window,
                              soft_cap=c.soft_cap)
    torch.cuda.synchronize()
    return out


def _mla_oracle(c, ckv, ckp, tokens=None):
    return oracle.mla(storage(c.ql_nope)[0], storage(c.q_pe)[0], oracle.BF16, ckv, ckp, c.kv_lens,
                      c.page_indices, c.cu_q_lens, c.num_seqs, sm_scale=c.sm_scale,
                      sliding_window=c.sliding_window, soft_cap=c.soft_cap, tokens=tokens)


def _host_caches_after_update(c):
    ckv = storage(c.cache_kv_c)[0].copy()
    ckp = storage(c.cache_k_pe)[0].copy()
    oracle.kv_update(oracle.LAYOUT_MLA_SPLIT, storage(c.new_kv_c)[0], storage(c.new_k_pe)[0], ckv,
                     ckp, oracle.BF16, kv_lens=c.kv_lens, page_indices=c.page_indices,
                     cu_q_lens=c.cu_q_lens, num_seqs=c.num_seqs)
    return ckv, ckp


MLA_CASES = [
    # (seqs, heads, page_size, window, cap, name)
    ([(1, 100), (1, 2000), (1, 1), (1, 64), (1, 65)], 128, 64, None, None, "decode-h128"),
    ([(3, 300), (1, 777), (5, 64), (2, 2)], 16, 64, None, None, "ragged-h16"),
    ([(1, 5000), (4, 1300), (1, 129)], 128, 16, 700, None, "page16-window"),
    ([(2, 400), (1, 3000)], 40, 32, None, 30.0, "h40-cap"),
    ([(1, 900), (2, 150)], 130, 64, None, None, "h130-two-groups"),
    # page 16 and 20000 keys: the query tiles span 1250 pages, past the 1024
    # page ids a workgroup caches, so the page window refills mid-tile
    ([(2, 20000), (1, 300)], 128, 16, None, None, "page16-refill"),
]


@pytest.mark.parametrize("idx", range(len(MLA_CASES)), ids=[c[-1] for c in MLA_CASES])
def test_mla_update_and_attention(idx):
    seqs, H, ps, window, cap, name = MLA_CASES[idx]
    _say(f"mla {name}")
    c = wl.make_mla(seqs, num_heads=H, page_size=ps, seed=200 + idx, device="cuda",
                    sliding_window=window, soft_cap=cap, name=name)
    ckv, ckp = _host_caches_after_update(c)
    got = _mla_gpu(c)
    # The scatter must land bit-exactly in both caches.
    assert np.array_equal(storage(c.cache_kv_c)[0], ckv)
    assert np.array_equal(storage(c.cache_k_pe)[0], ckp)
    want = _mla_oracle(c, ckv, ckp)
    n = int(c.cu_q_lens[c.num_seqs])
    assert_close(as_f64(got)[:n], want[:n], *TOL, what=name)


def test_mla_attention_only_and_determinism():
    _say("mla attention only")
    c = wl.make_mla([(1, 3000), (1, 17), (2, 600)], num_heads=128, page_size=64, seed=210,
                    device="cuda")
    a = _mla_gpu(c, update=False).clone()
    b = _mla_gpu(c, update=False)
    assert torch.equal(a, b)
    want = _mla_oracle(c, storage(c.cache_kv_c)[0], storage(c.cache_k_pe)[0])
    assert_close(as_f64(a)[:4], want[:4], *TOL)


def test_mla_decode_full_size_sampled():
    _say("mla_decode full size (64 seqs, kv 4096..32768, 128 heads), sampled tokens")
    c = wl.mla_decode(device="cuda")
    ckv, ckp = _host_caches_after_update(c)
    got = _mla_gpu(c)
    tokens = np.arange(0, 64, 6)
    want = _mla_oracle(c, ckv, ckp, tokens=tokens)
    assert_close(as_f64(got)[tokens], want[tokens], *TOL, what="mla_decode")


def test_mla_explicit_min_share():
    """mla_rpa_forward with the smallest share fixed by the caller (64 keys:
    every workgroup takes a share on a small batch; 4096: few workgroups, few
    cut tokens) instead of the tile table; the caches and outputs match."""
    _say("mla explicit min share")
    for sk in (64, 4096):
        c = wl.make_mla([(1, 1500), (3, 900), (1, 64), (2, 2)], num_heads=128, page_size=16,
                        seed=470, device="cuda", name=f"share-{sk}")
        ckv, ckp = _host_caches_after_update(c)
        kl, pi, cu, ns = _meta(c)
        got = rpa.mla_rpa_forward(c.ql_nope, c.q_pe, c.new_kv_c, c.new_k_pe, c.cache_kv_c,
                                  c.cache_k_pe, kl, pi, cu, ns, sm_scale=c.sm_scale, split_keys=sk)
        torch.cuda.synchronize()
        assert np.array_equal(storage(c.cache_kv_c)[0], ckv)
        assert np.array_equal(storage(c.cache_k_pe)[0], ckp)
        want = _mla_oracle(c, ckv, ckp)
        assert_close(as_f64(got), want, *TOL, what=f"share-{sk}")


def test_mla_scales_as_the_page_kernel():
    """q_scale and k_scale on the scores, v_scale on the value sum (the MLA
    page's kernel), with the fused update."""
    _say("mla q/k/v scales")
    c = wl.make_mla([(1, 3000), (2, 500), (1, 64)], num_heads=128, page_size=64, seed=475,
                    device="cuda", name="mla-scales")
    ckv, ckp = _host_caches_after_update(c)
    kl, pi, cu, ns = _meta(c)
    got = rpa.mla_rpa_forward(c.ql_nope, c.q_pe, c.new_kv_c, c.new_k_pe, c.cache_kv_c,
                              c.cache_k_pe, kl, pi, cu, ns, sm_scale=c.sm_scale, q_scale=0.5,
                              k_scale=3.0, v_scale=0.25)
    torch.cuda.synchronize()
    want = oracle.mla(storage(c.ql_nope)[0], storage(c.q_pe)[0], oracle.BF16, ckv, ckp, c.kv_lens,
                      c.page_indices, c.cu_q_lens, c.num_seqs, sm_scale=c.sm_scale, q_scale=0.5,
                      k_scale=3.0, v_scale=0.25)
    assert_close(as_f64(got), want, *TOL, what="mla-scales")


# ------------------------------------------------------------------ sparse --

def _sparse_gpu(c, indices=None):
    d = "cuda"
    idx = torch.from_numpy(c.indices if indices is None else indices).to(d)
    out = rpa.sparse_mla_forward(c.q, c.kv_cache, torch.from_numpy(c.page_table).to(d), idx,
                                 torch.from_numpy(c.positions).to(d), seq_len=c.seq_len,
                                 read_block=c.read_block, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    return out


def _sparse_oracle(c, indices=None, queries=None):
    return oracle.sparse_mla(storage(c.q)[0], oracle.BF16, storage(c.kv_cache)[0], c.page_table,
                             c.indices if indices is None else indices, c.positions,
                             seq_len=c.seq_len, read_block=c.read_block, sm_scale=c.sm_scale,
                             queries=queries)


SPARSE_CASES = [
    # (T, S, H, K, ps, RB, seq_len_cut, name)
    (2048, 48, 16, 8, 64, 64, 0, "page-units"),
    (2048, 40, 20, 12, 64, 32, 0, "h20-rb32"),
    (1500, 30, 8, 40, 128, 64, 300, "seq-len-cut"),
]


@pytest.mark.parametrize("idx", range(len(SPARSE_CASES)), ids=[c[-1] for c in SPARSE_CASES])
def test_sparse_small(idx):
    T, S, H, K, ps, RB, cut, name = SPARSE_CASES[idx]
    _say(f"sparse {name}")
    rng = np.random.default_rng(300 + idx)
    pos = np.sort(rng.integers(0, T, S)).astype(np.int32)
    c = wl.make_sparse(T=T, S=S, H=H, K=K, page_size=ps, read_block=RB, seed=300 + idx,
                       device="cuda", positions=pos, pad_frac=0.3, name=name)
    if cut:
        c.seq_len = T - cut
    idx_arr = c.indices.copy()
    idx_arr[0, -1] = idx_arr[0, 0]     # a repeated unit counts twice
    idx_arr[1, :] = -1                 # empty selection -> zeros
    got = as_f64(_sparse_gpu(c, idx_arr))
    want = _sparse_oracle(c, idx_arr)
    assert np.all(got[1] == 0.0)
    assert_close(got, want, *TOL, what=name)


def test_sparse_nan_outside_selection_is_never_read():
    _say("sparse nan hygiene")
    c = wl.make_sparse(T=1024, S=16, H=16, K=4, seed=320, device="cuda")
    clean = _sparse_gpu(c).clone()
    # Poison every page row that no selected, causal key of any query reads.
    used = np.zeros(c.kv_cache.shape[0] * 64, dtype=bool)
    for s in range(16):
        for u in c.indices[s]:
            if u < 0:
                continue
            for r in range(64):
                kp = u * 64 + r
                if kp <= c.positions[s] and kp < c.seq_len:
                    used[c.page_table[kp // 64] * 64 + kp % 64] = True
    flat = c.kv_cache.view(-1, c.kv_cache.shape[2])
    flat[torch.from_numpy(~used).cuda()] = float("nan")
    dirty = _sparse_gpu(c)
    assert torch.isfinite(dirty).all()
    assert torch.equal(dirty, clean)


def test_sparse_full_size_sampled():
    _say("sparse_mla full size (4096 queries x 32 units x 64 tokens), sampled queries")
    c = wl.sparse_mla(device="cuda")
    got = as_f64(_sparse_gpu(c))
    qs = np.arange(0, 4096, 97)
    want = _sparse_oracle(c, queries=qs)
    assert_close(got[qs], want[qs], *TOL, what="sparse_mla")


# ----------------------------------------------------------- sparse ragged --

def _sparse_ragged_gpu(c, indices=None, positions=None):
    d = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    out = rpa.sparse_mla_forward_ragged(
        c.q, c.kv_cache, t(c.page_indices), t(c.indices if indices is None else indices),
        t(c.positions if positions is None else positions), t(c.cu_q_lens), t(c.seq_lens),
        t(c.cu_kv_lens), read_block=c.read_block, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    return out


def _sparse_ragged_oracle(c, indices=None, positions=None, queries=None):
    return oracle.sparse_mla(storage(c.q)[0], oracle.BF16, storage(c.kv_cache)[0], c.page_indices,
                             c.indices if indices is None else indices,
                             c.positions if positions is None else positions,
                             read_block=c.read_block, sm_scale=c.sm_scale, queries=queries,
                             cu_q_lens=c.cu_q_lens, seq_lens=c.seq_lens, cu_kv_lens=c.cu_kv_lens)


SPARSE_RAGGED_CASES = [
    # (seq_lens, q_lens, H, K, ps, RB, pad_tokens, name)
    ((3000, 700, 1900, 64), (24, 1, 9, 1), 16, 12, 64, 64, 2, "mixed-extend-decode"),
    ((2500, 4000, 130), (1, 1, 1), 20, 20, 128, 32, 0, "decodes-rb32-ps128"),
    ((5000,), (1,), 16, 32, 64, 64, 0, "single-decode"),
]


@pytest.mark.parametrize("idx", range(len(SPARSE_RAGGED_CASES)),
                         ids=[c[-1] for c in SPARSE_RAGGED_CASES])
def test_sparse_ragged_small(idx):
    seq_lens, q_lens, H, K, ps, RB, pad_tokens, name = SPARSE_RAGGED_CASES[idx]
    _say(f"sparse ragged {name}")
    c = wl.make_sparse_ragged(seq_lens=list(seq_lens), q_lens=list(q_lens), H=H, K=K, page_size=ps,
                              read_block=RB, seed=340 + idx, device="cuda", pad_tokens=pad_tokens,
                              pad_frac=0.3, name=name)
    idx_arr = c.indices.copy()
    if idx_arr.shape[0] > 2:
        idx_arr[0, -1] = idx_arr[0, 0]     # a repeated unit counts twice
        idx_arr[1, :] = -1                 # empty selection -> zeros
    got = as_f64(_sparse_ragged_gpu(c, idx_arr))
    want = _sparse_ragged_oracle(c, idx_arr)
    if idx_arr.shape[0] > 2:
        assert np.all(got[1] == 0.0)
    assert_close(got, want, *TOL, what=name)


def test_sparse_ragged_bound_is_per_request():
    """Query positions past every request's kv length: keys stop at that
    request's seq_lens entry (the last selected unit is cut there)."""
    _say("sparse ragged per-request bound")
    c = wl.make_sparse_ragged(seq_lens=[1000, 333, 2100], q_lens=[3, 2, 4], H=16, K=8, page_size=64,
                              read_block=64, seed=350, device="cuda", name="bound")
    pos = c.positions.copy()
    idx = np.full_like(c.indices, -1)
    for r in range(3):
        rows = slice(c.cu_q_lens[r], c.cu_q_lens[r + 1])
        pos[rows] = int(c.seq_lens[r]) + 100
        n = -(-int(c.seq_lens[r]) // 64)
        idx[rows, :min(8, n)] = np.arange(max(0, n - 8), n)
    got = as_f64(_sparse_ragged_gpu(c, idx, pos))
    want = _sparse_ragged_oracle(c, idx, pos)
    assert_close(got, want, *TOL, what="bound")


def test_sparse_ragged_matches_single_sequence_calls_bitwise():
    """Each request's rows of a packed call equal the single-sequence call on
    that request's page-table window and length, bit for bit."""
    _say("sparse ragged vs single-sequence calls")
    c = wl.make_sparse_ragged(seq_lens=[1500, 64, 2200], q_lens=[7, 1, 5], H=16, K=10, page_size=64,
                              read_block=64, seed=351, device="cuda", pad_frac=0.2, name="vs-single")
    got = _sparse_ragged_gpu(c)
    ps = c.page_size
    for r in range(3):
        rows = slice(int(c.cu_q_lens[r]), int(c.cu_q_lens[r + 1]))
        base = int(c.cu_kv_lens[r]) // ps
        npg = (int(c.cu_kv_lens[r + 1]) - int(c.cu_kv_lens[r])) // ps
        one = rpa.sparse_mla_forward(
            c.q[rows].contiguous(), c.kv_cache, torch.from_numpy(c.page_indices[base:base + npg].copy()).cuda(),
            torch.from_numpy(c.indices[rows].copy()).cuda(), torch.from_numpy(c.positions[rows].copy()).cuda(),
            seq_len=int(c.seq_lens[r]), read_block=c.read_block, sm_scale=c.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(got[rows], one), r


def test_sparse_ragged_large_sampled():
    """Four packed requests (64k, 32k, 16k and 8k keys; 1024, 512 and 256
    extend tokens and one decode), 16 heads, 32 units of 64 tokens; sampled
    tokens against the oracle, the decode token included."""
    _say("sparse ragged large (4 requests, 1793 tokens), sampled tokens")
    c = wl.make_sparse_ragged(seq_lens=[65536, 32768, 16384, 8192], q_lens=[1024, 512, 256, 1],
                              H=16, K=32, page_size=64, read_block=64, seed=352, device="cuda",
                              name="large")
    got = as_f64(_sparse_ragged_gpu(c))
    qs = np.unique(np.concatenate([np.arange(0, c.q.shape[0], 37), [c.q.shape[0] - 1],
                                   c.cu_q_lens[1:-1], c.cu_q_lens[1:-1] - 1]))
    want = _sparse_ragged_oracle(c, queries=qs)
    assert_close(got[qs], want[qs], *TOL, what="sparse ragged large")


def test_mla_page_window_refill_page1():
    """Decode pieces spanning more than the 1024 page ids a workgroup caches in
    LDS: at page size 1, 16 sequences of 20000 keys give shares of ~1250 keys,
    so the page window refills inside a piece; the step's new rows go through
    the fused scatter at the same time."""
    _say("mla page-window refill (page size 1)")
    c = wl.make_mla([(1, 20000 - 7 * i) for i in range(16)], num_heads=32, page_size=1,
                    seed=230, device="cuda", name="page1-refill")
    ckv, ckp = _host_caches_after_update(c)
    got = _mla_gpu(c)
    assert np.array_equal(storage(c.cache_kv_c)[0], ckv)
    assert np.array_equal(storage(c.cache_k_pe)[0], ckp)
    tokens = np.array([0, 5, 15])
    want = _mla_oracle(c, ckv, ckp, tokens=tokens)
    assert_close(as_f64(got)[tokens], want[tokens], *TOL, what="page1-refill")
