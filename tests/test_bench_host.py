"""Host-side logic of bench.py (CPU only): the algorithmic work the roofline
divides by, the decode-subset selection, and the one-GPU refusal.

The work counts are pinned by brute force: every (query, key) pair of every
sequence is tested against the causal and window rule written out directly
(a key t is visible to the query at position p iff p - W < t <= p, W = 0
meaning no window), and the K/V bytes are the distinct visible rows."""
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
from ragged_paged_attention_rpa_amd import workloads as wl


def _brute_work(case):
    W = case.sliding_window or 0
    Hq, Hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    eb = case.kv_pages.element_size()
    pairs = rows = dec_bytes = pre_pairs = 0
    for i in range(case.num_seqs):
        ql = int(case.cu_q_lens[i + 1] - case.cu_q_lens[i])
        L = int(case.kv_lens[i])
        seen = set()
        n = 0
        for r in range(ql):
            p = L - ql + r
            for t in range(L):
                if t <= p and (W == 0 or t > p - W):
                    n += 1
                    seen.add(t)
        pairs += n
        rows += len(seen)
        if ql == 1:
            dec_bytes += len(seen) * 2 * Hkv * D * eb
        else:
            pre_pairs += n
    return {"kv_bytes": rows * 2 * Hkv * D * eb, "flops": pairs * Hq * 4 * D,
            "decode_kv_bytes": dec_bytes, "prefill_flops": pre_pairs * Hq * 4 * D}


@pytest.mark.parametrize("window", [None, 5, 40])
def test_gqa_work_matches_brute_force(window):
    seqs = [(1, 1), (1, 37), (3, 3), (9, 50), (1, 64), (12, 30)]
    c = wl.make_gqa(seqs, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=9,
                    sliding_window=window, name="work")
    got = bench.gqa_work(c)
    want = _brute_work(c)
    for k, v in want.items():
        assert got[k] == v, (k, got[k], v)
    assert got["q_tokens"] == sum(q for q, _ in seqs)


def test_leading_decodes():
    # 32/8 heads (G = 4): q_len * G <= 16 is decode-class, so q_len <= 4.
    c = wl.make_gqa([(1, 10), (4, 20), (1, 5), (5, 30), (1, 9)], num_q_heads=32, num_kv_heads=8,
                    head_dim=128, page_size=16, q_dtype=torch.bfloat16,
                    kv_dtype=torch.bfloat16, seed=3, name="lead")
    assert bench._leading_decodes(c) == 3
    c2 = wl.make_gqa([(1, 10), (2, 20)], num_q_heads=32, num_kv_heads=8, head_dim=128,
                     page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=3,
                     name="all-decode")
    assert bench._leading_decodes(c2) == 2


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_mla_work_matches_brute_force():
    seqs = [(1, 40), (1, 1), (3, 70)]
    c = wl.make_mla(seqs, num_heads=16, page_size=16, seed=4)
    got = bench.mla_work(c, 16)
    pairs = rows = 0
    for i, (ql, L) in enumerate(seqs):
        seen = set()
        for r in range(ql):
            p = L - ql + r
            for t in range(L):
                if t <= p:
                    pairs += 1
                    seen.add(t)
        rows += len(seen)
    assert got["kv_bytes"] == rows * (512 + 64) * 2
    assert got["flops"] == pairs * 16 * (2 * 576 + 2 * 512)


def test_sparse_work_matches_brute_force():
    c = wl.make_sparse(T=640, S=6, H=16, K=4, page_size=64, read_block=64, seed=5)
    got = bench.sparse_work(c)
    keys = 0
    for s in range(c.q.shape[0]):
        for u in c.indices[s]:
            if u < 0:
                continue
            for r in range(c.read_block):
                kp = int(u) * c.read_block + r
                if kp <= int(c.positions[s]) and kp < c.seq_len:
                    keys += 1
    assert keys > 0
    assert got["gathered_bytes"] == keys * 576 * 2
    assert got["flops"] == keys * 16 * 2 * (576 + 512)
