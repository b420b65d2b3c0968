"""GPU parity of rpa_forward and kv_cache_update against the CPU oracle.

Each case prints its name before the GPU call so a failure names its case.
Tolerances (max-abs / mean-abs over the compared outputs): fp32 1e-4 / -,
bf16 2e-2 / 2e-3, fp8 KV 5e-2 / 5e-3; kv_cache_update is bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_rpa_amd as rpa
from ragged_paged_attention_rpa_amd import workloads as wl
from tests.helpers import as_f64, assert_close, storage

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, None), "bf16": (2e-2, 2e-3), "fp8": (5e-2, 5e-3)}


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev_meta(c):
    dev = "cuda"
    return (torch.from_numpy(c.kv_lens).to(dev), torch.from_numpy(c.page_indices).to(dev),
            torch.from_numpy(c.cu_q_lens).to(dev),
            torch.tensor([c.num_seqs], dtype=torch.int32, device=dev))


def _run_gpu(c, **kw):
    kl, pi, cu, ns = _dev_meta(c)
    out = rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, sm_scale=c.sm_scale,
                          sliding_window=c.sliding_window, soft_cap=c.soft_cap,
                          k_scale=c.k_scale, v_scale=c.v_scale, **kw)
    torch.cuda.synchronize()
    return out


def _run_oracle(c, tokens=None, kv_pages=None):
    q, qd = storage(c.q)
    kv, kd = storage(c.kv_pages if kv_pages is None else kv_pages)
    return oracle.rpa(q, qd, kv, kd, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs,
                      sm_scale=c.sm_scale, sliding_window=c.sliding_window, soft_cap=c.soft_cap,
                      k_scale=c.k_scale, v_scale=c.v_scale, tokens=tokens)


def _check(c, got, want, tol, tokens=None):
    rows = np.arange(int(c.cu_q_lens[c.num_seqs])) if tokens is None else np.asarray(tokens)
    return assert_close(as_f64(got)[rows], want[rows], *TOL[tol], what=c.name)


def test_tiny_gqa_fp32():
    _say("tiny_gqa fp32")
    c = wl.tiny_gqa(device="cuda")
    _check(c, _run_gpu(c), _run_oracle(c), "f32")


RAGGED = [
    # (seqs, Hq, Hkv, ps, window, cap, name)
    ([(1, 1), (1, 63), (1, 64), (1, 65), (3, 200), (1, 1000)], 32, 8, 16, None, None, "decode-ish"),
    ([(17, 17), (64, 100), (5, 300), (1, 77), (130, 700)], 32, 8, 16, None, None, "prefill-mix"),
    ([(1, 300), (40, 1200), (2, 129), (70, 70)], 16, 16, 32, 100, None, "mha-window"),
    ([(9, 200), (1, 5000), (33, 513)], 8, 1, 64, None, 30.0, "mqa-cap"),
    ([(4, 4), (2, 1025), (24, 900)], 16, 2, 16, 257, 20.0, "g8-window-cap"),
    # decode sequences long enough that the split count hits its cap and the
    # chunks grow past the target split size
    ([(1, 20000), (2, 17000), (4, 1500), (1, 16385)], 32, 8, 16, None, None, "long-decode"),
    ([(1, 18000), (3, 9000)], 16, 4, 16, 5000, 30.0, "long-window"),
    # prefill kernel at its smallest page size (8: one page per wave's keys)
    ([(70, 300), (1, 33), (300, 1100)], 32, 8, 8, None, None, "page8"),
    # page size 4: prefill-class tiles fall back to the four-wave kernel
    ([(40, 300), (1, 77), (70, 200)], 16, 4, 4, 90, None, "page4-fallback"),
    # large groups: 16 and 32 rows per query token (16 and 8 tokens per tile)
    ([(33, 1000), (1, 500), (100, 100)], 32, 2, 16, None, 50.0, "g16"),
    ([(20, 700), (57, 640), (1, 64)], 32, 1, 32, 200, None, "g32-window"),
    # groups that are not powers of two: 255 of the prefill kernel's 256 rows
    # (G=3) or 252 (G=7) are live, decode tiles hold 15 or 14 rows
    ([(1, 700), (3, 500), (300, 1200), (8, 8)], 16, 8, 16, 400, 30.0, "g2-window-cap"),
    ([(5, 900), (1, 300), (170, 800), (4, 4), (2, 3000)], 24, 8, 16, 300, 25.0, "g3-window-cap"),
    ([(2, 1000), (1, 64), (200, 700), (7, 7), (1, 5000)], 28, 4, 32, None, 40.0, "g7-cap"),
    # page size 128 (256 KB of K and V per page for 8 kv heads)
    ([(1, 3000), (200, 1500), (1, 129), (9, 700)], 32, 8, 128, None, None, "page128"),
]


@pytest.mark.parametrize("room", ["tight", "room"])
@pytest.mark.parametrize("idx", range(len(RAGGED)), ids=[r[-1] for r in RAGGED])
def test_ragged_bf16(idx, room):
    """Each ragged case twice: with the token capacity the batch needs (a bf16
    batch with fewer than 256 tokens beyond one per sequence keeps every tile
    on the tile kernel) and with 300 spare tokens of capacity (prefill-class
    tiles on the prefill kernel)."""
    seqs, Hq, Hkv, ps, window, cap, name = RAGGED[idx]
    _say(f"ragged bf16 {name} ({room})")
    c = wl.make_gqa(seqs, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=100 + idx,
                    device="cuda", sliding_window=window, soft_cap=cap, name=name,
                    extra_tokens=300 if room == "room" else 0)
    _check(c, _run_gpu(c), _run_oracle(c), "bf16")
    extra = int(c.q.shape[0]) - c.num_seqs
    if ps >= 8:
        assert rpa.last_path() == ("gqa_mfma_prefill" if extra >= 256 else "gqa_mfma")


@pytest.mark.parametrize("idx", range(len(RAGGED)), ids=[r[-1] for r in RAGGED])
def test_ragged_fp8(idx):
    """The ragged cases over an fp8 pool with k/v scales: decode-class tiles go
    to the fp8 decode kernel (128-key raw blocks) whenever the prefill kernel
    takes the prefill-class tiles, and to the 64-key tile kernel otherwise
    (page size 4)."""
    seqs, Hq, Hkv, ps, window, cap, name = RAGGED[idx]
    _say(f"ragged fp8 {name}")
    c = wl.make_gqa(seqs, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=torch.float8_e4m3fn, seed=200 + idx,
                    device="cuda", kv_value_scale=2.0, sliding_window=window, soft_cap=cap,
                    k_scale=0.5, v_scale=0.5, name=name + "-fp8")
    _check(c, _run_gpu(c), _run_oracle(c), "fp8")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_decode_page_window_refill(kv):
    """Decode splits longer than the 512 page ids a workgroup caches in LDS:
    at page size 8, sequences of 66k-70k keys hit the 16-split cap, so each
    split spans ~550 pages and the decode kernels refill their page window
    mid-tile (bf16: gqa_tile_kernel; fp8: gqa_decode8_kernel)."""
    _say(f"decode page-window refill {kv}")
    kvd = torch.bfloat16 if kv == "bf16" else torch.float8_e4m3fn
    extra = dict(kv_value_scale=2.0, k_scale=0.5, v_scale=0.5) if kv == "fp8" else {}
    c = wl.make_gqa([(1, 70000), (2, 66001), (1, 9000)], num_q_heads=8, num_kv_heads=2,
                    head_dim=128, page_size=8, q_dtype=torch.bfloat16, kv_dtype=kvd, seed=77,
                    device="cuda", sliding_window=None, soft_cap=None, name=f"refill-{kv}",
                    **extra)
    _check(c, _run_gpu(c), _run_oracle(c), kv)


@pytest.mark.parametrize("idx,kv", [(1, "bf16"), (4, "fp8"), (6, "fp8")])
def test_side_stream_launch(idx, kv):
    """Batches whose token capacity leaves room for a prefill share run the
    decode-class launch on the library's side stream, concurrently with the
    prefill kernel: parity, and three back-to-back calls on one workspace give
    identical outputs (each call's planner waits for the previous call's side
    work)."""
    seqs, Hq, Hkv, ps, window, cap, name = RAGGED[idx]
    _say(f"side stream {name} {kv}")
    kvd = torch.bfloat16 if kv == "bf16" else torch.float8_e4m3fn
    extra = dict(kv_value_scale=2.0, k_scale=0.5, v_scale=0.5) if kv == "fp8" else {}
    c = wl.make_gqa(seqs, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=kvd, seed=300 + idx, device="cuda",
                    sliding_window=window, soft_cap=cap, extra_tokens=4096,
                    name=f"{name}-side-{kv}", **extra)
    kl, pi, cu, ns = _dev_meta(c)
    need = rpa.rpa_workspace_size(kl, pi, c.q.shape[0], Hq, Hkv, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        out = torch.zeros_like(c.q)
        rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, sm_scale=c.sm_scale,
                        sliding_window=c.sliding_window, soft_cap=c.soft_cap,
                        k_scale=c.k_scale, v_scale=c.v_scale, out=out, workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    T = int(c.cu_q_lens[c.num_seqs])
    for o in outs[1:]:
        assert torch.equal(o[:T], outs[0][:T])
    _check(c, outs[0], _run_oracle(c), kv)


def test_graph_capture_with_side_stream():
    """rpa_forward captured into a HIP graph (through torch) on a batch that
    takes the side-stream path: the fork and join events pull the side stream
    into the capture. Replays, with eager work between them, match the eager
    call bit for bit (the planner resets its counters with a kernel, so no
    memset node is recorded)."""
    _say("graph capture, side stream")
    seqs, Hq, Hkv, ps, window, cap, name = RAGGED[4]
    c = wl.make_gqa(seqs, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=torch.float8_e4m3fn, seed=400,
                    device="cuda", kv_value_scale=2.0, sliding_window=window, soft_cap=cap,
                    k_scale=0.5, v_scale=0.5, extra_tokens=4096, name="graph-side")
    kl, pi, cu, ns = _dev_meta(c)
    need = rpa.rpa_workspace_size(kl, pi, c.q.shape[0], Hq, Hkv, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(c.q)

    def call():
        rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, sm_scale=c.sm_scale,
                        sliding_window=c.sliding_window, soft_cap=c.soft_cap,
                        k_scale=c.k_scale, v_scale=c.v_scale, out=out, workspace=ws)
    call()  # eager first: creates the library's side stream outside the capture
    torch.cuda.synchronize()
    T = int(c.cu_q_lens[c.num_seqs])
    eager = out[:T].clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(3):
        out.zero_()
        ws.fill_(0xFF)  # eager work between replays; the planner must reset what it needs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[:T], eager), f"replay {k} differs from the eager call"
    _check(c, eager, _run_oracle(c), "fp8")


@pytest.mark.parametrize("cap,qscale,ps", [(None, 1.0, 16), (50.0, 1.0, 16), (50.0, 16.0, 16),
                                            (50.0, 3.0, 16), (50.0, 6.0, 16), (None, 1.0, 8)])
def test_ragged_fp8_scales(cap, qscale, ps):
    """fp8 pool with scales; with the cap, queries x1 keep the scores within
    the range of the capped logit's series form, x16 put nearly every wave on
    the exact form, and x3 / x6 straddle the bound within one launch."""
    _say(f"ragged fp8 cap={cap} qscale={qscale} page={ps}")
    seqs = [(1, 700), (1, 33), (150, 900), (2, 2), (64, 64)]
    c = wl.make_gqa(seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=torch.float8_e4m3fn, seed=31, device="cuda",
                    kv_value_scale=2.0, q_value_scale=qscale, sliding_window=300, soft_cap=cap,
                    k_scale=0.5, v_scale=0.5, name="fp8")
    _check(c, _run_gpu(c), _run_oracle(c), "fp8")


def test_nan_pages_and_tails_are_never_read():
    _say("nan hygiene")
    seqs = [(1, 37), (20, 90), (1, 16)]
    c = wl.make_gqa(seqs, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=5, device="cuda",
                    spare_pages=4)
    clean = _run_gpu(c).clone()
    kv = c.kv_pages.clone()
    used = {}
    for i, (ql, L) in enumerate(seqs):
        for lp in range(wl.cdiv(L, 16)):
            used[int(c.page_indices[i, lp])] = (i, lp)
    for pg in range(kv.shape[0]):
        if pg not in used:
            kv[pg] = float("nan")
        else:
            i, lp = used[pg]
            tail = seqs[i][1] - lp * 16
            if tail < 16:
                kv[pg, tail:] = float("nan")
    c.kv_pages = kv
    dirty = _run_gpu(c)
    n = int(c.cu_q_lens[c.num_seqs])
    assert torch.isfinite(dirty[:n].float()).all()
    assert torch.equal(dirty[:n], clean[:n])


def test_deterministic_and_page_permutation_invariant():
    _say("determinism + permutation")
    seqs = [(1, 500), (30, 400), (1, 2000)]
    c = wl.make_gqa(seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=6, device="cuda")
    a = _run_gpu(c).clone()
    b = _run_gpu(c).clone()
    n = int(c.cu_q_lens[c.num_seqs])
    assert torch.equal(a[:n], b[:n])
    perm = torch.randperm(c.kv_pages.shape[0], generator=torch.Generator().manual_seed(1))
    kv2 = torch.empty_like(c.kv_pages)
    kv2[perm.cuda()] = c.kv_pages
    c.kv_pages = kv2
    c.page_indices = perm.numpy().astype(np.int32)[c.page_indices]
    d = _run_gpu(c)
    assert torch.equal(a[:n], d[:n])


def test_kv_len_one_and_equal_scores():
    _say("kv_len=1 and Q=0")
    c = wl.make_gqa([(1, 1), (1, 50)], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=7,
                    device="cuda")
    c.q[0].zero_()
    c.q[1].zero_()
    out = _run_gpu(c).float().cpu()
    kv = c.kv_pages.float().cpu()
    pg = int(c.page_indices[0, 0])
    for h in range(8):
        assert torch.equal(out[0, h], kv[pg, 0, 2 * (h // 4) + 1].bfloat16().float())
    # Q = 0: the mean of the 50 visible values.
    rows = [kv[int(c.page_indices[1, t // 16]), t % 16] for t in range(50)]
    mean = torch.stack(rows).double().mean(0)
    for h in range(8):
        want = mean[2 * (h // 4) + 1]
        assert (out[1, h].double() - want).abs().max() < 1e-2


def test_empty_batch_and_padding_rows_untouched():
    _say("num_seqs=0 and padding rows")
    c = wl.make_gqa([(3, 40), (1, 20)], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=8,
                    device="cuda", extra_tokens=5)
    kl, pi, cu, ns = _dev_meta(c)
    sentinel = torch.full_like(c.q, 7.0)
    out = rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, torch.zeros_like(ns), out=sentinel.clone(),
                          sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel)
    out = rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, out=sentinel.clone(), sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out[4:], sentinel[4:])
    want = _run_oracle(c)
    assert_close(as_f64(out)[:4], want[:4], *TOL["bf16"])


def test_debug_validate_rejects_bad_metadata():
    _say("debug_validate")
    c = wl.make_gqa([(3, 40), (1, 20)], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=9,
                    device="cuda")
    kl, pi, cu, ns = _dev_meta(c)
    bad_kl = kl.clone()
    bad_kl[0] = 2   # q_len 3 > kv_len 2
    with pytest.raises(rpa.RpaError, match="q_len"):
        rpa.rpa_forward(c.q, c.kv_pages, bad_kl, pi, cu, ns, debug_validate=True)
    bad_pi = pi.clone()
    bad_pi[1, 0] = c.kv_pages.shape[0]
    with pytest.raises(rpa.RpaError, match="page id"):
        rpa.rpa_forward(c.q, c.kv_pages, kl, bad_pi, cu, ns, debug_validate=True)
    with pytest.raises(rpa.RpaError, match="num_seqs"):
        rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns + 5, debug_validate=True)
    out = rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, debug_validate=True, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    assert_close(as_f64(out), _run_oracle(c), *TOL["bf16"])


# --------------------------------------------------------- full workloads --

def test_decode_gqa_full_size_sampled():
    _say("decode_gqa full size (128 seqs, kv 512..8192), sampled rows")
    c = wl.decode_gqa(device="cuda")
    got = _run_gpu(c)
    tokens = np.arange(0, 128, 5)
    want = _run_oracle(c, tokens=tokens)
    _check(c, got, want, "bf16", tokens=tokens)


def _mixed_sample(c, block=64):
    """Every decode token, plus the first and last token of every 64-token
    query block of every prefill chunk (the prefill kernel's query-block size
    at 32/8 heads), so each of its tiles has rows compared."""
    toks = []
    for i in range(c.num_seqs):
        a, b = int(c.cu_q_lens[i]), int(c.cu_q_lens[i + 1])
        if b - a == 1:
            toks.append(a)
            continue
        for t0 in range(a, b, block):
            toks += [t0, min(t0 + block, b) - 1]
    return np.unique(np.array(toks, np.int32))


@pytest.mark.parametrize("variant", ["ordered", "shuffled", "q_x16"])
def test_mixed_gqa_full_size_sampled(variant):
    """The mixed batch at full size (120 decodes + 8 prefill chunks, fp8 pool,
    window 4096, cap 50), in the generator's order, in a shuffled sequence
    order, and with queries x16 so the soft cap is engaged."""
    _say(f"mixed_gqa full size {variant}, every decode + both ends of every prefill block")
    c = wl.mixed_gqa(device="cuda", shuffle_order=variant == "shuffled",
                     q_value_scale=16.0 if variant == "q_x16" else 1.0)
    got = _run_gpu(c)
    tokens = _mixed_sample(c)
    assert len(tokens) > 400
    want = _run_oracle(c, tokens=tokens)
    _check(c, got, want, "fp8", tokens=tokens)


# ------------------------------------------------------------- kv update --

def test_kv_update_combined_bit_exact():
    _say("kv_cache_update combined")
    seqs = [(1, 37), (20, 90), (3, 3)]
    c = wl.make_gqa(seqs, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=10, device="cuda",
                    spare_pages=2)
    T = int(c.cu_q_lens[-1])
    g = torch.Generator(device="cuda").manual_seed(3)
    newk = torch.randn((T, 2, 128), generator=g, device="cuda").bfloat16()
    newv = torch.randn((T, 2, 128), generator=g, device="cuda").bfloat16()
    host = storage(c.kv_pages)[0].copy()
    kl, pi, cu, ns = _dev_meta(c)
    rpa.kv_cache_update(rpa.LAYOUT_COMBINED_GQA, newk, newv, c.kv_pages, kv_lens=kl,
                        page_indices=pi, cu_q_lens=cu, num_seqs=ns, debug_validate=True)
    torch.cuda.synchronize()
    oracle.kv_update(oracle.LAYOUT_COMBINED_GQA, storage(newk)[0], storage(newv)[0], host, None,
                     oracle.BF16, kv_lens=c.kv_lens, page_indices=c.page_indices,
                     cu_q_lens=c.cu_q_lens, num_seqs=c.num_seqs)
    assert np.array_equal(storage(c.kv_pages)[0], host)


@pytest.mark.parametrize("fused", [False, True])
def test_kv_update_mla_bit_exact(fused):
    _say(f"kv_cache_update mla fused={fused}")
    c = wl.make_mla([(1, 100), (5, 64), (2, 200)], num_heads=4, page_size=64, seed=11,
                    device="cuda", spare_pages=2)
    if fused:
        P, ps = c.cache_kv_c.shape[:2]
        cache = torch.randn((P, ps, 640), device="cuda").bfloat16()
        host = storage(cache)[0].copy()
        loc = torch.tensor([5, -1, 70, 3, 129, -1, 64, 200], dtype=torch.int32, device="cuda")
        rpa.kv_cache_update(rpa.LAYOUT_MLA_FUSED, c.new_kv_c, c.new_k_pe, cache, slot_loc=loc,
                            debug_validate=True)
        torch.cuda.synchronize()
        oracle.kv_update(oracle.LAYOUT_MLA_FUSED, storage(c.new_kv_c)[0], storage(c.new_k_pe)[0],
                         host, None, oracle.BF16, slot_loc=loc.cpu().numpy())
        assert np.array_equal(storage(cache)[0], host)
        return
    ha = storage(c.cache_kv_c)[0].copy()
    hb = storage(c.cache_k_pe)[0].copy()
    kl, pi, cu, ns = _dev_meta(c)
    rpa.kv_cache_update(rpa.LAYOUT_MLA_SPLIT, c.new_kv_c, c.new_k_pe, c.cache_kv_c, c.cache_k_pe,
                        kv_lens=kl, page_indices=pi, cu_q_lens=cu, num_seqs=ns)
    torch.cuda.synchronize()
    oracle.kv_update(oracle.LAYOUT_MLA_SPLIT, storage(c.new_kv_c)[0], storage(c.new_k_pe)[0], ha,
                     hb, oracle.BF16, kv_lens=c.kv_lens, page_indices=c.page_indices,
                     cu_q_lens=c.cu_q_lens, num_seqs=c.num_seqs)
    assert np.array_equal(storage(c.cache_kv_c)[0], ha)
    assert np.array_equal(storage(c.cache_k_pe)[0], hb)


def test_kv_update_rejects_aliased_slots():
    _say("kv_cache_update aliasing")
    c = wl.make_mla([(1, 100)], num_heads=4, page_size=64, seed=12, device="cuda")
    P, ps = c.cache_kv_c.shape[:2]
    cache = torch.zeros((P, ps, 640), device="cuda", dtype=torch.bfloat16)
    loc = torch.tensor([7], dtype=torch.int32, device="cuda")
    two_kvc = torch.cat([c.new_kv_c, c.new_kv_c])
    two_kpe = torch.cat([c.new_k_pe, c.new_k_pe])
    with pytest.raises(rpa.RpaError, match="twice"):
        rpa.kv_cache_update(rpa.LAYOUT_MLA_FUSED, two_kvc, two_kpe, cache,
                            slot_loc=torch.cat([loc, loc]), debug_validate=True)


def test_rows_whose_window_starts_in_a_later_block():
    """Rows of one tile whose visible keys begin in different key blocks (the
    first block is fully masked for some rows only): regression test for the
    per-row rescale when other rows of the wave move their reference max."""
    _say("window starting in a later block")
    for Hq, Hkv in [(16, 16), (16, 4), (8, 1)]:
        c = wl.make_gqa([(40, 1200), (70, 70), (3, 1000)], num_q_heads=Hq, num_kv_heads=Hkv,
                        head_dim=128, page_size=32, q_dtype=torch.bfloat16,
                        kv_dtype=torch.bfloat16, seed=102, device="cuda", sliding_window=100,
                        name=f"late-window-{Hq}-{Hkv}")
        _check(c, _run_gpu(c), _run_oracle(c), "bf16")


def test_bf16_values_beyond_half_range_stay_finite():
    """Split decodes of a bf16 pool whose values exceed IEEE half's range
    (|V| up to ~4e5): the split partials must not saturate, so the output is
    finite and matches the oracle to the bf16 tolerance scaled by |V|."""
    _say("bf16 values beyond half range")
    scale = 1.0e5
    c = wl.make_gqa([(1, 9000), (1, 3000), (2, 5000)], num_q_heads=32, num_kv_heads=8,
                    head_dim=128, page_size=16, q_dtype=torch.bfloat16,
                    kv_dtype=torch.bfloat16, seed=90, device="cuda", name="big-v")
    c.kv_pages[:, :, 1::2] *= scale
    got = _run_gpu(c)
    n = int(c.cu_q_lens[c.num_seqs])
    assert torch.isfinite(got[:n].float()).all()
    want = _run_oracle(c)
    assert_close(as_f64(got)[:n] / scale, want[:n] / scale, *TOL["bf16"], what="big-v")


_CAPTURE_FIRST = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import ragged_paged_attention_rpa_amd as rpa
from ragged_paged_attention_rpa_amd import workloads as wl
c = wl.make_gqa([(4, 4), (2, 1025), (24, 900)], num_q_heads=16, num_kv_heads=2, head_dim=128,
                page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=401,
                device="cuda", extra_tokens=4096, name="capture-first")
d = "cuda"
kl, pi = torch.from_numpy(c.kv_lens).to(d), torch.from_numpy(c.page_indices).to(d)
cu, ns = torch.from_numpy(c.cu_q_lens).to(d), torch.tensor([c.num_seqs], dtype=torch.int32, device=d)
ws = torch.empty(rpa.rpa_workspace_size(kl, pi, c.q.shape[0], 16, 2, 128), dtype=torch.uint8,
                 device=d)
out = torch.zeros_like(c.q)
def call():
    rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, sm_scale=c.sm_scale, out=out, workspace=ws)
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        call()                  # the process's first rpa_forward: under capture
torch.cuda.current_stream().wait_stream(s)
torch.cuda.synchronize()
T = int(c.cu_q_lens[c.num_seqs])
g.replay(); torch.cuda.synchronize()
captured = out[:T].clone()
out.zero_(); call(); torch.cuda.synchronize()   # eager: creates the side stream
assert torch.equal(out[:T], captured), "capture-first replay differs from eager"
out.zero_(); g.replay(); torch.cuda.synchronize()
assert torch.equal(out[:T], captured), "second replay differs"
print("capture-first ok", rpa.last_path())
"""


def test_first_call_under_capture_stays_on_one_stream():
    """A process whose very first rpa_forward is captured: the library must not
    create its side stream mid-capture (it stays on the caller's stream), and
    the replays equal the later eager call (run in a fresh process so no
    earlier call has created the side stream)."""
    import os
    import subprocess
    import sys
    _say("first call under capture (fresh process)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _CAPTURE_FIRST, root], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "capture-first ok" in r.stdout


def test_last_path_names_the_kernel_path():
    _say("rpa_last_path")
    c = wl.make_gqa([(1, 100), (40, 200)], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=91,
                    device="cuda")
    _run_gpu(c)
    assert rpa.last_path() == "gqa_mfma"          # bf16, no room for a prefill chunk
    c = wl.make_gqa([(1, 100), (400, 600)], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=91,
                    device="cuda")
    _run_gpu(c)
    assert rpa.last_path() == "gqa_mfma_prefill"
    c = wl.make_gqa([(1, 100), (3, 200)], num_q_heads=8, num_kv_heads=2, head_dim=64,
                    page_size=16, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, seed=92,
                    device="cuda")
    _check(c, _run_gpu(c), _run_oracle(c), "bf16")
    assert rpa.last_path() == "gqa_generic"


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_explicit_split_keys_agree_with_the_oracle(kv):
    """Decode splits fixed by the caller (rpa_opts.split_keys) instead of the
    tile table: 64-key splits (the smallest; long sequences hit the 16-split
    cap and take larger chunks), 448 and 8192 keys, with a window and a cap,
    on decodes and a short prefill chunk; each matches the oracle."""
    _say(f"explicit split sizes ({kv})")
    kvd = torch.bfloat16 if kv == "bf16" else torch.float8_e4m3fn
    seqs = [(1, 5000), (1, 700), (2, 64), (1, 1), (1, 3000), (7, 2100), (1, 12345)]
    c = wl.make_gqa(seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=kvd, seed=460, device="cuda",
                    sliding_window=4000, soft_cap=30.0, k_scale=0.5 if kv == "fp8" else None,
                    v_scale=0.5 if kv == "fp8" else None, name=f"split-{kv}")
    want = _run_oracle(c)
    outs = []
    for sk in (None, 64, 448, 8192):
        got = _run_gpu(c, split_keys=sk)
        _check(c, got, want, kv)
        outs.append(as_f64(got))
    rows = np.arange(int(c.cu_q_lens[c.num_seqs]))
    for o in outs[1:]:
        assert_close(o[rows], outs[0][rows], *TOL[kv], what=f"split-{kv} vs table")


INT8_CASES = {
    # prefill chunks (prefill kernel) next to decodes (one-byte decode kernel)
    "mixed": ([(1, 3000), (300, 1200), (1, 17), (64, 64), (1, 5000), (700, 2100)], 16, 4, 128, 16,
              "gqa_mfma_prefill"),
    # page size 4 (below the prefill kernel's minimum): every tile on the tile
    # kernel's one-byte blocks, decodes and a short chunk
    "tile-kernel-ps4": ([(1, 3000), (40, 700), (1, 17), (1, 9000), (3, 64)], 32, 8, 128, 4,
                        "gqa_mfma"),
    # head_dim 64: the generic kernel
    "generic-d64": ([(1, 300), (5, 70), (1, 1)], 8, 2, 64, 16, "gqa_generic"),
}


@pytest.mark.parametrize("mode", list(INT8_CASES))
def test_int8_pool(mode):
    """int8 pools with per-tensor scales (the integers of N(0,1) quantised at
    1/32, dequantised by k_scale = v_scale = 1/32), on every kernel path."""
    seqs, hq, hkv, d, ps, path = INT8_CASES[mode]
    _say(f"int8 pool ({mode})")
    c = wl.make_gqa(seqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=torch.int8, seed=480, device="cuda",
                    sliding_window=2500 if mode == "mixed" else None,
                    soft_cap=30.0 if mode != "tile-kernel-ps4" else None, k_scale=1 / 32,
                    v_scale=1 / 32,
                    name=f"int8-{mode}")
    got = _run_gpu(c)
    assert rpa.last_path() == path
    _check(c, got, _run_oracle(c), "bf16")


@pytest.mark.parametrize("fused", [False, True])
def test_int4_pool(fused):
    """Packed int4 pools (the integers of 2 N(0,1), dequantised by k_scale =
    v_scale = 1/2) on the generic kernel, with a window and a cap; with
    ``fused`` the call also scatters the step's new rows (packed bytes), and
    the pool afterwards is bit-exact against the oracle's scatter."""
    _say(f"int4 pool (fused={fused})")
    seqs = [(1, 700), (30, 400), (1, 17), (8, 8), (3, 1200)]
    c = wl.make_gqa(seqs, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                    q_dtype=torch.bfloat16, kv_dtype=torch.uint8, seed=520, device="cuda",
                    sliding_window=300, soft_cap=30.0, k_scale=0.5, v_scale=0.5, spare_pages=2,
                    name=f"int4-fused{int(fused)}")
    new_kv = None
    if fused:
        T = int(c.cu_q_lens[-1])
        new_kv = wl.randn((T, 8, 128), torch.uint8, wl._gen("cuda", 521), "cuda")
        host = storage(c.kv_pages)[0].copy()
        oracle.kv_update(oracle.LAYOUT_COMBINED_GQA, storage(new_kv[:, 0::2])[0],
                         storage(new_kv[:, 1::2])[0], host, None, oracle.INT4,
                         kv_lens=c.kv_lens, page_indices=c.page_indices, cu_q_lens=c.cu_q_lens,
                         num_seqs=c.num_seqs)
    got = _run_gpu(c, new_kv=new_kv) if fused else _run_gpu(c)
    assert rpa.last_path() == "gqa_generic"
    if fused:
        assert np.array_equal(storage(c.kv_pages)[0], host)
    _check(c, got, _run_oracle(c), "bf16")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_fp8_queries_with_q_scale(kv):
    """fp8 queries dequantised by q_scale (widened exactly to bf16 on load),
    on a mixed batch; the output is bf16."""
    _say(f"fp8 queries ({kv} pool)")
    kvd = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "int8": torch.int8}[kv]
    ks = {"bf16": None, "fp8": 0.5, "int8": 1 / 32}[kv]
    c = wl.make_gqa([(1, 2000), (400, 1500), (1, 33), (5, 600)], num_q_heads=16, num_kv_heads=4,
                    head_dim=128, page_size=16, q_dtype=torch.float8_e4m3fn, kv_dtype=kvd,
                    seed=490, device="cuda", q_value_scale=4.0, k_scale=ks, v_scale=ks,
                    name=f"fp8q-{kv}")
    got = _run_gpu(c, q_scale=0.25)
    assert got.dtype == torch.bfloat16
    q, qd = storage(c.q)
    kvs, kd = storage(c.kv_pages)
    want = oracle.rpa(q, qd, kvs, kd, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs,
                      sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale, q_scale=0.25)
    _check(c, got, want, "fp8" if kv == "fp8" else "bf16")


@pytest.mark.parametrize("variant", ["plain", "window-cap"])
def test_fp8_scores_over_fp8_pool(variant):
    """fp8 queries over an fp8 pool: the decode tiles take their scores from
    the fp8 MFMA on the raw bytes; split keys, ragged tails, a window and a
    soft cap, against the oracle's exact fp8 decode."""
    win, cap = (None, None) if variant == "plain" else (1500, 30.0)
    _say(f"fp8 scores over an fp8 pool ({variant})")
    c = wl.make_gqa([(1, 9000), (1, 1), (1, 47), (200, 900), (1, 4100), (3, 3000), (1, 16)],
                    num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=16,
                    q_dtype=torch.float8_e4m3fn, kv_dtype=torch.float8_e4m3fn, seed=610,
                    device="cuda", q_value_scale=4.0, k_scale=0.5, v_scale=0.5,
                    sliding_window=win, soft_cap=cap, name=f"fp8q-fp8kv-{variant}")
    got = _run_gpu(c, q_scale=0.25)
    assert rpa.last_path() == "gqa_mfma_prefill"
    q, qd = storage(c.q)
    kvs, kd = storage(c.kv_pages)
    want = oracle.rpa(q, qd, kvs, kd, c.kv_lens, c.page_indices, c.cu_q_lens, c.num_seqs,
                      sm_scale=c.sm_scale, sliding_window=win, soft_cap=cap,
                      k_scale=c.k_scale, v_scale=c.v_scale, q_scale=0.25)
    _check(c, got, want, "fp8")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_tiny_cap_with_zero_queries(kv):
    """A soft cap of 1e-25 (the series coefficients overflow fp32, so 0 * inf
    would follow for a zero score; the exact form must serve) over a batch
    where one decode and one prefill chunk have all-zero queries (every score
    exactly 0): uniform weights, no NaN."""
    _say(f"tiny cap, zero queries ({kv})")
    kvd = torch.bfloat16 if kv == "bf16" else torch.float8_e4m3fn
    ks = None if kv == "bf16" else 0.5
    c = wl.make_gqa([(1, 700), (1, 300), (300, 900), (200, 400), (1, 33)], num_q_heads=32,
                    num_kv_heads=8, head_dim=128, page_size=16, q_dtype=torch.bfloat16,
                    kv_dtype=kvd, seed=620, device="cuda", soft_cap=1e-25, k_scale=ks,
                    v_scale=ks, name=f"tinycap-{kv}")
    cu = c.cu_q_lens
    for i in (1, 3):
        c.q[int(cu[i]):int(cu[i + 1])].zero_()
    got = _run_gpu(c)
    assert torch.isfinite(got[: int(cu[-1])].float()).all()
    _check(c, got, _run_oracle(c), "fp8" if kv == "fp8" else "bf16")


FUSED_CASES = {
    # (seqs, Hq, Hkv, D, page size, pool dtype, window, cap, kernel path)
    "bf16-prefill-kernel": ([(1, 3000), (300, 1200), (1, 17), (64, 64), (1, 9000), (700, 2100)],
                            16, 4, 128, 16, torch.bfloat16, 2500, 30.0, "gqa_mfma_prefill"),
    "fp8-decode8": ([(1, 3000), (130, 900), (1, 1), (2, 5000)], 32, 8, 128, 16,
                    torch.float8_e4m3fn, None, 50.0, "gqa_mfma_prefill"),
    "int8-tile-ps4": ([(1, 3000), (40, 700), (1, 17), (1, 9000), (3, 64)], 32, 8, 128, 4,
                      torch.int8, 1000, None, "gqa_mfma"),
    "bf16-generic-d64": ([(1, 300), (5, 70), (1, 1), (17, 17)], 8, 2, 64, 16, torch.bfloat16,
                         None, None, "gqa_generic"),
}


@pytest.mark.parametrize("mode", list(FUSED_CASES))
def test_fused_cache_update(mode):
    """rpa_forward with the step's new rows (new_kv): the pool afterwards is
    bit-exact against the oracle's scatter, the outputs match the oracle on
    the updated pool, and they equal kv_cache_update + rpa_forward bit for bit
    (the keys of the step's tokens come from new_kv, the same values)."""
    seqs, hq, hkv, d, ps, kvd, win, cap, path = FUSED_CASES[mode]
    _say(f"fused cache update ({mode})")
    scales = {torch.float8_e4m3fn: 0.5, torch.int8: 1 / 32}.get(kvd)
    c = wl.make_gqa(seqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    q_dtype=torch.bfloat16, kv_dtype=kvd, seed=500, device="cuda",
                    sliding_window=win, soft_cap=cap, k_scale=scales, v_scale=scales,
                    spare_pages=2, name=f"fused-{mode}")
    T = int(c.cu_q_lens[-1])
    new_kv = wl.randn((T, 2 * hkv, d), kvd, wl._gen("cuda", 501), "cuda")
    host = storage(c.kv_pages)[0].copy()
    oracle.kv_update(oracle.LAYOUT_COMBINED_GQA, storage(new_kv[:, 0::2])[0],
                     storage(new_kv[:, 1::2])[0], host, None, storage(c.kv_pages)[1],
                     kv_lens=c.kv_lens, page_indices=c.page_indices, cu_q_lens=c.cu_q_lens,
                     num_seqs=c.num_seqs)
    two_step_pool = c.kv_pages.clone()
    got = _run_gpu(c, new_kv=new_kv, debug_validate=True)
    assert rpa.last_path() == path
    assert np.array_equal(storage(c.kv_pages)[0], host)
    kl, pi, cu, ns = _dev_meta(c)
    rpa.kv_cache_update(rpa.LAYOUT_COMBINED_GQA, new_kv[:, 0::2].contiguous(),
                        new_kv[:, 1::2].contiguous(), two_step_pool, kv_lens=kl, page_indices=pi,
                        cu_q_lens=cu, num_seqs=ns)
    ref = rpa.rpa_forward(c.q, two_step_pool, kl, pi, cu, ns, sm_scale=c.sm_scale,
                          sliding_window=c.sliding_window, soft_cap=c.soft_cap,
                          k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    rows = slice(0, T)
    assert torch.equal(got[rows], ref[rows])
    want = _run_oracle(c)  # the device pool is the updated one (checked above)
    _check(c, got, want, "fp8" if kvd == torch.float8_e4m3fn else "bf16")
