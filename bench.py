#!/usr/bin/env python3
"""Benchmark of the ragged paged attention hot path on one MI355X.

A "step" is one full call of the entry point over one synthetic batch (all
launches: work-list plan, attention tiles, split merge). Inputs are resident
in HBM before timing starts. Prints ONE JSON line.

Workloads (--config):
  decode_gqa  (default) 128 decodes, kv_len U[512,8192], 32/8 heads, d128,
              page 16, bf16 — metric: decode KV GB/s (algorithmic KV bytes)
  mixed_gqa   120 decodes + 8 prefill chunks, fp8 KV, window 4096, cap 50
  mla_decode  64 MLA decodes, kv_len U[4096,32768], 128 heads, page 64
  sparse_mla  4096 queries x 32 page units of 64 tokens, 16 heads
  tiny_gqa    3 sequences, fp32

The roofline object refers to the dominant kernel, timed with HIP events that
the library records on its own stream right around that kernel. `traffic`
comes from the committed rocprofv3 PMC summary for the same workload when it
was taken on the current kernel source, else null. `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV GB/s (% HBM peak) + prefill TFLOPS (% MFMA peak), tokens/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3

KERNEL_SOURCES = {
    "decode_gqa": "ragged_paged_attention_rpa_amd/csrc/gqa_attn.hip",
    "mixed_gqa": "ragged_paged_attention_rpa_amd/csrc/gqa_prefill.hip",
    "tiny_gqa": "ragged_paged_attention_rpa_amd/csrc/gqa_attn.hip",
    "mla_decode": "ragged_paged_attention_rpa_amd/csrc/mla_decode.hip",
    "sparse_mla": "ragged_paged_attention_rpa_amd/csrc/mla_attn.hip",
    # the mixed batch's decode subset (--decode-subset only): the fp8 decode kernel
    "mixed_gqa_decode": "ragged_paged_attention_rpa_amd/csrc/gqa_attn.hip",
}
KERNEL_NAMES = {
    "decode_gqa": "gqa_tile_kernel",
    "mixed_gqa": "gqa_prefill_kernel",
    "tiny_gqa": "gqa_generic_kernel",
    "mla_decode": "mla_tile_kernel",
    "sparse_mla": "sparse_mla_kernel",
    "mixed_gqa_decode": "gqa_decode8_kernel",
}


def source_sha(config):
    """Hash of the dominant kernel's source plus the shared device header."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[config], "ragged_paged_attention_rpa_amd/csrc/rpa_device.h"):
        p = os.path.join(ROOT, rel)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ work counts --

def gqa_work(case):
    """Algorithmic work of one GQA call: visible (query, key) pairs and the
    bytes of the distinct visible K/V rows each sequence must read."""
    W = case.sliding_window or 0
    Hq, Hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    eb = case.kv_pages.element_size()
    pairs = 0
    kv_rows = 0
    dec_rows = pre_pairs = 0
    dec_bytes = pre_bytes = 0
    for i in range(case.num_seqs):
        ql = int(case.cu_q_lens[i + 1] - case.cu_q_lens[i])
        L = int(case.kv_lens[i])
        pos = np.arange(L - ql, L, dtype=np.int64)
        vis = pos + 1 if W == 0 else np.minimum(pos + 1, W)
        p = int(vis.sum())
        lo = 0 if W == 0 else max(0, L - ql - W + 1)
        rows = L - lo
        pairs += p
        kv_rows += rows
        if ql == 1:
            dec_rows += rows
            dec_bytes += rows * 2 * Hkv * D * eb
        else:
            pre_pairs += p
            pre_bytes += rows * 2 * Hkv * D * eb
    return {
        "kv_bytes": kv_rows * 2 * Hkv * D * eb,
        "flops": pairs * Hq * 4 * D,
        "q_tokens": int(case.cu_q_lens[case.num_seqs]),
        "decode_kv_bytes": dec_bytes,
        "prefill_flops": pre_pairs * Hq * 4 * D,
        "prefill_kv_bytes": pre_bytes,
    }


def mla_work(case, heads, dl=512, dr=64):
    """Visible (query, key) pairs x heads x (2*(dl+dr) for QK + 2*dl for PV);
    bytes of the distinct latent rows read (dl + dr bf16 per key, pad excluded)."""
    pairs = rows = 0
    for i in range(case.num_seqs):
        ql = int(case.cu_q_lens[i + 1] - case.cu_q_lens[i])
        L = int(case.kv_lens[i])
        pairs += int((np.arange(L - ql, L) + 1).sum())
        rows += L
    return {"kv_bytes": rows * (dl + dr) * 2, "flops": pairs * heads * (2 * (dl + dr) + 2 * dl),
            "q_tokens": int(case.cu_q_lens[case.num_seqs])}


def sparse_work(case):
    S, H = case.q.shape[0], case.q.shape[1]
    dk = case.kv_lora_rank + case.rope_dim
    keys = 0
    rb = case.read_block
    for s in range(S):
        u = case.indices[s]
        u = u[u >= 0]
        kp = (u[:, None] * rb + np.arange(rb)[None, :]).ravel()
        keys += int(((kp <= case.positions[s]) & (kp < case.seq_len)).sum())
    return {"gathered_bytes": keys * dk * 2, "flops": keys * H * 2 * (dk + case.kv_lora_rank),
            "q_tokens": S}


# --------------------------------------------------------------- runners --

def _storage(t):
    """(numpy storage array, oracle dtype code) of a torch tensor."""
    import torch
    import oracle
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy(), oracle.F32
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), oracle.BF16
    return t.view(torch.uint8).numpy(), oracle.FP8_E4M3


class HipEvents:
    """hipEvent_t pairs created through the HIP runtime (torch creates its
    events lazily, so their handles are not usable before torch records them)."""

    def __init__(self, n):
        import ctypes
        self._ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0
            assert self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def elapsed_ms(self, k, missing_ok=False):
        """Milliseconds between pair k's events; with missing_ok, None when the
        pair was never recorded (its kernel was not launched)."""
        ms = self._ct.c_float()
        rc = self.hip.hipEventElapsedTime(self._ct.byref(ms), self.pairs[k][0], self.pairs[k][1])
        if rc != 0:
            if missing_ok:
                # Clear the error the query left as HIP's last error, which the
                # library's next launch check would otherwise report.
                self.hip.hipGetLastError()
                return None
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        self.pairs = []


FLUSH_BYTES = 512 << 20
_flush_buf = []


def cache_flush(torch):
    """Reads a 512 MB scratch buffer on the current stream, which evicts the
    L2s and the 256 MB MALL: the step after it reads its inputs from HBM. A
    read, not a write: a written buffer leaves dirty lines whose write-back
    then competes with the next step's reads (measured: the decode batch's
    kernel 14% slower after a 512 MB fill than after this read)."""
    if not _flush_buf:
        _flush_buf.append(torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda"))
        _flush_buf.append(torch.zeros((), dtype=torch.int64, device="cuda"))
    torch.sum(_flush_buf[0], dim=0, dtype=torch.int64, out=_flush_buf[1])


def timed_loop(torch, rpa, fn, steps, warmup, split=False, flush=None):
    """Runs `warmup` untimed steps, then exactly `steps` steps between two
    device synchronisations; returns (wall ms/step, mean and median duration
    of the dominant kernel(s) in ms from the library's event hook, and a dict
    with their minimum and, with `split`, the mean and minimum durations of
    rpa_forward's prefill-tile and decode-tile kernels in ms). With `flush`,
    it runs before every step (cold caches; the wall time then includes it)."""
    for _ in range(warmup):
        if flush:
            flush()
        fn()
    torch.cuda.synchronize()
    ev = HipEvents(steps)
    evs = HipEvents(2 * steps) if split else None
    lib = rpa.load_library()
    t0 = time.perf_counter()
    for k in range(steps):
        if flush:
            flush()
        lib.rpa_set_profile_events(ev.pairs[k][0], ev.pairs[k][1])
        if split:
            lib.rpa_set_profile_events_split(evs.pairs[2 * k][0], evs.pairs[2 * k][1],
                                             evs.pairs[2 * k + 1][0], evs.pairs[2 * k + 1][1])
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.rpa_set_profile_events(None, None)
    kern = [ev.elapsed_ms(k) for k in range(steps)]
    ev.close()
    parts = {"kernel_ms_min": float(np.min(kern))}
    if split:
        lib.rpa_set_profile_events_split(None, None, None, None)
        # The prefill-tile kernel is not launched on a batch without room for
        # prefill chunks (its events then stay unrecorded).
        pre = [evs.elapsed_ms(2 * k, missing_ok=True) for k in range(steps)]
        dec = [evs.elapsed_ms(2 * k + 1) for k in range(steps)]
        evs.close()
        pre_ok = all(p is not None for p in pre)
        parts.update(prefill_kernel_ms=float(np.mean(pre)) if pre_ok else None,
                     decode_kernel_ms=float(np.mean(dec)),
                     prefill_kernel_ms_min=float(np.min(pre)) if pre_ok else None,
                     decode_kernel_ms_min=float(np.min(dec)))
    return (t1 - t0) * 1e3 / steps, float(np.mean(kern)), float(np.median(kern)), parts


def graph_loop(torch, fn, steps, warmup):
    """Wall ms per step of `steps` replays of one captured call of `fn` (a HIP
    graph: the call's launches without host launch overhead), after `warmup`
    untimed replays, between two device synchronisations."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return ms


def measure(args, torch, rpa, fn, split=False):
    """The warm loop (back-to-back steps: the timed region behind `value` and
    the roofline) and the cold loop (a read of a 512 MB buffer before each step
    evicts L2 and MALL, so each step reads its inputs from HBM; reported beside
    the warm figures). --cache warm runs only the warm loop (profiling runs, so
    a trace holds exactly the launches the roofline averages); --cache cold
    only the cold one. Returns (primary, cold or None)."""
    mode = getattr(args, "cache", "both")
    cold = None
    if mode != "warm":
        cold = timed_loop(torch, rpa, fn, args.steps, max(1, args.warmup // 2), split,
                          flush=lambda: cache_flush(torch))
    warm = timed_loop(torch, rpa, fn, args.steps, args.warmup, split) if mode != "cold" else None
    if warm is not None and getattr(args, "graph", "on") == "on":
        # The step the line reports: the call replayed from a HIP graph, as a
        # serving loop issues it; the eager wall time stays beside it.
        gms = graph_loop(torch, fn, args.steps, args.warmup)
        warm[3]["ms_per_step_eager"] = warm[0]
        warm = (gms,) + tuple(warm[1:])
    return (warm or cold), cold


def cold_summary(cold, key="kernel"):
    """Cold-start kernel durations (ms) from a measure() result."""
    if cold is None:
        return None
    _, kmean, kmed, parts = cold
    out = {"flush": "512 MB read before each step", "kernel_ms_mean": kmean,
           "kernel_ms_median": kmed, "kernel_ms_min": parts["kernel_ms_min"]}
    for k in ("prefill_kernel_ms", "decode_kernel_ms"):
        if k in parts:
            out[k] = parts[k]
            out[k + "_min"] = parts[k + "_min"]
    return out


def setup_gqa(torch, rpa, wl, config):
    case = {"decode_gqa": wl.decode_gqa, "mixed_gqa": wl.mixed_gqa,
            "tiny_gqa": wl.tiny_gqa}[config](device="cuda")
    dev = "cuda"
    kl = torch.from_numpy(case.kv_lens).to(dev)
    pi = torch.from_numpy(case.page_indices).to(dev)
    cu = torch.from_numpy(case.cu_q_lens).to(dev)
    ns = torch.tensor([case.num_seqs], dtype=torch.int32, device=dev)
    out = torch.empty_like(case.q)
    need = rpa.rpa_workspace_size(kl, pi, case.q.shape[0], case.num_q_heads, case.num_kv_heads,
                                  case.head_dim)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def fn():
        rpa.rpa_forward(case.q, case.kv_pages, kl, pi, cu, ns, sm_scale=case.sm_scale,
                        sliding_window=case.sliding_window, soft_cap=case.soft_cap,
                        k_scale=case.k_scale, v_scale=case.v_scale, out=out, workspace=ws)
    # `ns` is the device-side sequence count the call reads: setting it to the
    # number of leading decode sequences runs the decode subset of the batch.
    fn.ns = ns
    return case, fn


def cpu_baseline_gqa(case, work, budget_s=15.0, prefill_only=False):
    """Times the CPU oracle on a bounded sample of the workload's query tokens
    (with prefill_only, of the tokens of its prefill chunks)."""
    import oracle
    q, qd = _storage(case.q)
    kv, kd = _storage(case.kv_pages)
    T = int(case.cu_q_lens[case.num_seqs])
    rng = np.random.default_rng(0)
    pool = np.arange(T)
    if prefill_only:
        ql = np.diff(case.cu_q_lens[:case.num_seqs + 1])
        pool = np.concatenate([np.arange(case.cu_q_lens[i], case.cu_q_lens[i + 1])
                               for i in range(case.num_seqs) if ql[i] > 1])
    order = pool[rng.permutation(len(pool))]

    def run(tokens):
        t0 = time.perf_counter()
        oracle.rpa(q, qd, kv, kd, case.kv_lens, case.page_indices, case.cu_q_lens, case.num_seqs,
                   sm_scale=case.sm_scale, sliding_window=case.sliding_window,
                   soft_cap=case.soft_cap, k_scale=case.k_scale, v_scale=case.v_scale,
                   tokens=tokens)
        return time.perf_counter() - t0

    probe = np.sort(order[:max(1, min(len(order), 8))])
    dt = run(probe)
    n = int(min(len(order), max(len(probe), len(probe) * budget_s / max(dt, 1e-3))))
    tokens = np.sort(order[:n])
    dt = run(tokens)
    # Work of the sampled tokens: their visible keys (bytes of K/V rows read,
    # counted once per token) and their flops.
    W = case.sliding_window or 0
    seq_of = np.searchsorted(case.cu_q_lens[1:case.num_seqs + 1], tokens, side="right")
    rows = 0
    for t, i in zip(tokens, seq_of):
        ql = int(case.cu_q_lens[i + 1] - case.cu_q_lens[i])
        L = int(case.kv_lens[i])
        pos = L - ql + (int(t) - int(case.cu_q_lens[i]))
        rows += pos + 1 if W == 0 else min(pos + 1, W)
    eb = case.kv_pages.element_size()
    kv_bytes = rows * 2 * case.num_kv_heads * case.head_dim * eb
    flops = rows * case.num_q_heads * 4 * case.head_dim
    what = "prefill-chunk query tokens" if prefill_only else "query tokens"
    return {"seconds": dt, "tokens": len(tokens), "kv_bytes": kv_bytes, "flops": flops,
            "cores": oracle.num_threads(),
            "sample": f"{len(tokens)} of {len(pool)} {what} (all q heads), drawn with seed 0"}


def load_traffic(config):
    """Per-launch HBM bytes of the dominant kernel from the committed PMC
    summary, if it was measured on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_sha") != source_sha(config):
        return None
    return d.get("hbm_bytes_per_launch")


def _leading_decodes(case):
    """Number of leading decode-class sequences (q_len * G <= 16) of a batch."""
    G = case.num_q_heads // case.num_kv_heads
    big = np.diff(case.cu_q_lens[:case.num_seqs + 1]) * G > 16
    return int(np.argmax(big)) if np.any(big) else case.num_seqs


def bench_gqa(args, torch, rpa, wl):
    case, fn = setup_gqa(torch, rpa, wl, args.config)
    work = gqa_work(case)
    subset = getattr(args, "decode_subset", "on")
    if args.config == "mixed_gqa" and subset == "only":
        fn.ns.fill_(_leading_decodes(case))
    (ms, kern_mean, kern_med, parts), cold = measure(args, torch, rpa, fn, split=True)
    step_s = ms / 1e3
    res = {"ms_per_step": ms, "attention_kernels_ms_mean": kern_mean,
           "attention_kernels_ms_median": kern_med, "q_tokens": work["q_tokens"],
           "tokens_per_s": work["q_tokens"] / step_s}
    res.update(parts)
    if cold is not None:
        res["cold"] = cold_summary(cold)
    traffic = load_traffic(args.config)
    if args.config == "decode_gqa" or args.config == "tiny_gqa":
        # Dominant kernel: the decode-tile kernel (a batch of decodes has no
        # prefill-class tiles; the prefill-tile kernel finds an empty list).
        kern_s = parts["decode_kernel_ms"] / 1e3
        res["kernel_ms_mean"] = parts["decode_kernel_ms"]
        gbs = work["kv_bytes"] / step_s / 1e9
        res.update(value=gbs, unit="GB/s", pct_hbm_peak=100 * gbs / HBM_PEAK_GBS)
        ach = work["kv_bytes"] / kern_s / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                           "algorithmic_bytes_per_launch": work["kv_bytes"],
                           "kernel": "gqa_tile_kernel"}
    elif subset == "only":
        # Profiling aid: the mixed batch's leading decode sequences alone.
        kern_s = parts["decode_kernel_ms"] / 1e3
        res["kernel_ms_mean"] = parts["decode_kernel_ms"]
        gbs = work["decode_kv_bytes"] / step_s / 1e9
        res.update(value=gbs, unit="GB/s", pct_hbm_peak=100 * gbs / HBM_PEAK_GBS,
                   decode_seqs=_leading_decodes(case))
        ach = work["decode_kv_bytes"] / kern_s / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": load_traffic("mixed_gqa_decode"),
                           "algorithmic_bytes_per_launch": work["decode_kv_bytes"],
                           "kernel": "gqa_decode8_kernel"}
    else:  # mixed: prefill TFLOP/s on the prefill-tile kernel, decode GB/s on the decode-tile kernel
        pre_s = parts["prefill_kernel_ms"] / 1e3
        res["kernel_ms_mean"] = parts["prefill_kernel_ms"]
        tf = work["flops"] / step_s / 1e12
        res.update(value=tf, unit="TFLOP/s", pct_mfma_peak=100 * tf / BF16_PEAK_TFLOPS,
                   kv_gbs=work["kv_bytes"] / step_s / 1e9)
        ach = work["prefill_flops"] / pre_s / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "traffic": traffic,
                           "algorithmic_flops_per_launch": work["prefill_flops"],
                           "kernel": "gqa_prefill_kernel"}
        # In the full batch the decode-tile launch runs on the library's side
        # stream next to the prefill kernel, so its event span includes waiting
        # for CUs; its rate is taken on the batch's decode subset (the leading
        # decode sequences alone, same kernel, same inputs).
        res["decode_kernel_span_in_batch_ms"] = res.pop("decode_kernel_ms")
        if subset == "on":
            n_dec = _leading_decodes(case)
            fn.ns.fill_(n_dec)
            (_, _, _, dparts), dcold = measure(args, torch, rpa, fn, split=True)
            fn.ns.fill_(case.num_seqs)
            dec_s = dparts["decode_kernel_ms"] / 1e3
            dgb = work["decode_kv_bytes"] / dec_s / 1e9
            res["decode_part"] = {"kernel": "gqa_decode8_kernel", "decode_seqs": n_dec,
                                  "kernel_ms": dparts["decode_kernel_ms"], "achieved_GBs": dgb,
                                  "frac_hbm": dgb / HBM_PEAK_GBS,
                                  "traffic": load_traffic("mixed_gqa_decode"),
                                  "algorithmic_bytes_per_launch": work["decode_kv_bytes"]}
            if dcold is not None:
                dc = dcold[3]["decode_kernel_ms"]
                res["decode_part"]["cold"] = {"kernel_ms": dc,
                                              "achieved_GBs": work["decode_kv_bytes"] / dc / 1e6}
        roof_s = max(work["flops"] / (BF16_PEAK_TFLOPS * 1e12),
                     work["kv_bytes"] / (HBM_PEAK_GBS * 1e9))
        res["combined_roof_us"] = roof_s * 1e6
        res["frac_of_combined_roof"] = roof_s / (kern_mean / 1e3)
    res["work"] = work
    if not args.no_cpu_baseline:
        cb = cpu_baseline_gqa(case, work, args.cpu_budget,
                              prefill_only=args.config == "mixed_gqa" and subset != "only")
        if res["unit"] == "GB/s":
            v, unit = cb["kv_bytes"] / cb["seconds"] / 1e9, "GB/s"
        else:
            v, unit = cb["flops"] / cb["seconds"] / 1e12, "TFLOP/s"
        res["cpu_baseline"] = {"value": v, "unit": unit, "cores": cb["cores"], "kind": "oracle",
                               "sample": cb["sample"], "seconds": cb["seconds"],
                               "tokens_per_s": cb["tokens"] / cb["seconds"]}
    cfg = {"decode_gqa": {"workload": "decode_gqa", "num_seqs": 128, "q_len": 1,
                          "kv_len": "U[512,8192]", "q_heads": 32, "kv_heads": 8, "head_dim": 128,
                          "page_size": 16, "kv_dtype": "bf16"},
           "mixed_gqa": {"workload": "mixed_gqa", "decodes": 120, "prefill_chunks": 8,
                         "q_heads": 32, "kv_heads": 8, "head_dim": 128, "page_size": 16,
                         "kv_dtype": "fp8_e4m3fn", "sliding_window": 4096, "soft_cap": 50},
           "tiny_gqa": {"workload": "tiny_gqa", "num_seqs": 3, "dtype": "fp32"}}[args.config]
    return res, cfg


def _budgeted(run, order, budget_s, probe_n=2):
    """Runs run(sample) on a probe, then on a sample sized for ~budget_s."""
    probe = np.sort(order[:max(1, min(len(order), probe_n))])
    dt = run(probe)
    n = int(min(len(order), max(len(probe), len(probe) * budget_s / max(dt, 1e-3))))
    sample = np.sort(order[:n])
    return sample, run(sample)


def bench_latent(args, torch, rpa, wl):
    import oracle
    dev = "cuda"
    if args.config == "mla_decode":
        case = wl.mla_decode(device=dev)
        kl = torch.from_numpy(case.kv_lens).to(dev)
        pi = torch.from_numpy(case.page_indices).to(dev)
        cu = torch.from_numpy(case.cu_q_lens).to(dev)
        ns = torch.tensor([case.num_seqs], dtype=torch.int32, device=dev)
        out = torch.empty_like(case.ql_nope)
        H = case.ql_nope.shape[1]
        need = rpa.mla_rpa_workspace_size(kl, pi, case.ql_nope.shape[0], H, 512)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def fn(update=True):
            rpa.mla_rpa_forward(case.ql_nope, case.q_pe, case.new_kv_c if update else None,
                                case.new_k_pe if update else None, case.cache_kv_c,
                                case.cache_k_pe, kl, pi, cu, ns, sm_scale=case.sm_scale, out=out,
                                workspace=ws)
        work = mla_work(case, H)
        (ms, kmean, kmed, kparts), cold = measure(args, torch, rpa, fn)
        ms_attn = timed_loop(torch, rpa, lambda: fn(False), args.steps, args.warmup)[0] \
            if getattr(args, "cache", "both") == "both" else None
        gbs = work["kv_bytes"] / (ms / 1e3) / 1e9
        ach = work["kv_bytes"] / (kmean / 1e3) / 1e9
        res = {"value": gbs, "unit": "GB/s", "ms_per_step": ms, "kernel_ms_mean": kmean,
               "kernel_ms_median": kmed, "kernel_ms_min": kparts["kernel_ms_min"],
               "ms_per_step_eager": kparts.get("ms_per_step_eager"),
               "cold": cold_summary(cold), "ms_per_step_attention_only": ms_attn,
               "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS,
               "tokens_per_s": work["q_tokens"] / (ms / 1e3),
               "mfma_tflops_in_kernel": work["flops"] / (kmean / 1e3) / 1e12,
               "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": ach / HBM_PEAK_GBS, "traffic": load_traffic(args.config),
                            "algorithmic_bytes_per_launch": work["kv_bytes"]},
               "work": work}
        if not args.no_cpu_baseline:
            ckv, _ = _storage(case.cache_kv_c)
            ckp, _ = _storage(case.cache_k_pe)
            ql, d = _storage(case.ql_nope)
            qp, _ = _storage(case.q_pe)

            def run(tokens):
                t0 = time.perf_counter()
                oracle.mla(ql, qp, d, ckv, ckp, case.kv_lens, case.page_indices, case.cu_q_lens,
                           case.num_seqs, sm_scale=case.sm_scale, tokens=tokens)
                return time.perf_counter() - t0
            order = np.random.default_rng(0).permutation(work["q_tokens"])
            toks, dt = _budgeted(run, order, args.cpu_budget, 1)
            kvb = int(sum(int(case.kv_lens[t]) for t in toks)) * 1152
            res["cpu_baseline"] = {"value": kvb / dt / 1e9, "unit": "GB/s",
                                   "cores": oracle.num_threads(), "kind": "oracle",
                                   "sample": f"{len(toks)} of {work['q_tokens']} decode tokens "
                                             "(all 128 heads), drawn with seed 0",
                                   "seconds": dt, "tokens_per_s": len(toks) / dt}
        cfg = {"workload": "mla_decode", "num_seqs": 64, "q_len": 1, "kv_len": "U[4096,32768]",
               "heads": 128, "kv_lora_rank": 512, "rope_dim": 64, "page_size": 64,
               "dtype": "bf16", "includes_kv_cache_update": True}
        return res, cfg
    # sparse_mla
    case = wl.sparse_mla(device=dev)
    pt = torch.from_numpy(case.page_table).to(dev)
    idx = torch.from_numpy(case.indices).to(dev)
    pos = torch.from_numpy(case.positions).to(dev)
    out = torch.empty((case.q.shape[0], case.q.shape[1], 512), dtype=torch.float32, device=dev)

    def fn():
        rpa.sparse_mla_forward(case.q, case.kv_cache, pt, idx, pos, seq_len=case.seq_len,
                               read_block=case.read_block, sm_scale=case.sm_scale, out=out)
    work = sparse_work(case)
    (ms, kmean, kmed, kparts), cold = measure(args, torch, rpa, fn)
    tf = work["flops"] / (ms / 1e3) / 1e12
    ach = work["flops"] / (kmean / 1e3) / 1e12
    res = {"value": tf, "unit": "TFLOP/s", "ms_per_step": ms, "kernel_ms_mean": kmean,
           "kernel_ms_median": kmed, "kernel_ms_min": kparts["kernel_ms_min"],
           "ms_per_step_eager": kparts.get("ms_per_step_eager"),
           "cold": cold_summary(cold),
           "pct_mfma_peak": 100 * tf / BF16_PEAK_TFLOPS,
           "gathered_gbs_in_kernel": work["gathered_bytes"] / (kmean / 1e3) / 1e9,
           "tokens_per_s": work["q_tokens"] / (ms / 1e3),
           "roofline": {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                        "traffic": load_traffic(args.config),
                        "algorithmic_flops_per_launch": work["flops"]},
           "work": work}
    if not args.no_cpu_baseline:
        q, d = _storage(case.q)
        kv, _ = _storage(case.kv_cache)

        def run(qs):
            t0 = time.perf_counter()
            oracle.sparse_mla(q, d, kv, case.page_table, case.indices, case.positions,
                              seq_len=case.seq_len, read_block=case.read_block,
                              sm_scale=case.sm_scale, queries=qs)
            return time.perf_counter() - t0
        order = np.random.default_rng(0).permutation(q.shape[0])
        qs, dt = _budgeted(run, order, args.cpu_budget, 2)
        flops = work["flops"] * len(qs) / q.shape[0]
        res["cpu_baseline"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"{len(qs)} of {q.shape[0]} queries (all 16 heads), "
                                         "drawn with seed 0; flops scaled by the sample share",
                               "seconds": dt, "tokens_per_s": len(qs) / dt}
    cfg = {"workload": "sparse_mla", "seq_tokens": 65536, "queries": 4096, "heads": 16,
           "top_k_units": 32, "read_block": 64, "page_size": 64, "dtype": "bf16"}
    return res, cfg


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode_gqa",
                    choices=["decode_gqa", "mixed_gqa", "tiny_gqa", "mla_decode", "sparse_mla"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cache", choices=("both", "warm", "cold"), default="both",
                    help="both: the warm timed region (value, roofline) plus a cold pass (a "
                         "512 MB read evicts L2 and MALL before each step); warm / cold: only "
                         "that loop (warm for profiling runs)")
    ap.add_argument("--decode-subset", choices=("on", "off", "only"), default="on",
                    help="mixed_gqa: also time the batch's decode subset alone (on), skip it "
                         "(off), or time only the subset (only; for profiling that kernel)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="target seconds of oracle CPU work for cpu_baseline")
    ap.add_argument("--extras", choices=("on", "off"), default="on",
                    help="decode_gqa only: also measure the other full-size workloads (the mixed "
                         "batch's prefill kernel and decode subset, MLA decode, sparse MLA) and "
                         "attach each, with its own roofline and cpu_baseline, to the line "
                         "(off for profiling runs of the decode kernel alone)")
    ap.add_argument("--extras-cpu-budget", type=float, default=8.0,
                    help="target seconds of oracle CPU work for each extra workload")
    ap.add_argument("--graph", choices=("on", "off"), default="on",
                    help="time the steps as replays of a captured HIP graph of the call (on), "
                         "or as eager calls (off); the eager time is reported either way")
    ap.add_argument("--probe", action="store_true",
                    help="instead of the benchmark, run the ceiling probes (LDS-DMA streaming "
                         "read, MFMA / LDS / exp issue rates, MFMA chain clocks per step) and "
                         "print one JSON line per measurement")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many bytes "
                         "(calibration run for the PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU part: tiles are independent, so each GPU would run its own sequences or kv heads)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import ragged_paged_attention_rpa_amd as rpa
    from ragged_paged_attention_rpa_amd import workloads as wl
    rpa.load_library()
    if args.probe:
        from ragged_paged_attention_rpa_amd import probes
        for row in probes.run_all(torch):
            print(json.dumps(row), flush=True)
        return
    if args.copy_bytes:
        n = args.copy_bytes // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4}))
        return
    res, cfg = run_config(args, torch, rpa, wl)
    line = {"metric": METRIC, "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"),
            "step_timing": "hip_graph_replay" if args.graph == "on" else "eager_calls",
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if args.config != "tiny_gqa" else "f32", "data": "synthetic",
            "config": cfg}
    line.update(res)
    if args.config == "decode_gqa" and args.extras == "on":
        # The metric's other half and the other full-size workloads, each timed
        # the same way (warm timed region + cold pass) on its own dominant
        # kernel: "prefill" is the mixed batch (prefill kernel TFLOP/s, with its
        # decode subset's GB/s under decode_part).
        for key, config in (("prefill", "mixed_gqa"), ("mla_decode", "mla_decode"),
                            ("sparse_mla", "sparse_mla")):
            sub = argparse.Namespace(**vars(args))
            sub.config = config
            sub.cpu_budget = args.extras_cpu_budget
            print(f"[bench] {config}", file=sys.stderr, flush=True)
            r, c = run_config(sub, torch, rpa, wl)
            r["config"] = c
            line[key] = r
            torch.cuda.empty_cache()
    print(json.dumps(line))


def run_config(args, torch, rpa, wl):
    if args.config in ("decode_gqa", "mixed_gqa", "tiny_gqa"):
        return bench_gqa(args, torch, rpa, wl)
    return bench_latent(args, torch, rpa, wl)


if __name__ == "__main__":
    main()
