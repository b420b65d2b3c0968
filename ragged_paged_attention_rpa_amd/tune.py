"""Sweep of the shape-keyed tile sizes on the GPU (the measurements behind the
rows of csrc/tile_table.cpp).

For each batch below it times the whole call (planner, tile kernels, merge)
for every candidate ``split_keys`` — rpa_forward's keys per decode split, or
mla_rpa_forward's smallest share — with HIP events over repeated calls, and
prints the per-candidate times and the fastest value. Rows of the table are
written by hand from this output; the table's comment names this command.

Usage: python -m ragged_paged_attention_rpa_amd.tune [--reps N] [--only NAME]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def _time_candidates(torch, fns, reps):
    """Median milliseconds per call of each candidate. The candidates take
    turns call by call, so clock ramps and thermal drift fall on all alike."""
    for fn in fns.values():
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    times = {k: [] for k in fns}
    for _ in range(reps):
        for k, fn in fns.items():
            start.record()
            fn()
            stop.record()
            stop.synchronize()
            times[k].append(start.elapsed_time(stop))
    return {k: round(float(np.median(v)), 4) for k, v in times.items()}


def _gqa_batches(torch, wl):
    rng = np.random.default_rng(7)
    bf16, fp8 = torch.bfloat16, torch.float8_e4m3fn

    def dec(name, n, lo, hi, hq, hkv, kv_dtype, ps, pps):
        seqs = [(1, int(x)) for x in rng.integers(lo, hi + 1, n)]
        return name, dict(seqs=seqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                          page_size=ps, q_dtype=bf16, kv_dtype=kv_dtype, pages_per_seq=pps)

    return [
        dec("decode 128 x 512..8192, 32/8, bf16, page 16", 128, 512, 8192, 32, 8, bf16, 16, 512),
        dec("decode 128 x 512..8192, 32/8, fp8, page 16", 128, 512, 8192, 32, 8, fp8, 16, 512),
        dec("decode 8 x 16k..32k, 32/8, bf16, page 16", 8, 16384, 32768, 32, 8, bf16, 16, 2048),
        dec("decode 8 x 16k..32k, 32/8, fp8, page 16", 8, 16384, 32768, 32, 8, fp8, 16, 2048),
        dec("decode 32 x 2k..16k, 8/1, bf16, page 64", 32, 2048, 16384, 8, 1, bf16, 64, 256),
        dec("decode 16 x 16k..64k, 16/2, fp8, page 64", 16, 16384, 65536, 16, 2, fp8, 64, 1024),
        dec("decode 256 x 128..2048, 32/8, bf16, page 16", 256, 128, 2048, 32, 8, bf16, 16, 128),
    ]


def _mla_batches(rng):
    return [
        ("mla 64 x 4096..32768, 128 heads", [(1, int(x)) for x in rng.integers(4096, 32769, 64)]),
        ("mla 8 x 1024..4096, 128 heads", [(1, int(x)) for x in rng.integers(1024, 4097, 8)]),
        ("mla 2 x 2048, 128 heads", [(1, 2048), (1, 2048)]),
        ("mla 4 x 512 (q 4), 128 heads", [(4, 512)] * 4),
    ]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=30)
    ap.add_argument("--only", default="", help="substring of the batch names to run")
    args = ap.parse_args(argv)
    import torch
    import ragged_paged_attention_rpa_amd as rpa
    from ragged_paged_attention_rpa_amd import workloads as wl
    rpa.load_library()
    d = "cuda"
    results = []

    for name, kw in _gqa_batches(torch, wl):
        if args.only not in name:
            continue
        c = wl.make_gqa(kw.pop("seqs"), seed=11, device=d, spare_pages=0, name=name, **kw)
        kl, pi = torch.from_numpy(c.kv_lens).to(d), torch.from_numpy(c.page_indices).to(d)
        cu = torch.from_numpy(c.cu_q_lens).to(d)
        ns = torch.tensor([c.num_seqs], dtype=torch.int32, device=d)
        out = torch.empty_like(c.q)
        ws = torch.empty(max(1, rpa.rpa_workspace_size(kl, pi, c.q.shape[0], c.q.shape[1],
                                                       c.kv_pages.shape[2] // 2, 128)),
                         dtype=torch.uint8, device=d)
        row = {"batch": name, "path": "rpa_forward decode split"}
        fns = {}
        for sk in (256, 512, 1024, 2048, 4096):
            def fn(sk=sk):
                rpa.rpa_forward(c.q, c.kv_pages, kl, pi, cu, ns, sm_scale=c.sm_scale, out=out,
                                workspace=ws, split_keys=sk)
            fns[sk] = fn
        row["ms"] = _time_candidates(torch, fns, args.reps)
        row["table"] = rpa.tile_config(rpa.TILE_DECODE_SPLIT, c.kv_pages.dtype, c.q.shape[1],
                                       c.kv_pages.shape[2] // 2, 128, c.kv_pages.shape[1],
                                       c.page_indices.shape[1])[0]
        row["best"] = min(row["ms"], key=row["ms"].get)
        print(json.dumps(row), flush=True)
        results.append(row)
        del c, out, ws
        torch.cuda.empty_cache()

    rng = np.random.default_rng(8)
    for name, seqs in _mla_batches(rng):
        if args.only not in name:
            continue
        c = wl.make_mla(seqs, num_heads=128, page_size=64, seed=12, device=d, name=name)
        kl, pi = torch.from_numpy(c.kv_lens).to(d), torch.from_numpy(c.page_indices).to(d)
        cu = torch.from_numpy(c.cu_q_lens).to(d)
        ns = torch.tensor([c.num_seqs], dtype=torch.int32, device=d)
        out = torch.empty_like(c.ql_nope)
        ws = torch.empty(max(1, rpa.mla_rpa_workspace_size(kl, pi, c.ql_nope.shape[0], 128, 512)),
                         dtype=torch.uint8, device=d)
        row = {"batch": name, "path": "mla_rpa_forward smallest share"}
        fns = {}
        for sk in (64, 128, 256, 512, 1024):
            def fn(sk=sk):
                rpa.mla_rpa_forward(c.ql_nope, c.q_pe, None, None, c.cache_kv_c, c.cache_k_pe, kl,
                                    pi, cu, ns, sm_scale=c.sm_scale, out=out, workspace=ws,
                                    split_keys=sk)
            fns[sk] = fn
        row["ms"] = _time_candidates(torch, fns, args.reps)
        row["table"] = rpa.tile_config(rpa.TILE_MLA_SHARE, torch.bfloat16, 128, 1, 576, 64,
                                       c.page_indices.shape[1])[0]
        row["best"] = min(row["ms"], key=row["ms"].get)
        print(json.dumps(row), flush=True)
        results.append(row)
        del c, out, ws
        torch.cuda.empty_cache()
    return results


if __name__ == "__main__":
    main(sys.argv[1:])
