"""Practical ceilings of one MI355X, measured with the probes of librpa.so
(include/rpa_probe.h): HBM read bandwidth through the attention kernels' own
LDS-DMA scheme (default and non-temporal cache policy), MFMA / LDS / exp issue rates per CU, clocks per step of a
dependent MFMA chain next to softmax-like VALU and LDS work, and the clocks a
wave spends issuing 1 KB reads.

Each function returns a dict ready for JSON; `python bench.py --probe` prints
them. Rates per CU per clock are given at the nominal 2.4 GHz (wall-clock
timing), the chain probe in shader clocks counted by the kernel itself.
"""
from __future__ import annotations

import ctypes

NOMINAL_GHZ = 2.4
THREADS = 256
CHAIN_STEPS = 256 * 36
RATE_PER_WG = {0: (536870912.0, "flop"), 1: (16777216.0, "byte"), 2: (16384.0, "wave_instr"),
               3: (16384.0, "wave_instr")}
RATE_NAMES = {0: "mfma_32x32x16_bf16", 1: "ds_read_b128", 2: "v_exp_f32", 3: "v_fma_f32"}
CHAIN_NAMES = {0: "mfma chain, accumulator in VGPRs", 2: "+ 4 VALU per step",
               4: "+ 1 LDS operand read per step", 6: "+ 4 VALU + 1 LDS read per step",
               8: "mfma chain, accumulator in AGPRs", 10: "AGPR + 4 VALU per step",
               12: "AGPR + 1 LDS read per step", 14: "AGPR + 4 VALU + 1 LDS read per step"}


def _lib():
    import ragged_paged_attention_rpa_amd as rpa
    lib = rpa.load_library()
    if not getattr(lib, "_probe_sigs", False):
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.rpa_probe_stream.argtypes = [P, SZ, I32, I32, P]
        lib.rpa_probe_stream.restype = I32
        lib.rpa_probe_rate.argtypes = [I32, I32, P, P]
        lib.rpa_probe_rate.restype = I32
        lib.rpa_probe_chain.argtypes = [I32, I32, P, P, P]
        lib.rpa_probe_chain.restype = I32
        lib.rpa_probe_issue.argtypes = [I32, I32, I32, I32, P, SZ, P, P, P]
        lib.rpa_probe_issue.restype = I32
        lib._probe_sigs = True
    return lib


def _check(status, what):
    if status != 0:
        raise RuntimeError(f"{what} returned status {status}")


def _timed(torch, launch, reps):
    """Milliseconds per launch: `reps` launches between two events on the
    current stream, after two untimed ones."""
    for _ in range(2):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def stream(torch, nbytes=4 << 30, wg_per_cu=2, interleave=True, nontemporal=False, regs=False,
           reps=10):
    """GB/s of a single read of `nbytes` with the LDS-DMA scheme, or with plain
    loads into registers (regs), with the default or the non-temporal cache
    policy."""
    lib = _lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus * wg_per_cu
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    stage = 32 * 1024
    read = (nbytes // stage) // grid * grid * stage
    flags = int(interleave) | (2 if nontemporal else 0) | (4 if regs else 0)
    ms = _timed(torch, lambda: _check(lib.rpa_probe_stream(buf.data_ptr(), nbytes, grid, flags,
                                                           st),
                                      "rpa_probe_stream"), reps)
    del buf
    return {"probe": ("stream_regs" if regs else "stream_lds_dma") + ("_nt" if nontemporal else ""),
            "bytes": read, "workgroups": grid,
            "chunks": "interleaved" if interleave else "contiguous per workgroup",
            "stages": "8 KB per wave in registers" if regs else "2 x 32 KB per workgroup",
            "ms": round(ms, 4),
            "GB_per_s": round(read / (ms * 1e-3) / 1e9, 1),
            "frac_of_8TBps": round(read / (ms * 1e-3) / 8e12, 3)}


def rate(torch, kind, waves_per_simd=1, reps=5):
    """Issue rate of one instruction kind, per CU per clock at 2.4 GHz."""
    lib = _lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus * waves_per_simd
    sink = torch.empty(grid * THREADS, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    ms = _timed(torch, lambda: _check(lib.rpa_probe_rate(kind, grid, sink.data_ptr(), st),
                                      "rpa_probe_rate"), reps)
    per_wg, unit = RATE_PER_WG[kind]
    total = per_wg * grid
    out = {"probe": RATE_NAMES[kind], "waves_per_simd": waves_per_simd, "ms": round(ms, 4),
           f"{unit}_per_cu_per_clk": round(total / cus / (ms * 1e-3 * NOMINAL_GHZ * 1e9), 2)}
    if kind == 0:
        out["TFLOP_per_s"] = round(total / (ms * 1e-3) / 1e12, 1)
        out["frac_of_2.5PF"] = round(total / (ms * 1e-3) / 2.5e15, 3)
    return out


def chain(torch, mode):
    """Shader clocks per MFMA step (mean over one workgroup per CU)."""
    lib = _lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cycles = torch.zeros(cus, dtype=torch.int64, device="cuda")
    sink = torch.empty(cus * THREADS, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        _check(lib.rpa_probe_chain(mode, cus, cycles.data_ptr(), sink.data_ptr(), st),
               "rpa_probe_chain")
    torch.cuda.synchronize()
    per_step = cycles.double().mean().item() / CHAIN_STEPS
    return {"probe": "mfma_chain", "mode": mode, "what": CHAIN_NAMES[mode],
            "clocks_per_step": round(per_step, 1)}


ISSUE_NAMES = {0: "global_load_lds_dwordx4", 1: "global_load_dwordx4"}


def issue(torch, kind, waves, count=16, src_bytes=64 << 20):
    """Shader clocks a wave spends issuing `count` 1 KB reads back to back
    (median over one workgroup per CU of `waves` waves), and until they land."""
    lib = _lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = cus * waves
    src = torch.ones(src_bytes // 4, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    sink = torch.empty(n * 64, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        _check(lib.rpa_probe_issue(kind, waves, count, cus, src.data_ptr(), src_bytes,
                                   ticks.data_ptr(), sink.data_ptr(), st), "rpa_probe_issue")
    torch.cuda.synchronize()
    t = ticks.view(n, 2).double()
    iss, tot = t[:, 0].median().item(), t[:, 1].median().item()
    return {"probe": "issue_" + ISSUE_NAMES[kind], "waves_per_cu": waves, "reads_per_wave": count,
            "clocks_to_issue": round(iss), "clocks_per_read": round(iss / count, 1),
            "clocks_to_land": round(tot)}


def run_all(torch):
    rows = [stream(torch, wg_per_cu=w, interleave=il, nontemporal=nt)
            for nt in (False, True) for il in (True, False) for w in (2, 1)]
    rows += [stream(torch, wg_per_cu=w, regs=True, nontemporal=nt)
             for nt in (False, True) for w in (2, 1)]
    for kind in (0, 1, 2, 3):
        for w in (1, 2):
            rows.append(rate(torch, kind, w))
    for mode in sorted(CHAIN_NAMES):
        rows.append(chain(torch, mode))
    for kind in (0, 1):
        for w in (1, 4, 8):
            rows.append(issue(torch, kind, w))
    return rows
