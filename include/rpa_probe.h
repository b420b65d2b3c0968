/*
 * rpa_probe.h — measurement probes exported by librpa.so beside the attention
 * operations (rpa.h). They are not part of the attention path: they measure
 * the practical ceilings the attention kernels are compared with
 * (`python bench.py --probe` runs and reports them).
 *
 *   rpa_probe_stream  HBM read bandwidth with the attention kernels' own
 *                     LDS-DMA scheme (global_load_lds_dwordx4, 1 KB per
 *                     instruction, two 32 KB stages per workgroup, no compute);
 *   rpa_probe_rate    issue throughput of one instruction kind per CU:
 *                     32x32x16 bf16 MFMA, ds_read_b128, v_exp_f32, v_fma_f32;
 *   rpa_probe_chain   shader clocks (s_memtime) per step of a dependent chain
 *                     of 36 32x32x16 bf16 MFMAs per loop trip, alone or next
 *                     to the VALU and LDS work a softmax step adds;
 *   rpa_probe_issue   shader clocks a wave spends issuing 1 KB reads (LDS-DMA
 *                     or into registers) back to back, and until they land.
 *
 * Buffers are DEVICE memory owned by the caller; calls are asynchronous on
 * `stream` (NULL = the default stream); launches use 256-thread workgroups
 * (rpa_probe_issue: 64 * waves). Return values are rpa_status codes (rpa.h): RPA_E_INVALID for a
 * value out of range, RPA_E_HIP when the launch fails; nothing is launched
 * on an invalid argument.
 */
#ifndef RPA_PROBE_H_
#define RPA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "rpa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streams the first floor(bytes / 32 KiB / workgroups) * workgroups chunks of
 * 32 KiB of `buf` once. flags bit 0 set: workgroup b reads chunks b,
 * b + workgroups, b + 2 workgroups, ...; clear: workgroup b reads its own
 * contiguous run of chunks. flags bit 1: the loads carry the non-temporal
 * cache policy (nt). flags bit 2: plain loads into registers (one 8 KiB
 * chunk share in flight per wave) instead of LDS-DMA. Nothing is written to
 * global memory. workgroups in [1, 65536]; flags in [0, 7]; `bytes` must hold
 * at least one chunk per workgroup. Time the launch with events to get bytes
 * per second.
 */
int rpa_probe_stream(const void* buf, size_t bytes, int workgroups, int flags,
                     rpa_stream_t stream);

/*
 * kind 0: four independent 32x32x16 bf16 MFMA chains per wave, 4096 MFMAs per
 *         wave (536,870,912 flop per workgroup);
 * kind 1: ds_read_b128 over a 64 KiB LDS array, 4096 reads per wave
 *         (16 MiB read per workgroup);
 * kind 2: v_exp_f32 in eight independent chains, 4096 per wave
 *         (16,384 wave-instructions per workgroup);
 * kind 3: v_fma_f32 likewise (16,384 wave-instructions per workgroup).
 * `sink` receives workgroups * 256 floats (values meaningless; they keep the
 * work live). workgroups in [1, 65536].
 */
int rpa_probe_rate(int kind, int workgroups, float* sink, rpa_stream_t stream);

/*
 * One dependent chain of 32x32x16 bf16 MFMAs per wave, 256 trips of 36 steps
 * (9,216 steps); `cycles[b]` receives workgroup b's s_memtime delta over the
 * loop (divide by 9,216 for clocks per step). mode bits: 2 = four independent
 * VALU instructions per step (fma, mul, exp, max); 4 = one ds_read_b128
 * operand per step, issued four steps ahead; 8 = accumulator held in AGPRs
 * (else VGPRs). mode in {0, 2, 4, 6, 8, 10, 12, 14}; `sink` receives
 * workgroups * 256 floats; workgroups in [1, 65536] (one per CU gives one
 * wave per SIMD).
 */
int rpa_probe_chain(int mode, int workgroups, unsigned long long* cycles, float* sink,
                    rpa_stream_t stream);

/*
 * Each of `waves` waves per workgroup (1..8) issues `count` (4 or 16) reads of
 * 1 KiB (64 lanes x 16 bytes) back to back: kind 0 global_load_lds_dwordx4
 * into LDS (the attention kernels' staging), kind 1 global_load_dwordx4 into
 * registers. Wave g = workgroup * waves + w reads the count KiB at
 * (g * count KiB) mod span of `src`, span = src_bytes rounded down to a
 * multiple of count KiB (src_bytes >= count KiB). ticks[2g] receives the
 * s_memtime clocks spent issuing the reads, ticks[2g + 1] the clocks until
 * they have landed; ticks holds 2 * workgroups * waves entries, `sink`
 * workgroups * waves * 64 floats (values meaningless). workgroups in
 * [1, 65536].
 */
int rpa_probe_issue(int kind, int waves, int count, int workgroups, const void* src,
                    size_t src_bytes, unsigned long long* ticks, float* sink,
                    rpa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RPA_PROBE_H_ */
