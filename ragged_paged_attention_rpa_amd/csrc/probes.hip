// Measurement probes behind the practical ceilings the kernels are compared
// with (bench.py --probe): a streaming read with the attention kernels' own
// LDS-DMA scheme, MFMA chains next to VALU and LDS work (cycles per step),
// raw MFMA / LDS / transcendental throughput, and the clocks a wave spends
// issuing 1 KB reads. Not part of the attention
// path; every access stays inside the buffers and LDS arrays below.
#include "rpa_probe.h"

#include <hip/hip_runtime.h>

#include "rpa_device.h"

namespace rpa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kStreamStage = 32 * 1024;  // bytes per stage: 8 DMA instructions per wave

// Streams `nchunks` 32 KB chunks of `buf` through two alternating 32 KB LDS
// stages per workgroup with global_load_lds_dwordx4 (1 KB per instruction),
// keeping two stages in flight per wave, and computes nothing. Workgroup b
// takes chunks b, b + grid, b + 2 grid, ... (INTERLEAVE) or its own
// contiguous run of nchunks / grid chunks. nt: loads with the non-temporal
// cache policy. REGS: plain global_load_dwordx4 into registers instead of
// LDS-DMA (one chunk in flight per wave, folded by XOR and kept live).
template <bool INTERLEAVE, bool REGS, bool REGS_NT>
__global__ void __launch_bounds__(kProbeThreads) probe_stream_kernel(const char* buf,
                                                                     int64_t nchunks, int nt) {
  __shared__ __attribute__((aligned(1024))) char stage[REGS ? 1 : 2][kStreamStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t per_wg = nchunks / gridDim.x;
  const int64_t first = INTERLEAVE ? blockIdx.x : blockIdx.x * per_wg;
  const int64_t step = INTERLEAVE ? gridDim.x : 1;
  if constexpr (REGS) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = 0; i < per_wg; ++i) {
      const char* src = buf + (first + i * step) * kStreamStage + wave * 8192 + lane * 16;
      u32x4 r[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x4* p = reinterpret_cast<const u32x4*>(src + k * 1024);
        // (A compile-time choice: a run-time one lets the compiler merge the
        // two loads and drop the hint.)
        if constexpr (REGS_NT)
          r[k] = __builtin_nontemporal_load(p);
        else
          r[k] = *p;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= r[k];
    }
    asm volatile("" : : "v"(acc));
    return;
  }
  for (int64_t i = 0; i < per_wg; ++i) {
    const uint32_t dst = lds_addr(stage[i & 1]) + (uint32_t)wave * 8192;
    const char* src = buf + (first + i * step) * kStreamStage + wave * 8192 + lane * 16;
#pragma unroll
    for (int k = 0; k < 8; ++k) dma_b128(src + k * 1024, dst + (uint32_t)k * 1024, nt != 0);
    wait_vmcnt<8>();
  }
  wait_vmcnt<0>();
}

__device__ __forceinline__ floatx16 mfma_v(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ void mfma_a(floatx16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <typename T>
__device__ __forceinline__ void keep(T& x) {
  asm volatile("" : "+v"(x));
}

// Cycles (s_memtime) per step of a 36-MFMA loop like the MLA kernel's score
// loop. MODE bit 1: four independent VALU instructions per step (fma, mul,
// exp, max); bit 2: one ds_read_b128 operand per step, four steps ahead;
// bit 3: accumulator in AGPRs (asm MFMA) instead of VGPRs.
constexpr int kChainIters = 256;
template <int MODE>
__global__ void __launch_bounds__(kProbeThreads, 1) probe_chain_kernel(unsigned long long* cycles,
                                                                       float* sink) {
  __shared__ __attribute__((aligned(16))) char lds[36864];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 36864 / 4; i += kProbeThreads)
    reinterpret_cast<float*>(lds)[i] = 0.0001f * (i & 255);
  __syncthreads();
  const uint32_t sb = lds_addr(lds) + (uint32_t)(lane * 16);  // reads stay below 36 KB
  u32x4 qv[36];
  for (int i = 0; i < 36; ++i) qv[i] = u32x4{(uint32_t)lane * 7u + i, 1u, 2u, 3u};
  float f[16];
  for (int i = 0; i < 16; ++i) f[i] = 0.5f + 0.01f * (lane + i);
  floatx16 s0 = {};
  if (MODE & 8) asm volatile("" : "=a"(s0) : "0"(s0));
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kChainIters; ++it) {
    u32x4 kr[4];
    if (MODE & 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = lds_read_b128(sb + (uint32_t)(i * 1024));
    }
#pragma unroll
    for (int st = 0; st < 36; ++st) {
      u32x4 kf;
      if (MODE & 4) {
        kf = kr[st % 4];
        pin_after(kf);
        if (st + 4 < 36) kr[st % 4] = lds_read_b128(sb + (uint32_t)(((st + 4) % 36) * 1024));
      } else {
        kf = qv[(st + 1) % 36];
      }
      if (MODE & 8)
        mfma_a(s0, kf, qv[st]);
      else
        s0 = mfma_v(kf, qv[st], s0);
      if (MODE & 2) {
        const int r = st & 15;
        f[r] = __builtin_fmaf(f[r], 0.999f, 0.001f);
        keep(f[r]);
        const int r2 = (st + 5) & 15;
        f[r2] = f[r2] * 1.0001f;
        keep(f[r2]);
        const int r3 = (st + 9) & 15;
        f[r3] = __builtin_amdgcn_exp2f(-f[r3] * 0.01f);
        keep(f[r3]);
        const int r4 = (st + 13) & 15;
        f[r4] = fmaxf(f[r4], 0.3f);
        keep(f[r4]);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (MODE & 8) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float acc = 0.f;
  for (int i = 0; i < 16; ++i) acc += s0[i] + f[i];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

// Throughput loops, timed by the caller: KIND 0 four independent MFMA chains
// per wave; 1 ds_read_b128 streams over a 64 KB LDS array; 2 v_exp_f32;
// 3 v_fma_f32 (eight independent chains per lane in both VALU kinds).
constexpr int kRateIters = 4096;
template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) probe_rate_kernel(float* sink) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float out = 0.f;
  if (KIND == 0) {
    const u32x4 a = {(uint32_t)lane, 1u, 2u, 3u}, b = {(uint32_t)lane * 3u, 5u, 6u, 7u};
    floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < kRateIters / 4; ++it) {
      c0 = mfma_v(a, b, c0);
      c1 = mfma_v(b, a, c1);
      c2 = mfma_v(a, a, c2);
      c3 = mfma_v(b, b, c3);
    }
    for (int i = 0; i < 16; ++i) out += c0[i] + c1[i] + c2[i] + c3[i];
  } else if (KIND == 1) {
    for (int i = threadIdx.x; i < 65536 / 4; i += kProbeThreads)
      reinterpret_cast<float*>(lds)[i] = (float)i;
    __syncthreads();
    const uint32_t a = lds_addr(lds) + (uint32_t)(wave * 16384 + lane * 16);  // < 57 KB
    u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = r0, r2 = r0, r3 = r0;
    for (int it = 0; it < kRateIters / 8; ++it) {
      asm volatile(
          "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
          "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
          "ds_read_b128 %0, %4 offset:4096\n\tds_read_b128 %1, %4 offset:5120\n\t"
          "ds_read_b128 %2, %4 offset:6144\n\tds_read_b128 %3, %4 offset:7168\n\t"
          "s_waitcnt lgkmcnt(4)"
          : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3)
          : "v"(a)
          : "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const u32x4 x = r0 ^ r1 ^ r2 ^ r3;
    out = (float)(x[0] ^ x[1] ^ x[2] ^ x[3]);
  } else {
    float v[8];
    for (int i = 0; i < 8; ++i) v[i] = 0.01f * (threadIdx.x + i);
    for (int it = 0; it < kRateIters / 8; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = KIND == 2 ? __builtin_amdgcn_exp2f(-v[i]) : __builtin_fmaf(v[i], 0.999f, 0.001f);
    }
    for (int i = 0; i < 8; ++i) out += v[i];
  }
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = out;
}

// Issue cost of 1 KB vector-memory reads: each wave issues COUNT of them
// back to back (KIND 0: global_load_lds_dwordx4 into its own 8 KB of LDS;
// KIND 1: global_load_dwordx4 into registers) from its own COUNT KB of `src`
// (wave g of the grid reads at (g * COUNT KB) mod span, span a multiple of
// COUNT KB no larger than the buffer). ticks[2g] = s_memtime clocks spent
// issuing them, ticks[2g + 1] = until the data has landed.
constexpr int kIssueMaxWaves = 8;
template <int KIND, int COUNT>
__global__ void __launch_bounds__(64 * kIssueMaxWaves) probe_issue_kernel(
    const char* src, size_t span, unsigned long long* ticks, float* sink) {
  __shared__ __attribute__((aligned(1024))) char stage[kIssueMaxWaves][8192];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t g = (size_t)blockIdx.x * (blockDim.x >> 6) + wave;
  const char* base = src + (g * (size_t)COUNT * 1024) % span + lane * 16;
  const uint32_t dst = lds_addr(stage[wave]);
  u32x4 r[KIND == 1 ? COUNT : 1];
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < COUNT; ++k) {
    if constexpr (KIND == 0) {
      dma_b128(base + k * 1024, dst + (uint32_t)(k & 7) * 1024);
    } else {
      u32x4 v;
      asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(base + k * 1024) : "memory");
      r[k] = v;
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const unsigned long long t2 = __builtin_amdgcn_s_memtime();
  uint32_t x = 0;
  if constexpr (KIND == 1) {
#pragma unroll
    for (int k = 0; k < COUNT; ++k) x ^= r[k][0] ^ r[k][3];
  } else {
    x = *reinterpret_cast<const uint32_t*>(stage[wave] + lane * 16);
  }
  sink[g * 64 + lane] = (float)x;
  if (lane == 0) {
    ticks[2 * g] = t1 - t0;
    ticks[2 * g + 1] = t2 - t0;
  }
}

}  // namespace

hipError_t probe_issue(int kind, int waves, int count, int grid, const void* src, size_t bytes,
                       unsigned long long* ticks, float* sink, hipStream_t stream) {
  // Every wave reads count KB at a multiple of count KB below span <= bytes.
  const size_t chunk = (size_t)count * 1024;
  const size_t span = bytes / chunk * chunk;
  if (span == 0) return hipErrorInvalidValue;
  const char* s = (const char*)src;
#define RPA_PROBE_ISSUE(K, C)                                                                     \
  if (kind == K && count == C) {                                                                  \
    hipLaunchKernelGGL((probe_issue_kernel<K, C>), dim3(grid), dim3(64 * waves), 0, stream, s, \
                       span, ticks, sink);                                                        \
    return hipGetLastError();                                                                     \
  }
  RPA_PROBE_ISSUE(0, 4)
  RPA_PROBE_ISSUE(0, 16)
  RPA_PROBE_ISSUE(1, 4)
  RPA_PROBE_ISSUE(1, 16)
#undef RPA_PROBE_ISSUE
  return hipErrorInvalidValue;
}

hipError_t probe_stream(const void* buf, size_t bytes, int grid, int flags,
                        hipStream_t stream) {
  const bool interleave = flags & 1;
  const int nt = (flags >> 1) & 1;
  const bool regs = flags & 4;
  // Chunks read: per_wg = floor(bytes / 32 KB / grid) per workgroup, so every
  // chunk index, interleaved or contiguous, is below per_wg * grid.
  const int64_t nchunks = (int64_t)(bytes / kStreamStage) / grid * grid;
  if (nchunks <= 0) return hipErrorInvalidValue;
#define RPA_PROBE_STREAM(IL, RG, RNT)                                                   \
  hipLaunchKernelGGL((probe_stream_kernel<IL, RG, RNT>), dim3(grid), dim3(kProbeThreads), 0, \
                     stream, (const char*)buf, nchunks, nt)
  if (regs) {
    if (interleave && nt)
      RPA_PROBE_STREAM(true, true, true);
    else if (interleave)
      RPA_PROBE_STREAM(true, true, false);
    else if (nt)
      RPA_PROBE_STREAM(false, true, true);
    else
      RPA_PROBE_STREAM(false, true, false);
  } else if (interleave) {
    RPA_PROBE_STREAM(true, false, false);
  } else {
    RPA_PROBE_STREAM(false, false, false);
  }
#undef RPA_PROBE_STREAM
  return hipGetLastError();
}

hipError_t probe_chain(int mode, int grid, unsigned long long* cycles, float* sink,
                       hipStream_t stream) {
#define RPA_PROBE_CHAIN(M)                                                                   \
  case M:                                                                                    \
    hipLaunchKernelGGL(probe_chain_kernel<M>, dim3(grid), dim3(kProbeThreads), 0, stream, \
                       cycles, sink);                                                        \
    break;
  switch (mode) {
    RPA_PROBE_CHAIN(0)
    RPA_PROBE_CHAIN(2)
    RPA_PROBE_CHAIN(4)
    RPA_PROBE_CHAIN(6)
    RPA_PROBE_CHAIN(8)
    RPA_PROBE_CHAIN(10)
    RPA_PROBE_CHAIN(12)
    RPA_PROBE_CHAIN(14)
    default:
      return hipErrorInvalidValue;
  }
#undef RPA_PROBE_CHAIN
  return hipGetLastError();
}

hipError_t probe_rate(int kind, int grid, float* sink, hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(probe_rate_kernel<0>, dim3(grid), dim3(kProbeThreads), 0, stream, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_rate_kernel<1>, dim3(grid), dim3(kProbeThreads), 0, stream, sink);
  else if (kind == 2)
    hipLaunchKernelGGL(probe_rate_kernel<2>, dim3(grid), dim3(kProbeThreads), 0, stream, sink);
  else if (kind == 3)
    hipLaunchKernelGGL(probe_rate_kernel<3>, dim3(grid), dim3(kProbeThreads), 0, stream, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rpa

namespace {
constexpr int kMaxProbeGrid = 65536;
int launched(hipError_t e) { return e == hipSuccess ? RPA_OK : RPA_E_HIP; }
}  // namespace

extern "C" int rpa_probe_stream(const void* buf, size_t bytes, int workgroups, int flags,
                                rpa_stream_t stream) {
  if (!buf || workgroups < 1 || workgroups > kMaxProbeGrid || flags < 0 || flags > 7 ||
      bytes / (size_t)workgroups < (size_t)(32 * 1024))
    return RPA_E_INVALID;
  return launched(rpa::probe_stream(buf, bytes, workgroups, flags, stream));
}

extern "C" int rpa_probe_rate(int kind, int workgroups, float* sink, rpa_stream_t stream) {
  if (!sink || kind < 0 || kind > 3 || workgroups < 1 || workgroups > kMaxProbeGrid)
    return RPA_E_INVALID;
  return launched(rpa::probe_rate(kind, workgroups, sink, stream));
}

extern "C" int rpa_probe_issue(int kind, int waves, int count, int workgroups, const void* src,
                               size_t src_bytes, unsigned long long* ticks, float* sink,
                               rpa_stream_t stream) {
  if (!src || !ticks || !sink || kind < 0 || kind > 1 || waves < 1 || waves > 8 ||
      (count != 4 && count != 16) || workgroups < 1 || workgroups > kMaxProbeGrid ||
      src_bytes < (size_t)count * 1024)
    return RPA_E_INVALID;
  return launched(
      rpa::probe_issue(kind, waves, count, workgroups, src, src_bytes, ticks, sink, stream));
}

extern "C" int rpa_probe_chain(int mode, int workgroups, unsigned long long* cycles, float* sink,
                               rpa_stream_t stream) {
  if (!cycles || !sink || mode < 0 || mode > 14 || (mode & 1) || workgroups < 1 ||
      workgroups > kMaxProbeGrid)
    return RPA_E_INVALID;
  return launched(rpa::probe_chain(mode, workgroups, cycles, sink, stream));
}
