// Device-side helpers shared by the gfx950 kernels of librpa.
//
// Everything here is wave64 / CDNA4 specific: MFMA builtins, the hardware
// exp2, OCP-fp8 conversions and lane shuffles. Nothing here is used by the
// CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rpa {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float floatx2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_INT8 = 3, DT_INT4 = 4 };

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

// Two fp32 -> packed pair of bf16 (low half = a), round to nearest even, with
// gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const floatx2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Four OCP E4M3FN bytes of `w` -> four fp32 (exact; the hardware converter
// of gfx950 uses the OCP encoding).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0];
  o[1] = lo[1];
  o[2] = hi[0];
  o[3] = hi[1];
}

// Four OCP E4M3FN bytes -> two dwords of packed bf16 (exact: every E4M3FN
// value is a bf16 value, so the bf16 pattern is the fp32 pattern's top half).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  u32x2 r;
  r[0] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
  r[1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  return r;
}

// Two fp32 -> packed pair of IEEE half (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
  const floatx2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, halfx2));
}
__device__ __forceinline__ void unpack_f16x2(uint32_t w, float& a, float& b) {
  typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
  const halfx2 h = __builtin_bit_cast(halfx2, w);
  a = (float)h[0];
  b = (float)h[1];
}

// Split-KV partials hold a split's output normalised by its own row sum: a
// convex combination of value rows, so |x| <= max |V|. Pools whose values fit
// IEEE half (fp8 E4M3FN: |V| <= 448) store them as fp16 (2^-11 relative);
// bf16 pools, whose values may exceed half's range, store bf16 (2^-9, the same
// rounding the final bf16 output takes anyway).
__device__ __forceinline__ uint32_t pack_part(float a, float b, bool f16) {
  return f16 ? pack_f16x2(a, b) : pack_bf16x2(a, b);
}
__device__ __forceinline__ void unpack_part(uint32_t w, float& a, float& b, bool f16) {
  if (f16) {
    unpack_f16x2(w, a, b);
  } else {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xffff0000u);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its definition, tanh(x) = 1 - 2 / (exp(2x) + 1), evaluated with
// the hardware exp2; saturates cleanly to +-1 for large |x|.
__device__ __forceinline__ float tanh_def(float x) {
  const float e = fast_exp2(2.0f * kLog2e * x);
  return 1.0f - 2.0f / (e + 1.0f);
}

// The capped logit in the log2 domain, cap * tanh(s * scale / cap) * log2(e),
// by its odd Taylor series in y = s * scale / cap up to y^5 (four VALU
// instructions against two transcendentals and a reciprocal for the exact
// form). For |y| <= ymax the series alternates with falling terms, so the
// first omitted one, 17/315 y^7, bounds the error: ymax is the largest |y|
// (at most 1/2) at which that term times cap * log2(e) stays within 1e-4,
// i.e. a relative error of the weight 2^logit below 1e-4, a twentieth of its
// rounding to bf16. smax is the matching bound on the raw score |s|; smax3
// the (smaller) one up to which the series may stop at y^3 (first omitted
// term 2/15 y^5, same tolerance).
struct CapSeries {
  float a0, a1, a2, smax, smax3;
};

// (cap * tanh(x / cap) is even in cap: |cap| is used; the scale keeps its sign.)
__device__ __forceinline__ CapSeries cap_series(float cap, float scale) {
  constexpr float kTol = 1e-4f;
  const float c = scale / fabsf(cap);
  const float k = fabsf(cap) * kLog2e;
  // ymax = (kTol / (k * 17 / 315))^(1/7), by the hardware log2 and exp2.
  const float ymax =
      fminf(0.5f, fast_exp2(__builtin_amdgcn_logf(kTol / (k * (17.f / 315.f))) * (1.f / 7.f)));
  // ymax3 = (kTol / (k * 2 / 15))^(1/5).
  const float ymax3 =
      fminf(0.5f, fast_exp2(__builtin_amdgcn_logf(kTol / (k * (2.f / 15.f))) * (1.f / 5.f)));
  const float c2 = c * c;
  CapSeries r;
  r.a0 = k * c;
  r.a1 = -r.a0 * c2 * (1.f / 3.f);
  r.a2 = r.a0 * c2 * c2 * (2.f / 15.f);
  r.smax = ymax / fabsf(c);
  r.smax3 = ymax3 / fabsf(c);
  // A cap so small that a coefficient overflows (below about 1e-11 at unit
  // scale) would give 0 * inf for a zero score: such calls keep the exact form.
  if (!(__builtin_isfinite(r.a1) && __builtin_isfinite(r.a2))) r.smax = r.smax3 = -1.f;
  return r;
}

// The series' capped logit of a raw score s plus `shift` (|s| <= smax).
__device__ __forceinline__ float cap_series_eval(const CapSeries& cs, float s, float shift) {
  const float s2 = s * s;
  return fmaf(s, fmaf(s2, fmaf(s2, cs.a2, cs.a1), cs.a0), shift);
}

// The same series stopped at y^3 (|s| <= smax3): one FMA less.
__device__ __forceinline__ float cap_series3_eval(const CapSeries& cs, float s, float shift) {
  return fmaf(s, fmaf(s * s, cs.a1, cs.a0), shift);
}

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16) on one wave.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16], and
// D[4*(l/16) + i][l%16] for i = 0..3.
__device__ __forceinline__ floatx4 mfma_16x16x32(const bf16x8& a, const bf16x8& b,
                                                 const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16) on one wave (twice the rate
// of the 16x16x32 form on gfx950). Lane l holds A[l%32][8*(l/32) .. +7],
// B[8*(l/32) .. +7][l%32], and D[8*(r/4) + 4*(l/32) + r%4][l%32] in register r.
__device__ __forceinline__ floatx16 mfma_32x32x16(const bf16x8& a, const bf16x8& b,
                                                  const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// {v of lane l, v of lane l ^ 16} (MASK 16) or {.., l ^ 32} (MASK 32) with
// gfx950's v_permlane16_swap / v_permlane32_swap: swapping v with itself
// leaves the even row's (even half's) value in the first result and the odd
// row's (odd half's) in the second, in both lanes of the pair. Plain VALU
// ops, unlike a ds_bpermute shuffle.
template <int MASK>
__device__ __forceinline__ void pair_xor(float v, float& a, float& b) {
  static_assert(MASK == 16 || MASK == 32, "row or half swap only");
  const uint32_t u = __float_as_uint(v);
  const auto r = MASK == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// max / sum of v over lanes l and l ^ MASK (MASK = 16 or 32); the sum adds
// in the same order in both lanes, so they get identical bits.
template <int MASK>
__device__ __forceinline__ float wave_max_xor(float v) {
  float a, b;
  pair_xor<MASK>(v, a, b);
  return fmaxf(a, b);
}
template <int MASK>
__device__ __forceinline__ float wave_sum_xor(float v) {
  float a, b;
  pair_xor<MASK>(v, a, b);
  return a + b;
}

__device__ __forceinline__ int cdiv_i(int a, int b) { return (a + b - 1) / b; }

// Online softmax with a lazily moved reference max (log2 domain). Weights are
// p = 2^(s - m_ref); the reference only moves (and the accumulators are
// rescaled by 2^(m_ref_old - m_ref_new)) when a block's row max exceeds it by
// more than kLazyTau, so p <= 2^kLazyTau and most blocks skip the rescale.
constexpr float kLazyTau = 8.0f;

__device__ __forceinline__ bool wave_any(bool v) {
  return __builtin_amdgcn_ballot_w64(v) != 0;
}

typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef short shortx4 __attribute__((__vector_size__(4 * sizeof(short))));

// D(16x16 f32) += A(16x16 bf16) * B(16x16 bf16); lane l holds A[l%16][4*(l/16)+i],
// B[4*(l/16)+i][l%16] (i = 0..3) and D as for mfma_16x16x32.
__device__ __forceinline__ floatx4 mfma_16x16x16(const u32x2& a, const u32x2& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                    __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
}

// ---- LDS direct loads and explicit synchronisation -------------------------
// One global_load_lds_dwordx4: lane L's 16 bytes at `gaddr` land in LDS at
// lds_base + 16*L, where lds_base (a byte address, wave-uniform) goes in M0.
// Issued through inline asm so the compiler's wait-count pass does not treat
// it as an LDS store and add waits before unrelated LDS reads; callers wait
// with wait_vmcnt<N>() (vector-memory ops complete in issue order).
// Because the compiler cannot see the memory instruction inside the asm, the
// asm carries its own wait states: one between the M0 write and the LDS-DMA
// load that reads M0, and five after the load before the compiler may reuse
// the address registers. Callers also read everything a block's DMA needs
// from LDS before issuing it: LDS reads interleaved between the LDS-DMA
// instructions of one wave gave wrong rows on gfx950.
// once: the rows are read by this launch only once (a decode tile's keys);
// the load then carries the non-temporal cache policy (nt), with which a
// streaming read through LDS-DMA measured 7.1 against 6.3 TB/s. Rows that
// other tiles read again (prefill query blocks, sparse selections) keep the
// default policy. The flag must be wave-uniform.
__device__ __forceinline__ void dma_b128(const void* gaddr, uint32_t lds_base, bool once = false) {
  if (__builtin_amdgcn_readfirstlane((int)once))
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_nop 4"
        :
        : "s"(lds_base), "v"(gaddr)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 4"
        :
        : "s"(lds_base), "v"(gaddr)
        : "memory");
}

// As dma_b128 with a wave-uniform 64-bit base (SGPRs) plus a per-lane 32-bit
// byte offset: lane L's 16 bytes at sbase + voff land at lds_base + 16*L.
__device__ __forceinline__ void dma_b128_s(const void* sbase, uint32_t voff, uint32_t lds_base,
                                           bool once = false) {
  if (__builtin_amdgcn_readfirstlane((int)once))
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_nop 4"
        :
        : "s"(lds_base), "v"(voff), "s"(sbase)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_nop 4"
        :
        : "s"(lds_base), "v"(voff), "s"(sbase)
        : "memory");
}

// x ^ s computed where it stands: the asm keeps the compiler from hoisting a
// set of such values out of a loop and holding (or spilling) them.
__device__ __forceinline__ uint32_t xor_here(uint32_t x, uint32_t s) {
  uint32_t r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(s), "v"(x));
  return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Waits for every outstanding vector-memory op with an s_waitcnt the
// compiler's wait-count pass can see (vmcnt 0, expcnt and lgkmcnt untouched).
// Called before a DMA-pipelined loop: the pass then knows the loads issued
// before the loop (queries, page ids) are complete and does not put a
// vmcnt(0) inside the loop, which would also drain the in-flight DMA.
__device__ __forceinline__ void drain_vmem_before_loop() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Compiler-only fence: memory accesses are not moved across it. Used to keep
// the scheduler from hoisting a whole unrolled loop's LDS loads at once.
__device__ __forceinline__ void sched_fence() { asm volatile("" : : : "memory"); }

// Compiler fence that also pins `x`: memory accesses stay on their side of it
// and every later use of x stays below it. Placed after a prefetch, it keeps
// the MFMA that consumes x from being scheduled above the prefetch.
template <typename T>
__device__ __forceinline__ void pin_after(T& x) {
  asm volatile("" : "+v"(x) : : "memory");
}

// x *= alpha for an MFMA accumulator element kept in an AGPR: the constraint
// keeps the value in its AGPR (a plain multiply would make the compiler hold
// the whole accumulator set in VGPRs around a rarely taken rescale).
__device__ __forceinline__ void scale_acc(float& x, float alpha) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "+a"(x), "=&v"(t)
      : "v"(alpha));
}

// Wait states between the MFMA that last wrote an accumulator and the
// hand-written AGPR accesses above (and between those and the next MFMA).
__device__ __forceinline__ void mfma_agpr_fence() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Workgroup barrier without the fence __syncthreads() carries (that fence
// would drain outstanding LDS DMA); also a compiler barrier for memory.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" : : : "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
      (__attribute__((address_space(3))) char*)(uintptr_t)addr);
}

__device__ __forceinline__ u32x2 lds_read_b64(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
      (__attribute__((address_space(3))) char*)(uintptr_t)addr);
}

// ds_read_b64_tr_b8: within each 16-lane group, lanes 2r and 2r+1 name the two
// 8-byte halves of a 16-byte row r (r = 0..7); lane j of the group receives
// byte j of rows 0..7, in row order.
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t addr) {
  typedef int intx2 __attribute__((ext_vector_type(2)));
  intx2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) intx2*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// ds_read_b64_tr_b16: within each 16-lane group the four lanes 4r..4r+3 name
// row r (4 consecutive b16 each); lane j of the group receives column j of the
// 4x16 block, i.e. element j of rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// Eight OCP E4M3FN bytes (in order) to eight bf16 (in order), exactly: every
// E4M3FN value is a bf16 value (v_cvt_scalef32_pk_bf16_fp8 at scale 1).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[h], 1.0f, false));
    r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[h], 1.0f, true));
  }
  return r;
}

// Four two's-complement bytes of `w` -> four fp32, exactly: byte n of
// w ^ 0x80808080 is b + 128 as an unsigned byte (one v_cvt_f32_ubyteN), and
// 128 comes off again.
__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float* o) {
  const uint32_t u = w ^ 0x80808080u;
#pragma unroll
  for (int n = 0; n < 4; ++n) o[n] = (float)((u >> (8 * n)) & 0xffu) - 128.f;
}

// Four int8 -> two dwords of packed bf16 (exact: integers of magnitude <= 128
// are bf16 values).
__device__ __forceinline__ u32x2 i8x4_to_bf16x4(uint32_t w) {
  float f[4];
  i8x4_to_f32(w, f);
  return u32x2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
}

// Eight int8 (in order) to eight bf16 (in order), exactly.
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(u32x2 w) {
  const u32x2 lo = i8x4_to_bf16x4(w[0]), hi = i8x4_to_bf16x4(w[1]);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// One-byte pool elements (fp8 E4M3FN or int8) widened to bf16, by pool dtype.
template <int DT>
__device__ __forceinline__ u32x2 kv8x4_to_bf16x4(uint32_t w) {
  if constexpr (DT == DT_INT8) return i8x4_to_bf16x4(w);
  else return fp8x4_to_bf16x4(w);
}
template <int DT>
__device__ __forceinline__ u32x4 kv8x8_to_bf16x8(u32x2 w) {
  if constexpr (DT == DT_INT8) return i8x8_to_bf16x8(w);
  else return fp8x8_to_bf16x8(w);
}

// Eight queries in storage type `dt` (bf16, or fp8 E4M3FN widened exactly) as
// eight bf16: `p` points at element `e` of a bf16 or byte array.
__device__ __forceinline__ u32x4 load_q8(const void* p, int64_t e, int dt) {
  if (dt == DT_FP8)
    return fp8x8_to_bf16x8(*reinterpret_cast<const u32x2*>((const uint8_t*)p + e));
  return *reinterpret_cast<const u32x4*>((const uint16_t*)p + e);
}

// Largest i in [0, n) with cu[i] <= t (the sequence owning packed token t),
// or -1 when t is past cu[n].
__device__ __forceinline__ int find_seq(const int32_t* cu, int n, int t) {
  if (n <= 0 || t >= cu[n] || t < cu[0]) return -1;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace rpa
