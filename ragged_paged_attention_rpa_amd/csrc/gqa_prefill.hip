// Prefill-class tiles of GQA ragged paged attention on gfx950 [RPA v2 page:
// ragged_paged_attention, flash_attention].
//
// A prefill tile is (sequence, kv head, block of query tokens): its rows are
// the (query token, q head of the group) pairs, up to 256 of them, against
// every key the block's queries can see. The per-row arithmetic is the
// page's: scale, optional soft cap, mask (causal offset kv_len - q_len,
// optional sliding window), online softmax, P V.
//
// Workgroup: eight waves, 32 rows each, in two groups of four (A = waves
// 0..3, B = waves 4..7; wave w and wave w + 4 share a SIMD). Keys arrive in
// blocks of 64 through a ring of LDS stages. Each wave alternates two kinds
// of phase over the blocks:
//   MFMA phase j:  O^T += V_{j-1}^T P_{j-1}^T, then S^T_j = K_j Q^T
//                  (v_mfma_f32_32x32x16_bf16 throughout);
//   VALU phase j:  the online softmax of S_j (mask, cap, row max, exp2,
//                  row sum) producing P_j in bf16.
// Group B runs one phase behind group A and every phase ends with a
// workgroup barrier, so on each SIMD one wave multiplies while the other
// does its softmax: the matrix core and the vector ALU work at the same
// time instead of taking turns inside one wave.
//
// Operand layouts (32x32x16, lane l, c = l / 32):
//  * S^T = K Q^T: A = 32 keys x 16 dims (lane: key l%32, dims 8c..), B = Q^T
//    held in registers for the whole tile (lane: row l%32, dims 16ks + 8c..).
//    Lane l ends with row l%32's scores for keys 8q + 4c + t in register
//    4q + t of each 32-key half of the block.
//  * O^T += V^T P^T over 16-key steps u: the step's reduction index 8c + jj
//    is taken to mean key 16u + 4c + jj (jj < 4) or 16u + 4c + 8 + (jj - 4),
//    which is exactly what lane l already holds (registers 8(u%2) .. +7 of
//    half u/2), so P needs no shuffle; V^T is read in the same key order with
//    two ds_read_b64_tr_b16 per operand.
//
// LDS block layout: key-major, 512 bytes per key (K dims in 16-byte columns
// 0..15, V dims in 16..31); column q of key k sits at q ^ kswz(k), which
// keeps the K reads (16 keys, one column) and the transposed V reads (four
// keys, four columns) free of bank conflicts. The DMA (global_load_lds,
// 1 KB per instruction) applies the swizzle by choosing which global column
// each lane fetches. fp8 pools land raw (256 bytes per key, column rc at
// rc ^ (k & 15)) and group A widens each block once to bf16, exactly (every
// E4M3FN value is a bf16 value), during its VALU phase; widening each
// wave's operands in registers instead would convert every block eight
// times over.
#include <type_traits>

#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kBN = 64;                            // keys per block
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kKeyBytes = 512;                     // K + V of one key, bf16
constexpr int kRawKeyBytes = 256;                  // K + V of one key, fp8
constexpr int kStage = kBN * kKeyBytes;            // 32 KB
constexpr int kRawStage = kBN * kRawKeyBytes;      // 16 KB
constexpr int kBf16Stages = 4;                     // bf16 pools: DMA ring
constexpr int kConvStages = 3;                     // fp8 pools: widened ring
constexpr int kRawStages = 2;                      // fp8 pools: raw DMA ring

__device__ __attribute__((aligned(16))) const uint8_t kPreZero[512] = {0};

template <int KV_DT>
struct PreSmem {
  char buf[KV_DT == DT_BF16 ? kBf16Stages * kStage : kConvStages * kStage + kRawStages * kRawStage];
  int tile;
};

// Column swizzle of a key (its low four bits): a bit rotation, so sixteen
// consecutive keys get sixteen distinct columns, and the four keys of an
// aligned quad get distinct values in bits 2..3.
__device__ __forceinline__ int kswz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }

__device__ __forceinline__ uint32_t key_col(int key, int q) {
  return (uint32_t)(key * kKeyBytes + ((q ^ kswz(key)) << 4));
}


// Scalar (SGPR) read of a wave-uniform int32 from global memory.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      (const __attribute__((address_space(4))) char*)p);
}

template <int KV_DT, bool CAP>
__device__ void prefill_tile(const GqaArgs& a, const Tile tile, PreSmem<KV_DT>& sm, int ps_log2) {
  constexpr bool F8 = KV_DT != DT_BF16;  // one-byte pool (fp8 or int8), widened in LDS
  constexpr int kIPW = (F8 ? kRawStage : kStage) / 1024 / kWaves;  // DMA instructions per wave per block
  constexpr int kEB = F8 ? 1 : 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int c = lane >> 5;
  const int G = a.geo.group;
  const int W = a.geo.window;

  // Tile and sequence metadata are workgroup-uniform: keep them in SGPRs.
  const int seq = __builtin_amdgcn_readfirstlane(tile.seq);
  const int qtok0 = __builtin_amdgcn_readfirstlane(tile.qtok0);
  const int kvh = __builtin_amdgcn_readfirstlane(tile.kvh);
  const int cu0 = __builtin_amdgcn_readfirstlane(a.cu_q_lens[seq]);
  const int q_len = __builtin_amdgcn_readfirstlane(a.cu_q_lens[seq + 1]) - cu0;
  const int kv_len = __builtin_amdgcn_readfirstlane(a.kv_lens[seq]);
  const int kv_cap = min(kv_len, a.pages_per_seq << ps_log2);
  const int ntok = min(a.geo.bq, q_len - qtok0);
  const int first = kv_len - q_len + qtok0;  // position of the block's first query
  const int lo = W > 0 ? max(0, first - W + 1) : 0;
  const int hi = min(first + ntok, kv_cap);
  const int nrows = ntok * G;

  const int r = kRowsPerWave * wave + (lane & 31);
  const bool row_ok = r < nrows;
  const bool wave_active = kRowsPerWave * wave < nrows;
  const int qpos = first + r / G;
  // Keys row r sees: [vlo_r, vhi_r) (empty past the tile's rows).
  const int vlo_r = row_ok ? max(lo, W > 0 ? qpos - W + 1 : 0) : 0;
  const int vhi_r = row_ok ? min(hi, qpos + 1) : 0;

  // Q^T operand, k-step ks: row r, dims 16ks + 8c .. +7.
  u32x4 qv[8];
  {
    const int tok = cu0 + qtok0 + (row_ok ? r / G : 0);
    const int head = kvh * G + (row_ok ? r % G : 0);
    const int64_t q0 = ((int64_t)tok * a.num_q_heads + head) * kD + 8 * c;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = load_q8(a.q, q0 + 16 * ks, a.q_dtype);
      qv[ks] = v;
    }
  }

  floatx16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  }
  floatx16 sv[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[tt][i] = 0.f;
  u32x4 pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = u32x4{0u, 0u, 0u, 0u};
  float m_run = -INFINITY, l_run = 0.f;

  const int kb0 = (lo / kBN) * kBN;
  const int nblk = hi > kb0 ? cdiv_i(hi - kb0, kBN) : 0;
  const int32_t* table = a.page_indices + (int64_t)seq * a.pages_per_seq;
  const int ps_mask = (1 << ps_log2) - 1;
  const int64_t token_bytes = (int64_t)2 * a.num_kv_heads * kD * kEB;
  const char* kv_head = (const char*)a.kv + (int64_t)(2 * kvh) * kD * kEB;
  // Keys at or past new_start are the step's new tokens, read from new_kv
  // (same row layout as the pool, one row per packed token).
  const int new_start = a.new_kv != nullptr ? kv_len - q_len : 0x7fffffff;
  const char* new_head = (const char*)a.new_kv + (int64_t)(2 * kvh) * kD * kEB;
  const uint32_t sbase = lds_addr(sm.buf);

  // LDS byte address of the bf16 block j (j >= -1; block -1 is the zeroed
  // stage the first MFMA phase multiplies by P = 0), and (fp8) of its raw
  // copy.
  constexpr int kStages = F8 ? kConvStages : kBf16Stages;
  auto stage = [&](int j) -> uint32_t {
    return sbase + (uint32_t)((j + kStages) % kStages) * kStage;
  };
  auto raw_stage = [&](int j) -> uint32_t {
    return sbase + (uint32_t)(kConvStages * kStage) + (uint32_t)(j % kRawStages) * kRawStage;
  };

  // This wave's share of block j: keys k8 .. k8 + 7, all in one page (page
  // size >= 8). Its id comes through a scalar load issued an iteration ahead
  // of the DMA (page_of), so the DMA never waits for the page table. Keys
  // outside [lo, hi) or on an invalid page read zeros instead.
  auto page_of = [&](int j) -> int {
    const int k8 = kb0 + j * kBN + 8 * wave;
    return load_uniform(table + min(k8 >> ps_log2, a.pages_per_seq - 1));
  };
  // This wave's share of block j: kIPW DMA instructions of 1 KB. The wave's
  // eight keys start at k8 = kb0 + 64 j + 8 wave, so their low four bits (and
  // with them the swizzled columns) are the same in every block: each lane's
  // byte offset from the chunk's first row is fixed (dofs), and its low bits
  // are the column's offset (a row is a multiple of 512 bytes for bf16, of
  // 256 for fp8). A chunk wholly inside [lo, hi) on a valid page (all but the
  // range's ends) is addressed as one SGPR base plus these fixed offsets;
  // otherwise each lane checks its key and reads zeros for keys outside the
  // range or on an invalid page.
  uint32_t dofs[kIPW];
#pragma unroll
  for (int ii = 0; ii < kIPW; ++ii) {
    const int sub = F8 ? lane >> 4 : lane >> 5;
    const int e = (F8 ? 4 : 2) * ii + sub;
    const int klow = 8 * (wave & 1) + e;  // key & 15
    const int col = F8 ? ((lane & 15) ^ klow) : ((lane & 31) ^ kswz(klow));
    dofs[ii] = (uint32_t)(e * token_bytes + (col << 4));
  }
  auto issue = [&](int j, int page) {
    const int k8 = kb0 + j * kBN + 8 * wave;
    const bool page_ok = page >= 0 && page < a.total_num_pages;
    const char* rowbase = kv_head + (((int64_t)page << ps_log2) + (k8 & ps_mask)) * token_bytes;
    // Row of key k8 in new_kv (only lanes whose key is a new token use it).
    const char* newbase = new_head + (int64_t)(cu0 + k8 - new_start) * token_bytes;
    const uint32_t dst = __builtin_amdgcn_readfirstlane((F8 ? raw_stage(j) : stage(j)) +
                                                       (uint32_t)(wave * kIPW) * 1024);
    const bool whole = k8 >= lo && k8 + 8 <= hi;
    if (whole && page_ok && k8 + 8 <= new_start) {
#pragma unroll
      for (int ii = 0; ii < kIPW; ++ii) dma_b128_s(rowbase, dofs[ii], dst + (uint32_t)ii * 1024);
    } else if (whole && k8 >= new_start) {
#pragma unroll
      for (int ii = 0; ii < kIPW; ++ii) dma_b128_s(newbase, dofs[ii], dst + (uint32_t)ii * 1024);
    } else {
      const int sub = F8 ? lane >> 4 : lane >> 5;
#pragma unroll
      for (int ii = 0; ii < kIPW; ++ii) {
        const int key = k8 + (F8 ? 4 : 2) * ii + sub;
        const bool in = key >= lo && key < hi;
        const char* src = (const char*)kPreZero + (dofs[ii] & (F8 ? 0xF0u : 0x1F0u));
        if (in && key >= new_start)
          src = newbase + dofs[ii];
        else if (in && page_ok)
          src = rowbase + dofs[ii];
        dma_b128(src, dst + (uint32_t)ii * 1024);
      }
    }
  };

  // fp8: widen raw block j into bf16 stage j (group A's 256 threads; thread
  // t takes raw column t/16 of keys t%16 + 16i).
  auto widen = [&](int j) {
    // Keys tid%16 + 16i share their low four bits, hence their swizzles: one
    // lane offset per side, the key step is a constant (4 KB raw, 8 KB bf16).
    const int k0 = tid & 15, rc = tid >> 4;
    const uint32_t src = raw_stage(j) + (uint32_t)(k0 * kRawKeyBytes + ((rc ^ k0) << 4));
    const uint32_t dlo = stage(j) + key_col(k0, 2 * rc);
    const uint32_t dhi = stage(j) + key_col(k0, 2 * rc + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = lds_read_b128(src + (uint32_t)(i * 16 * kRawKeyBytes));
      const u32x4 lo4 = kv8x8_to_bf16x8<KV_DT>(u32x2{w[0], w[1]});
      const u32x4 hi4 = kv8x8_to_bf16x8<KV_DT>(u32x2{w[2], w[3]});
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (__attribute__((address_space(3))) char*)(uintptr_t)(dlo + (uint32_t)(i * 16 * kKeyBytes))) = lo4;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (__attribute__((address_space(3))) char*)(uintptr_t)(dhi + (uint32_t)(i * 16 * kKeyBytes))) = hi4;
      sched_fence();  // one key at a time: bounds the registers the widening holds
    }
  };

  // Per-lane operand offsets inside a block stage. K: key lane%32 of the
  // first 32-key half, column 2ks + c, at kbase ^ (ks << 5) (second half 16 KB
  // further). V^T: dims 16(lane/16 % 2) + lane%16 of 32-dim tile dt for keys
  // 4c + (lane%16)/4 at vbase[0] ^ (dt << 6) and the same + 8 at
  // vbase[1] ^ (dt << 6); 16-key step u is 8 KB further. The XORs are taken
  // at each read (xor_here): the MFMA wave has VALU slots to spare, and
  // sixteen precomputed offsets would be sixteen registers.
  uint32_t kbase, vbase[2];
  {
    const int kk = lane & 31;
    kbase = (uint32_t)(kk * kKeyBytes + ((c ^ kswz(kk)) << 4));
    const int jj = lane & 15;
    const int x = 16 + 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
    const int k_lo = 4 * c + (jj >> 2), k_hi = k_lo + 8;
    vbase[0] = (uint32_t)(k_lo * kKeyBytes + ((x ^ kswz(k_lo)) << 4) + 8 * (jj & 1));
    vbase[1] = (uint32_t)(k_hi * kKeyBytes + ((x ^ kswz(k_hi)) << 4) + 8 * (jj & 1));
  }

  // Log2-domain logit of a raw score s: s * c1, or with the soft cap
  // cap * tanh(s * scale / cap) * log2(e), tanh(z) taken as 1 - 2 / (e^{2z} + 1)
  // (hardware exp2 and reciprocal): c2 - c3 / (2^{s c1} + 1).
  // cap * tanh(x / cap) is even in cap: |cap| is used, so c1 > 0 whenever the
  // score scale is (the launcher's precondition).
  const float cap = fabsf(a.soft_cap);
  const float c1 = CAP ? 2.f * kLog2e * a.score_scale / cap : a.score_scale * kLog2e;
  const float c2 = cap * kLog2e, c3 = 2.f * cap * kLog2e;
  const CapSeries cs = cap_series(cap, a.score_scale);

  // MFMA phase j: O^T += V_{j-1}^T P_{j-1}^T (16 MFMAs), then S^T_j = K_j Q^T
  // (16 MFMAs). The 32 A operands (V^T from block j - 1, then K from block j)
  // stream through one ring of kAhead registers: operand t + kAhead is read
  // while MFMA t runs (an LDS read takes several MFMAs to return), and the
  // ring's first kAhead reads can be issued at the end of the wave's previous
  // phase (ring_start), so the phase opens with its operands in flight. One
  // copy of this code serves every phase: at j == 0 block -1 is a zeroed
  // stage (and P is zero), at j == nblk the QK half runs on a stale stage and
  // its scores are never used.
  auto pv_stage = [&](int j) -> uint32_t { return stage(j - 1); };
  // Per-phase bases: the stage address plus a lane's offset, taken once per
  // phase (ring_start); each read then only XORs in its column (stage
  // addresses are multiples of 16 KB, so the XOR stays inside the offset) and
  // adds a constant (folded into the read's offset field).
  uint32_t pvb[2] = {0u, 0u}, kb = 0u;
  auto phase_bases = [&](int j) {
    pvb[0] = pv_stage(j) + vbase[0];
    pvb[1] = pv_stage(j) + vbase[1];
    kb = stage(j) + kbase;
  };
  auto operand = [&](int t) -> u32x4 {
    if (t < 16) {
      const uint32_t u = (uint32_t)((t >> 2) * 16 * kKeyBytes);
      const u32x2 v0 = lds_read_tr16(xor_here(pvb[0], (uint32_t)((t & 3) << 6)) + u);
      const u32x2 v1 = lds_read_tr16(xor_here(pvb[1], (uint32_t)((t & 3) << 6)) + u);
      return u32x4{v0[0], v0[1], v1[0], v1[1]};
    }
    const int m = t - 16;  // k-step m/2 of 32-key half m%2
    return lds_read_b128(xor_here(kb, (uint32_t)((m >> 1) << 5)) + (uint32_t)((m & 1) * 32 * kKeyBytes));
  };
  constexpr int kAhead = 8;
  u32x4 ring[kAhead];
  auto ring_start = [&](int j) {
    sched_fence();  // the reads stay after the wave's preceding work
    phase_bases(j);
#pragma unroll
    for (int t = 0; t < kAhead; ++t) ring[t] = operand(t);
  };
  auto mfma_phase = [&](int j) {
    // With the soft cap the partner wave's long VALU stream would otherwise
    // win issue slots over this wave's operand reads (the older wave goes
    // first): the MFMA wave takes the higher priority for its phase
    // (measured: a loss without the cap, where the VALU phase is shorter).
    if constexpr (CAP) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      u32x4 x = ring[t % kAhead];
      pin_after(x);
      if (t < 16) {
        acc[t & 3] = mfma_32x32x16(as_bf16x8(x), as_bf16x8(pb[t >> 2]), acc[t & 3]);
      } else {
        const int m = t - 16;
        const floatx16 zero = {};  // k-step 0 starts from zero (an inline constant)
        sv[m & 1] = mfma_32x32x16(as_bf16x8(x), as_bf16x8(qv[m >> 1]), m < 2 ? zero : sv[m & 1]);
      }
      if (t + kAhead < 32) ring[t % kAhead] = operand(t + kAhead);
    }
    if constexpr (CAP) __builtin_amdgcn_s_setprio(0);
  };

  // VALU phase j: the online softmax of S_j. A row keeps a reference m_run
  // and its weights are p = 2^{logit - m_run} (log2-domain logits), in bf16
  // for the PV step. The reference only has to keep the weights in range, so
  // a block is first weighted against the current reference and its row sums
  // are checked (kSumBound). Only a fresh row (no reference yet) or a sum
  // above the bound takes the row maximum (on raw scores: both logit maps
  // are increasing) and moves the reference if the maximum passes it by
  // kLazyTau, rescaling O and l, before weighting the block again.
  auto valu_phase = [&](int j) {
    const int kb = kb0 + j * kBN;
    // Keys [kb, kb + 64) visible to every row of the wave: no mask needed.
    const bool full =
        __builtin_amdgcn_ballot_w64(row_ok && !(kb >= vlo_r && kb + kBN <= vhi_r)) == 0;
    // Keys outside the row's range become -inf.
    auto mask = [&]() {
      const uint32_t span = (uint32_t)(vhi_r - vlo_r);
      const int kbase_r = kb + 4 * c - vlo_r;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool vis = (uint32_t)(kbase_r + 32 * tt + 8 * (i >> 2) + (i & 3)) < span;
          sv[tt][i] = vis ? sv[tt][i] : -INFINITY;
        }
    };
    if (!CAP && !full) mask();
    // Logits are taken relative to mref (the reference, 0 for a fresh row).
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    if (CAP) {
      // Capped logits minus mref, in place. A block whose raw scores all lie
      // within the series' range (NaN garbage in masked lanes is ignored by
      // the maximum, and masked afterwards) takes the series; any other the
      // exact form, one pass per step over the 32 scores (independent
      // neighbours hide each step's latency).
      float am = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(sv[tt][i]));
      if (!wave_any(am > cs.smax3)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[tt][i] = cap_series3_eval(cs, sv[tt][i], -mref);
      } else if (!wave_any(am > cs.smax)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[tt][i] = cap_series_eval(cs, sv[tt][i], -mref);
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[tt][i] = fast_exp2(sv[tt][i] * c1) + 1.f;
        const float c2r = c2 - mref;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[tt][i] = fmaf(__builtin_amdgcn_rcpf(sv[tt][i]), -c3, c2r);
      }
      if (!full) mask();
    }
    // Weights p = 2^{logit - mref - shift} into pb (bf16); returns this
    // lane's half-row sum of the fp32 weights, in four add chains.
    // (v_dot2_f32_bf16 would sum the rounded pairs in one instruction, but on
    // gfx950 it waits for the SIMD's matrix pipe, which the partner wave
    // keeps busy.)
    auto weights = [&](float shift) -> float {
      const float nref = -(mref + shift);
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float w2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float x = sv[u >> 1][8 * (u & 1) + 2 * i + h];
            w2[h] = fast_exp2(CAP ? x - shift : fmaf(x, c1, nref));
          }
          pb[u][i] = pack_bf16x2(w2[0], w2[1]);
          ls[i & 3] += w2[0] + w2[1];
        }
      return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    // A row sum of at most 64 * 2^kLazyTau bounds every weight by 2^(kLazyTau
    // + 6) (a safe range for bf16 P and the fp32 sums), and a sum above it
    // means a weight above 2^kLazyTau, so the maximum then always moves the
    // reference. (A bound of 2^kLazyTau would also trip on blocks whose
    // weights are all in range, e.g. after a reference taken from a few keys,
    // and redo them every time.)
    constexpr float kSumBound = 64.f * 256.f;  // 64 * 2^kLazyTau
    float ls = 0.f;
    bool slow = wave_any(row_ok && m_run == -INFINITY);
    if (!slow) {
      ls = weights(0.f);
      float ap, bp;
      pair_xor<32>(ls, ap, bp);
      slow = wave_any(row_ok && ap + bp > kSumBound);
    }
    if (slow) {
      // Row maximum: four independent max chains (v_max3), then the row's
      // other lane; mb is the block maximum relative to mref.
      float mq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mq[q] = fmaxf(sv[q >> 1][8 * (q & 1)], sv[q >> 1][8 * (q & 1) + 1]);
#pragma unroll
        for (int i = 2; i < 8; ++i) mq[q] = fmaxf(mq[q], sv[q >> 1][8 * (q & 1) + i]);
      }
      const float mx = wave_max_xor<32>(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
      const float mb = CAP ? mx : (mx == -INFINITY ? -INFINITY : fmaf(mx, c1, -mref));
      const bool fresh = m_run == -INFINITY;
      const bool need = fresh ? mb != -INFINITY : mb > kLazyTau;
      const float d = need ? mb : 0.f;
      if (wave_any(need)) {
        const float alpha = (need && !fresh) ? fast_exp2(-d) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        m_run = need ? mref + d : m_run;
      }
      ls = weights(d);
    }
    l_run += ls;
  };

  // Block j is issued in phases 2j - 4 and 2j - 3 (one group each). A reads K_j
  // in phase 2j and V_j from the end of phase 2j + 1 through 2j + 2, B reads
  // K_j in phase 2j + 1 and V_j from the end of 2j + 2 through 2j + 3, so the
  // stage is free again when block j + 4 is issued in phase 2j + 4. Every
  // wave waits for its own DMA before the barrier that precedes the block's
  // first use.
  drain_vmem_before_loop();
  for (int j = 0; j < 2 && j < nblk; ++j) issue(j, page_of(j));
  int page_next = 2 < nblk ? page_of(2) : 0;  // page of the next block to issue
  {
    // Block -1 (the PV operand of MFMA phase 0): zeros.
    const uint32_t z = pv_stage(0) + (uint32_t)tid * 16;
#pragma unroll
    for (int i = 0; i < kStage / (16 * kThreads); ++i)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (__attribute__((address_space(3))) char*)(uintptr_t)(z + (uint32_t)(i * 16 * kThreads))) =
          u32x4{0u, 0u, 0u, 0u};
  }
  if (nblk > 1)
    wait_vmcnt<kIPW>();
  else
    wait_vmcnt<0>();
  if (F8) {
    wg_barrier();
    if (grp == 0 && nblk > 0) widen(0);
  }
  __syncthreads();

  // Whether group B issues its share of block b in phase 2b - 3 (and A in
  // 2b - 4) rather than the other way round. The DMA instructions go where
  // the wave has slack: in the VALU phases without the soft cap, in the MFMA
  // phases with it, whose softmax is the longer half.
  constexpr bool kLateB = CAP;

  // Closes phase p: this wave's DMA that the next phase needs has landed
  // (bf16: block (p + 1) / 2 after odd p; fp8: raw block p / 2 + 1 after even
  // p, before group A widens it; the late group has not issued the block
  // after that one yet), then the workgroup barrier (fp8: after the
  // widening's LDS writes have completed).
  auto close_phase = [&](int p, auto group_b) {
    constexpr bool kLate = decltype(group_b)::value == kLateB;
    const int jw = F8 ? ((p & 1) == 0 ? p / 2 + 1 : -1) : ((p & 1) == 1 ? (p + 1) / 2 : -1);
    if (jw >= 0 && jw < nblk) {
      if (jw + 1 < nblk && !(F8 && kLate))
        wait_vmcnt<kIPW>();
      else
        wait_vmcnt<0>();
    }
    if (F8) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wg_barrier();
  };
  // Whether the ring of the next MFMA phase is started at the end of the
  // VALU phase (measured faster without the soft cap) or at the start of the
  // MFMA phase (with it: its VALU phase is the longer one). fp8: group A's
  // VALU phase also widens the next block, and a ring held across it would
  // spill.
  constexpr bool kEarlyA = !CAP && !F8, kEarlyB = !CAP;
  // Group A: iteration j is MFMA phase j (phase 2j), then VALU phase j (phase
  // 2j + 1). Group B runs one phase later: after phase 0, its iteration j is
  // MFMA phase j (phase 2j + 1), then VALU phase j (phase 2j + 2). Each
  // group's loop thus carries only P across its back edge. Block b is issued
  // in phase 2b - 4 by the group that issues early and in phase 2b - 3 by the
  // other (kLateB), and each wave starts the ring of its next MFMA phase at
  // the end of its VALU phase when kEarly.
  using GA = std::false_type;
  using GB = std::true_type;
  auto run_a = [&]() {
    constexpr bool kLate = !kLateB;
    constexpr bool kEarly = kEarlyA;
    if (wave_active && kEarly) ring_start(0);
    for (int j = 0; j <= nblk; ++j) {
      const int page_dma = page_next;  // page of block j + 2
      if constexpr (!kLate) {
        if (j + 2 < nblk) issue(j + 2, page_dma);
      }
      if (wave_active) {
        if constexpr (!kEarly) ring_start(j);
        mfma_phase(j);
      }
      close_phase(2 * j, GA{});
      if constexpr (kLate) {
        if (j + 2 < nblk) issue(j + 2, page_dma);
      }
      if constexpr (F8) {
        if (j + 1 < nblk) widen(j + 1);
      }
      // The next page id is loaded where the VALU phase begins (after the
      // widening's LDS traffic): an outstanding scalar load makes every LDS
      // wait drain to zero.
      if (j + 3 < nblk) page_next = page_of(j + 3);
      if (wave_active && j < nblk) {
        valu_phase(j);
        if constexpr (kEarly) ring_start(j + 1);
      }
      close_phase(2 * j + 1, GA{});
    }
  };
  auto run_b = [&]() {
    constexpr bool kEarly = kEarlyB;
    if constexpr (!kLateB) {
      if (2 < nblk) issue(2, page_next);
      if (3 < nblk) page_next = page_of(3);
    }
    if (wave_active && kEarly) ring_start(0);
    close_phase(0, GB{});
    for (int j = 0; j <= nblk; ++j) {
      if constexpr (kLateB) {
        if (j + 2 < nblk) issue(j + 2, page_next);
      }
      if (wave_active) {
        if constexpr (!kEarly) ring_start(j);
        mfma_phase(j);
      }
      close_phase(2 * j + 1, GB{});
      if (j == nblk) break;
      // Page ids as in group A: loaded where the VALU phase begins.
      if constexpr (!kLateB) {
        if (j + 3 < nblk) issue(j + 3, page_next);
        if (j + 4 < nblk) page_next = page_of(j + 4);
      } else {
        if (j + 3 < nblk) page_next = page_of(j + 3);
      }
      if (wave_active) {
        valu_phase(j);
        if constexpr (kEarly) ring_start(j + 1);
      }
      close_phase(2 * j + 2, GB{});
    }
  };
  if (grp == 0)
    run_a();
  else
    run_b();

  if (!wave_active) return;
  // Normalise and store: row lane%32, dims 32dt + 8q + 4c .. +3 in registers
  // 4q .. 4q + 3 of acc[dt].
  float ap, bp;
  pair_xor<32>(l_run, ap, bp);
  const float l_row = ap + bp;
  if (!row_ok) return;
  const float inv = l_row > 0.f ? a.v_scale / l_row : 0.f;
  const int tok = cu0 + qtok0 + r / G;
  const int head = kvh * G + r % G;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)tok * a.num_q_heads + head) * kD + 4 * c;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[dt][4 * qq] * inv, acc[dt][4 * qq + 1] * inv);
      w[1] = pack_bf16x2(acc[dt][4 * qq + 2] * inv, acc[dt][4 * qq + 3] * inv);
      *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * qq) = w;
    }
}

// Workgroup b runs on XCD b % kXcds (the dispatcher places workgroups round
// robin over the XCDs). The prefill tiles, listed by (sequence, kv head,
// query block), are cut into kXcds contiguous ranges, one per XCD, so the
// query blocks that stream the same keys share one L2; a workgroup whose
// range is used up takes tiles from the other ranges.

template <int KV_DT, bool CAP>
__global__ void __launch_bounds__(kThreads, 1) gqa_prefill_kernel(GqaArgs a, int ps_log2) {
  __shared__ __attribute__((aligned(1024))) PreSmem<KV_DT> sm;
  const int npre = a.counters[3];
  const int home = blockIdx.x % kXcds;
  for (;;) {
    if (threadIdx.x == 0) {
      int t = -1;
      for (int k = 0; k < kXcds && t < 0; ++k) {
        const int x = (home + k) % kXcds;
        const int b = (int)((int64_t)npre * x / kXcds), e = (int)((int64_t)npre * (x + 1) / kXcds);
        if (b >= e) continue;
        const int i = atomicAdd(&a.counters[kXcdCursor0 + x], 1);
        if (b + i < e) t = b + i;
      }
      sm.tile = t;
    }
    __syncthreads();
    const int ti = sm.tile;
    __syncthreads();
    if (ti < 0) break;
    prefill_tile<KV_DT, CAP>(a, a.tiles[ti], sm, ps_log2);
    __syncthreads();
  }
}

}  // namespace

int gqa_prefill_rows() { return kWaves * kRowsPerWave; }

bool gqa_prefill_supported(int q_dtype, int kv_dtype, int head_dim, int group, int page_size) {
  return (q_dtype == DT_BF16 || q_dtype == DT_FP8) &&
         (kv_dtype == DT_BF16 || kv_dtype == DT_FP8 || kv_dtype == DT_INT8) && head_dim == kD &&
         group >= 1 && group <= kWaves * kRowsPerWave && page_size >= 8 &&
         (page_size & (page_size - 1)) == 0;
}

hipError_t launch_gqa_prefill(const GqaArgs& a, int ps_log2, int grid, hipStream_t stream) {
  const bool cap = a.soft_cap != 0.f;
#define RPA_PRE_LAUNCH(DT, CAP) \
  hipLaunchKernelGGL((gqa_prefill_kernel<DT, CAP>), dim3(grid), dim3(kThreads), 0, stream, a, ps_log2)
  if (a.kv_dtype == DT_BF16) {
    if (cap)
      RPA_PRE_LAUNCH(DT_BF16, true);
    else
      RPA_PRE_LAUNCH(DT_BF16, false);
  } else if (a.kv_dtype == DT_INT8) {
    if (cap)
      RPA_PRE_LAUNCH(DT_INT8, true);
    else
      RPA_PRE_LAUNCH(DT_INT8, false);
  } else {
    if (cap)
      RPA_PRE_LAUNCH(DT_FP8, true);
    else
      RPA_PRE_LAUNCH(DT_FP8, false);
  }
#undef RPA_PRE_LAUNCH
  return hipGetLastError();
}

}  // namespace rpa
