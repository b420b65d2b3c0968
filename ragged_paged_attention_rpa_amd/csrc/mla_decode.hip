// MLA latent attention on gfx950 [MLA v1 page: mla_ragged_paged_attention,
// ref_mla_ragged_paged_attention, flash_attention; update_kv_cache for the
// scatter of the step's new tokens, which here happens inside the attention
// launch].
//
// Every head of a query token attends the same 576-wide latent row per key:
// K_t = [kv_c_t (512) || k_pe_t (64)], V_t = kv_c_t.
//
// Launches, with no host synchronisation:
//   1. mla_plan_kernel   lays every query token's visible key range (one copy
//      per group of 128 heads) end to end and cuts that key space into
//      kMlaGrid equal shares; a token's range that crosses a cut becomes
//      several pieces. Workgroup w takes the pieces of share w, so every
//      workgroup streams the same number of keys whatever the lengths.
//   2. mla_tile_kernel   one workgroup per share: four waves for 128 heads,
//      on v_mfma_f32_32x32x16_bf16. Scores S^T = K Q^T are split by heads
//      (wave w: heads 32w .. 32w+31, Q^T in VGPRs) and so is the softmax;
//      each wave hands its softmax weights to the others through LDS, and
//      O^T += V^T P^T is split by value dims (wave w: dims 128w .. 128w+127
//      of all 128 heads, O^T in AGPRs), so one transposed V read feeds four
//      MFMAs. Keys move through a four-stage LDS ring of 32-key blocks (36 KB
//      each) filled by global_load_lds_dwordx4. The block loop is software
//      pipelined: while the matrix cores multiply the scores of block j + 1,
//      the softmax of block j runs between those MFMAs; then block j's
//      weights are exchanged and its PV products added. Blocks j + 2 and
//      j + 3 are in flight meanwhile. Pieces that cover a whole token write
//      the output; the others write (m, l, O / l) partials.
//   3. mla_merge_kernel  combines the partials of each token that was cut,
//      with the rescaling algebra of the page's flash_attention.
// When the call brings the step's new tokens (new_kv_c, new_k_pe), the keys
// at positions kv_len - q_len .. kv_len - 1 are read from those buffers, and
// the piece that holds a token's own position copies that token's row into
// its cache slot (k_pe padded with zeros): no separate scatter launch, and no
// piece reads a slot that is being written.
#include "rpa_device.h"
#include "rpa_internal.h"

#include <type_traits>

namespace rpa {

namespace {

constexpr int kDl = 512;                       // latent (and value) width
constexpr int kDr = 64;                        // rope width
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveHeads = 32;
constexpr int kHeadsPerWg = kWaves * kWaveHeads;  // 128
constexpr int kBlk = 32;                       // keys per LDS stage
constexpr int kStages = 4;
constexpr int kKvcBytes = kDl * 2;             // 1024: latent part of a key
constexpr int kKpeBytes = kDr * 2;             // 128: rope part of a key
constexpr int kKpeOff = kBlk * kKvcBytes;      // rope parts follow the latent parts
constexpr int kStageBytes = kBlk * (kKvcBytes + kKpeBytes);  // 36864
constexpr int kSteps = (kDl + kDr) / 16;       // 36 k-steps of 32x32x16
constexpr int kDt = kDl / 32;                  // 16 output tiles of 32 dims
constexpr int kDtPerWave = kDt / kWaves;       // 4: a wave's 128 value dims
constexpr int kDmaPerWave = 9;                 // per stage: 8 latent rows + 8 rope parts
constexpr int kPageWin = 1024;                 // page ids cached in LDS

__device__ __attribute__((aligned(16))) const uint8_t kZeroLatent[kKvcBytes + kKpeBytes] = {0};

// Chunk q (0..63) of a key's latent part sits at q ^ swz(key) (key = index in
// the 32-key stage). Bits 2..3 are key % 4 and bits 0..1 are (key / 4) % 4:
// one-to-one on 16 consecutive keys (the K reads: one chunk of 16 keys per
// 16-lane quarter) and the four chunk blocks {0..3} ^ swz of an aligned quad
// of keys are disjoint (the transposed V reads: 4 chunks of 4 keys per
// 32-lane half).
__device__ __forceinline__ int swz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }
// Rope chunk q (0..7) sits at q ^ swz_pe(key): one-to-one on the eight keys
// of either parity among 16 consecutive keys.
__device__ __forceinline__ int swz_pe(int key) { return ((key >> 1) & 7) ^ ((key & 1) << 2); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

struct SeqInfo {
  int cu0, q_len, kv_len, kv_cap;
};

__device__ __forceinline__ SeqInfo seq_info(const MlaArgs& a, int seq) {
  SeqInfo s;
  s.cu0 = a.cu_q_lens[seq];
  s.q_len = a.cu_q_lens[seq + 1] - s.cu0;
  s.kv_len = a.kv_lens[seq];
  s.kv_cap = min(s.kv_len, a.pages_per_seq * a.page_size);
  return s;
}

// Visible key range [lo, hi) of query token tok_rel of a sequence: causal
// offset kv_len - q_len, optional sliding window.
__device__ __forceinline__ void key_range(const MlaArgs& a, const SeqInfo& s, int tok_rel, int* lo,
                                          int* hi) {
  const int pos = s.kv_len - s.q_len + tok_rel;
  *lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;
  *hi = max(0, min(pos + 1, s.kv_cap));
  if (*lo > *hi) *lo = *hi;
}

__device__ __forceinline__ int num_seqs_clamped(const MlaArgs& a) {
  return clampi(*a.num_seqs, 0, a.max_num_seqs);
}

__device__ __forceinline__ int head_groups(const MlaArgs& a) {
  return (a.num_heads + kHeadsPerWg - 1) / kHeadsPerWg;
}

// Inclusive block scan of one 64-bit value per thread (256 threads).
__device__ long long block_scan_incl(long long v, long long* sh, long long* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const long long x = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  const long long r = sh[tid];
  *total = sh[kThreads - 1];
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ plan ----
// Piece record (two int4): {seq, token, lo, hi}, {head group, partial slot or
// -1 for a whole token, writes its token's new row (0/1), share}.
__global__ void __launch_bounds__(kThreads) mla_plan_kernel(MlaArgs a) {
  __shared__ long long sh[kThreads];
  __shared__ long long sh2[kThreads];
  const int tid = threadIdx.x;
  const int ns = num_seqs_clamped(a);
  const int T = ns > 0 ? clampi(a.cu_q_lens[ns], 0, a.max_num_tokens) : 0;
  const int HG = head_groups(a);
  const bool fused_update = a.new_kv_c != nullptr;

  // Pass 1: visible keys per token, inclusive prefix over tokens.
  long long run = 0;
  for (int base = 0; base < T; base += kThreads) {
    const int t = base + tid;
    long long n = 0;
    if (t < T) {
      const int seq = find_seq(a.cu_q_lens, ns, t);
      if (seq >= 0) {
        const SeqInfo s = seq_info(a, seq);
        int lo, hi;
        key_range(a, s, t - s.cu0, &lo, &hi);
        n = hi - lo;
      }
    }
    long long tot;
    const long long incl = block_scan_incl(n, sh, &tot);
    if (t < T) a.kpre[t] = run + incl;
    run += tot;
  }
  __threadfence_block();
  __syncthreads();
  const long long ktot = run;
  const long long space = ktot * HG;
  long long q = (space + kMlaGrid - 1) / kMlaGrid;
  q = (q + kBlk - 1) / kBlk * kBlk;
  if (q < a.min_share) q = a.min_share;

  // Pass 2: pieces per (head group, token) item, in key-space order.
  const int items = T * HG;
  long long prun = 0, srun = 0;
  for (int base = 0; base < items; base += kThreads) {
    const int i = base + tid;
    long long c = 0, sl = 0;
    long long S = 0, E = 0;
    int seq = -1, t = 0, hg = 0, lo = 0;
    if (i < items) {
      hg = i / T;
      t = i - hg * T;
      const long long pre = t > 0 ? a.kpre[t - 1] : 0;
      E = (long long)hg * ktot + a.kpre[t];
      S = (long long)hg * ktot + pre;
      c = E > S ? (E - 1) / q - S / q + 1 : 1;
      sl = c > 1 ? c : 0;
      seq = find_seq(a.cu_q_lens, ns, t);
      if (seq >= 0) {
        const SeqInfo s = seq_info(a, seq);
        int hi;
        key_range(a, s, t - s.cu0, &lo, &hi);
      }
    }
    long long ptot, stot;
    const long long pincl = block_scan_incl(c, sh, &ptot);
    const long long sincl = block_scan_incl(sl, sh2, &stot);
    if (i < items) {
      const long long poff = prun + pincl - c;
      const long long soff = srun + sincl - sl;
      const int64_t ti = (int64_t)hg * a.max_num_tokens + t;  // the merge's item index
      a.tok_slot[2 * ti] = c > 1 ? (int)soff : -1;
      a.tok_slot[2 * ti + 1] = (int)c;
      int write_tok = 0;
      if (fused_update && hg == 0 && seq >= 0) write_tok = 1;
      for (long long j = 0; j < c; ++j) {
        const long long pidx = poff + j;
        if (pidx >= a.piece_capacity) break;
        long long ps = S, pe = E;
        if (E > S) {
          ps = S / q * q + j * q;
          if (ps < S) ps = S;
          pe = (S / q + j + 1) * q;
          if (pe > E) pe = E;
        }
        int share = (int)(ps / q);
        if (share >= kMlaGrid) share = kMlaGrid - 1;
        const int plo = lo + (int)(ps - S), phi = lo + (int)(pe - S);
        int4 r0, r1;
        r0.x = seq;
        r0.y = t;
        r0.z = plo;
        r0.w = phi;
        r1.x = hg;
        r1.y = c > 1 ? (int)(soff + j) : -1;
        r1.z = (write_tok && j == c - 1) ? 1 : 0;  // the piece holding the token's own key
        r1.w = share;
        reinterpret_cast<int4*>(a.pieces)[2 * pidx] = r0;
        reinterpret_cast<int4*>(a.pieces)[2 * pidx + 1] = r1;
      }
    }
    prun += ptot;
    srun += stot;
  }
  __threadfence();
  __syncthreads();
  const int npieces = (int)(prun < a.piece_capacity ? prun : a.piece_capacity);
  // Pass 3: first piece of each share (pieces are ordered by share).
  for (int w = tid; w <= kMlaGrid; w += kThreads) {
    int lo_i = 0, hi_i = npieces;
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i) >> 1;
      const int sw = reinterpret_cast<const int4*>(a.pieces)[2 * mid + 1].w;
      if (sw < w)
        lo_i = mid + 1;
      else
        hi_i = mid;
    }
    a.wg_start[w] = lo_i;
  }
  if (tid == 0) {
    a.counters[0] = npieces;
    a.counters[1] = (int)(srun < (1ll << 30) ? srun : (1ll << 30));
  }
}

// ---- O^T accumulator in AGPRs ------------------------------------------------
// A wave's O^T (32 heads x 512 dims, fp32) is 16 tiles of 16 registers that
// must stay in the AGPR file (the VGPRs hold Q^T, S and the operands). The PV
// MFMAs are inline asm with an "a" (AGPR) operand, which keeps the tiles'
// values in AGPRs between statements; the rare rescale and the final read go
// through acc_read / acc_write. The compiler does not see MFMAs inside asm, so
// the wait states they need are explicit: 24 between an MFMA result and a
// v_accvgpr_read (acc_read) and mfma_agpr_fence() after writes before the
// next MFMA reads the tile. Their A and B operands come straight from LDS
// reads (no VALU write precedes them).
#define RPA_WAIT24 "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"

__device__ __forceinline__ void acc_mfma(floatx16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// acc = x (a VGPR tuple copied into the tile's AGPRs).
__device__ __forceinline__ void acc_write(floatx16& acc, const floatx16& x) {
  asm volatile("" : "=a"(acc) : "0"(x));
}

#define RPA_ACC_CASES(X)                                                        \
  X(0, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15)                    \
  X(1, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31)          \
  X(2, 32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47)          \
  X(3, 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63)          \
  X(4, 64, 65, 66, 67, 68, 69, 70, 71, 72, 73, 74, 75, 76, 77, 78, 79)          \
  X(5, 80, 81, 82, 83, 84, 85, 86, 87, 88, 89, 90, 91, 92, 93, 94, 95)          \
  X(6, 96, 97, 98, 99, 100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111) \
  X(7, 112, 113, 114, 115, 116, 117, 118, 119, 120, 121, 122, 123, 124, 125, 126, 127) \
  X(8, 128, 129, 130, 131, 132, 133, 134, 135, 136, 137, 138, 139, 140, 141, 142, 143) \
  X(9, 144, 145, 146, 147, 148, 149, 150, 151, 152, 153, 154, 155, 156, 157, 158, 159) \
  X(10, 160, 161, 162, 163, 164, 165, 166, 167, 168, 169, 170, 171, 172, 173, 174, 175) \
  X(11, 176, 177, 178, 179, 180, 181, 182, 183, 184, 185, 186, 187, 188, 189, 190, 191) \
  X(12, 192, 193, 194, 195, 196, 197, 198, 199, 200, 201, 202, 203, 204, 205, 206, 207) \
  X(13, 208, 209, 210, 211, 212, 213, 214, 215, 216, 217, 218, 219, 220, 221, 222, 223) \
  X(14, 224, 225, 226, 227, 228, 229, 230, 231, 232, 233, 234, 235, 236, 237, 238, 239) \
  X(15, 240, 241, 242, 243, 244, 245, 246, 247, 248, 249, 250, 251, 252, 253, 254, 255)

// Tile dt copied into VGPRs v0..v15, after the wait an MFMA result needs.
// The tile is read from a[16dt .. 16dt+15], where the allocator keeps it
// (were it elsewhere, the constraint makes the compiler move it there first).
__device__ __forceinline__ floatx16 acc_read(int dt, const floatx16& acc) {
  floatx16 x = {};
  switch (dt) {
#define RPA_X(D, r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15)      \
  case D:                                                                                 \
    asm volatile(RPA_WAIT24                                                               \
                 "v_accvgpr_read_b32 v0, a" #r0 "\n\tv_accvgpr_read_b32 v1, a" #r1 "\n\t"  \
                 "v_accvgpr_read_b32 v2, a" #r2 "\n\tv_accvgpr_read_b32 v3, a" #r3 "\n\t"  \
                 "v_accvgpr_read_b32 v4, a" #r4 "\n\tv_accvgpr_read_b32 v5, a" #r5 "\n\t"  \
                 "v_accvgpr_read_b32 v6, a" #r6 "\n\tv_accvgpr_read_b32 v7, a" #r7 "\n\t"  \
                 "v_accvgpr_read_b32 v8, a" #r8 "\n\tv_accvgpr_read_b32 v9, a" #r9 "\n\t"  \
                 "v_accvgpr_read_b32 v10, a" #r10 "\n\tv_accvgpr_read_b32 v11, a" #r11 "\n\t" \
                 "v_accvgpr_read_b32 v12, a" #r12 "\n\tv_accvgpr_read_b32 v13, a" #r13 "\n\t" \
                 "v_accvgpr_read_b32 v14, a" #r14 "\n\tv_accvgpr_read_b32 v15, a" #r15      \
                 : "={v[0:15]}"(x)                                                         \
                 : "{a[" #r0 ":" #r15 "]}"(acc));                                          \
    break;
    RPA_ACC_CASES(RPA_X)
#undef RPA_X
    default: break;
  }
  return x;
}

// Workgroup barrier after this wave's LDS writes have landed; unlike
// __syncthreads() it leaves the in-flight LDS-DMA loads alone.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Fixes where a value is computed: the empty asm uses it and may change it,
// and volatile asm statements keep their order, so the work that produces it
// stays between the MFMAs around this point instead of being sunk to its use.
template <typename T>
__device__ __forceinline__ void pin_here(T& x) {
  asm volatile("" : "+v"(x));
}

// ------------------------------------------------------------------ tile ----
struct MlaSmem {
  char stage[kStages][kStageBytes];
  int pages[kPageWin];
  u32x4 pex[kWaves][2][64];   // softmax weights P^T of each wave's 32 heads (MFMA B operands)
  float alpha[kWaves][32];    // per head: rescale of its accumulators this stage
  float lsum[kWaves][32];     // per head: row sum at the end of a piece
  alignas(16) int rescale[kWaves];  // per head tile: some head moved its reference
};
static_assert(sizeof(MlaSmem) <= 160 * 1024, "MLA LDS budget");

// One piece: the 128 heads of head group hg of one query token over keys
// [lo, hi). CAP: the soft cap is set (a compile-time switch: as a run-time
// flag the compiler if-converts the logit map, and every block then pays for
// the capped map's transcendentals).
template <bool CAP>
__device__ void process_piece(const MlaArgs& a, int4 r0, int4 r1, MlaSmem& sm, int ps_log2) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 5;
  const int seq = __builtin_amdgcn_readfirstlane(r0.x);
  const int tok = __builtin_amdgcn_readfirstlane(r0.y);
  const int lo = __builtin_amdgcn_readfirstlane(r0.z);
  const int hi = __builtin_amdgcn_readfirstlane(r0.w);
  const int hg = __builtin_amdgcn_readfirstlane(r1.x);
  const int slot = __builtin_amdgcn_readfirstlane(r1.y);
  const bool writes_new = r1.z != 0;
  if (seq < 0) return;  // a token no sequence owns (inconsistent metadata): nothing to do
  const SeqInfo s = seq_info(a, seq);
  const int new_start = s.kv_len - s.q_len;  // positions >= this are the step's new tokens
  const bool redirect = a.new_kv_c != nullptr;
  const int32_t* table = a.page_indices + (int64_t)seq * a.pages_per_seq;
  const int P = a.total_num_pages;
  const int ps_mask = (1 << ps_log2) - 1;
  const int64_t kvc_row = (int64_t)a.kvc_stride * 2, kpe_row = (int64_t)a.kpe_stride * 2;

  // The step's new row of this token goes to its cache slot (bitwise, k_pe
  // padded with zeros); every reader of that position this launch takes it
  // from new_kv_c / new_k_pe instead, so the write races with no read.
  if (writes_new) {
    const int pos = new_start + (tok - s.cu0);
    const int lp = pos >> ps_log2;
    const int page = (pos >= 0 && lp < a.pages_per_seq) ? table[lp] : -1;
    if (page >= 0 && page < P) {
      const int64_t row = ((int64_t)page << ps_log2) + (pos & ps_mask);
      char* dkvc = (char*)a.cache_kv_c + row * kvc_row;
      char* dkpe = (char*)a.cache_k_pe + row * kpe_row;
      const char* skvc = (const char*)a.new_kv_c + (int64_t)tok * kKvcBytes;
      const char* skpe = (const char*)a.new_k_pe + (int64_t)tok * kKpeBytes;
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int i = tid; i < (int)(kvc_row >> 4); i += kThreads)
        reinterpret_cast<u32x4*>(dkvc)[i] =
            i < kKvcBytes / 16 ? reinterpret_cast<const u32x4*>(skvc)[i] : z;
      for (int i = tid; i < (int)(kpe_row >> 4); i += kThreads)
        reinterpret_cast<u32x4*>(dkpe)[i] =
            i < kKpeBytes / 16 ? reinterpret_cast<const u32x4*>(skpe)[i] : z;
    }
  }

  // Every wave runs the whole block loop, also when its 32 heads are all past
  // num_heads (on zero queries; nothing of theirs is stored): it owns a
  // quarter of every head's value dims and of every stage's loads.
  const int head = hg * kHeadsPerWg + wave * kWaveHeads + (lane & 31);
  const bool head_ok = head < a.num_heads;

  const int kb0 = lo & ~(kBlk - 1);
  const int nst = hi > kb0 ? (hi - kb0 + kBlk - 1) / kBlk : 0;
  int pwin = kb0 >> ps_log2;
  for (int i = tid; i < kPageWin; i += kThreads) {
    const int lp = pwin + i;
    sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
  }
  __syncthreads();

  // Sources of this wave's eight keys 8*wave + lane/8 of stage j: 64-bit row
  // addresses of the latent and rope parts (the zero row outside [lo, hi)).
  // Called by all waves at the same point: a page-window refill synchronises.
  auto prep = [&](int j, uint64_t* kvc, uint64_t* kpe) {
    const int kb = kb0 + j * kBlk;
    if (((kb + kBlk - 1) >> ps_log2) - pwin >= kPageWin) {
      wg_barrier();
      pwin = kb >> ps_log2;
      for (int i = tid; i < kPageWin; i += kThreads) {
        const int lp = pwin + i;
        sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
      }
      __syncthreads();
    }
    const int key = kb + 8 * wave + (lane >> 3);
    uint64_t av = (uint64_t)(uintptr_t)kZeroLatent;
    uint64_t bv = av + kKvcBytes;
    if (key >= lo && key < hi) {
      if (redirect && key >= new_start) {
        const int64_t nt = s.cu0 + (key - new_start);
        av = (uint64_t)(uintptr_t)((const char*)a.new_kv_c + nt * kKvcBytes);
        bv = (uint64_t)(uintptr_t)((const char*)a.new_k_pe + nt * kKpeBytes);
      } else {
        const int page = sm.pages[(key >> ps_log2) - pwin];
        if (page >= 0 && page < P) {
          const int64_t row = ((int64_t)page << ps_log2) + (key & ps_mask);
          av = (uint64_t)(uintptr_t)((const char*)a.cache_kv_c + row * kvc_row);
          bv = (uint64_t)(uintptr_t)((const char*)a.cache_k_pe + row * kpe_row);
        }
      }
    }
    *kvc = av;
    *kpe = bv;
  };
  // DMA instruction k (0..8) of this wave for a stage at LDS address st:
  // k < 8 moves the latent part of key 8*wave + k (one 16-byte chunk per lane,
  // chunk q to position q ^ swz); k = 8 the rope parts of the eight keys.
  auto dma = [&](uint32_t st, uint64_t kvc, uint64_t kpe, int k) {
    if (k < 8) {
      const int key = 8 * wave + k;
      const uint32_t blo = __builtin_amdgcn_readlane((uint32_t)kvc, 8 * k);
      const uint32_t bhi = __builtin_amdgcn_readlane((uint32_t)(kvc >> 32), 8 * k);
      const void* base = (const void*)(uintptr_t)(((uint64_t)bhi << 32) | blo);
      dma_b128_s(base, xor_here((uint32_t)lane << 4, (uint32_t)(swz(key) << 4)),
                 __builtin_amdgcn_readfirstlane(st + (uint32_t)key * kKvcBytes));
    } else {
      const int key = 8 * wave + (lane >> 3);
      const char* src = (const char*)(uintptr_t)kpe + (((lane & 7) ^ swz_pe(key)) << 4);
      dma_b128(src, __builtin_amdgcn_readfirstlane(st + (uint32_t)(kKpeOff + wave * 1024)));
    }
  };

  const uint32_t st_base = lds_addr(sm.stage[0]);
  auto stage_addr = [&](int j) -> uint32_t { return st_base + (uint32_t)((j & (kStages - 1)) * kStageBytes); };

  // Prologue: the first two stages' loads go out before the queries'.
  {
#pragma unroll 1
    for (int j = 0; j < kStages - 2; ++j) {
      if (j >= nst) break;
      uint64_t kvc, kpe;
      prep(j, &kvc, &kpe);
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) dma(stage_addr(j), kvc, kpe, k);
    }
  }

  // Q^T operand: lane l holds head l%32; k-step s < 32 covers latent chunk
  // 32c + s (dims 256c + 8s .. +7), k-step 32 + m rope chunk 2m + c.
  u32x4 qv[kSteps];
  {
    const uint16_t* qn = (const uint16_t*)a.ql_nope + ((int64_t)tok * a.num_heads + head) * kDl;
    const uint16_t* qr = (const uint16_t*)a.q_pe + ((int64_t)tok * a.num_heads + head) * kDr;
#pragma unroll
    for (int st = 0; st < 32; ++st)
      qv[st] = head_ok ? *reinterpret_cast<const u32x4*>(qn + 256 * c + 8 * st) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < 4; ++m)
      qv[32 + m] = head_ok ? *reinterpret_cast<const u32x4*>(qr + 16 * m + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }
  drain_vmem_before_loop();

  // O^T accumulators of this wave: [dim tile d of its 128 dims][head tile h].
  floatx16 acc[kDtPerWave][kWaves];
  {
    floatx16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
#pragma unroll
    for (int d = 0; d < kDtPerWave; ++d)
#pragma unroll
      for (int h = 0; h < kWaves; ++h) acc_write(acc[d][h], z);
  }
  mfma_agpr_fence();
  float m_run = -INFINITY, l_run = 0.f;

  constexpr bool capped = CAP;
  const float c1 = capped ? 2.f * kLog2e * a.score_scale / a.soft_cap : a.score_scale * kLog2e;
  const float c2 = a.soft_cap * kLog2e, c3 = 2.f * a.soft_cap * kLog2e;
  // A masked key's raw score is -inf (mask_pass) and its logit stays -inf.
  auto logit = [&](float sraw) -> float {
    if (!capped) return sraw * c1;
    const float x = c2 - c3 * __builtin_amdgcn_rcpf(fast_exp2(sraw * c1) + 1.f);
    return sraw == -INFINITY ? -INFINITY : x;
  };

  // Lane operand offsets within a stage.
  const int kk = lane & 31;
  const uint32_t klat = (uint32_t)(kk * kKvcBytes + 512 * c + (swz(kk) << 4));
  const uint32_t krope = (uint32_t)(kKpeOff + kk * kKpeBytes + ((c ^ swz_pe(kk)) << 4));
  uint32_t vlo, vhi;
  {
    const int jj = lane & 15;
    const int x = 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
    const int k_lo = 4 * c + (jj >> 2), k_hi = k_lo + 8;
    vlo = (uint32_t)(k_lo * kKvcBytes + ((x ^ swz(k_lo)) << 4) + 8 * (jj & 1));
    vhi = (uint32_t)(k_hi * kKvcBytes + ((x ^ swz(k_hi)) << 4) + 8 * (jj & 1));
  }

  // Software pipeline over the stages. Iteration j (0 .. nst - 1):
  //   S^T(j+1) = K Q^T on stage j + 1: a plain chain of MFMAs with its K
  //   reads (the loads of stage j + 3 go out at its first step);
  //   O^T += V^T P^T(j) on stage j, with the online softmax of S(j+1) spread
  //   between those MFMAs (the PV MFMAs keep their accumulators in AGPRs, so
  //   the VALU work beside them costs little issue time);
  //   after a barrier (every wave is done with P(j)), P(j+1) and its rescale
  //   factors are published in LDS for iteration j + 1.
  // Iteration -1 computes S(0), its softmax and P(0) alone. Stage buffers in
  // use during iteration j: j (PV), j + 1 (QK), j + 2 (in flight), j + 3
  // (loads issued during the QK).
  floatx16 sn;  // S^T of the next stage, softmaxed in place

  // K operand of k-step st from the per-stage bases kl = stage + klat and
  // kp = stage + krope: stage addresses are multiples of 512 bytes, so the
  // column XOR (bits 4..8, or 5..6 for the rope part) commutes with adding
  // the stage address and each read costs one XOR.
  auto kread = [&](uint32_t kl, uint32_t kp, int st) -> u32x4 {
    return st < 32 ? lds_read_b128(xor_here(kl, (uint32_t)(st << 4)))
                   : lds_read_b128(xor_here(kp, (uint32_t)((st - 32) << 5)));
  };
  static_assert(kStageBytes % 512 == 0, "stage bases must leave the swizzle bits alone");

  auto qk = [&](uint32_t qst, uint32_t nxt, bool more, uint64_t nkvc, uint64_t nkpe) {
    constexpr int kAheadK = 4;  // K reads run four k-steps ahead of their MFMAs
    u32x4 kr[kAheadK];
    const uint32_t kl = qst + klat, kp = qst + krope;
#pragma unroll
    for (int i = 0; i < kAheadK; ++i) kr[i] = kread(kl, kp, i);
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[r] = 0.f;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      u32x4 kf = kr[st % kAheadK];
      pin_after(kf);
      sn = mfma_32x32x16(as_bf16x8(kf), as_bf16x8(qv[st]), sn);
      if (st + kAheadK < kSteps) kr[st % kAheadK] = kread(kl, kp, st + kAheadK);
      // Stage j + 3's loads go out together after the first MFMA: their
      // addresses then die at once (spreading them keeps them live across
      // the k-steps, which the register budget does not allow).
      if (more && st == 0) {
#pragma unroll
        for (int k = 0; k < kDmaPerWave; ++k) dma(nxt, nkvc, nkpe, k);
      }
    }
  };

  // Raw scores of keys outside [lo, hi) become -inf, for a stage whose first
  // key is kb (register r holds key kb + 8(r/4) + 4c + r%4). Run before the
  // softmax of a stage that crosses lo or hi.
  auto mask_pass = [&](int kb) {
    const uint32_t span = (uint32_t)(hi - lo);
    const int base = kb + 4 * c - lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool vis = (uint32_t)(base + 8 * (r >> 2) + (r & 3)) < span;
      sn[r] = vis ? sn[r] : -INFINITY;
    }
  };

  // Softmax item t (0 .. 33) of the scores in sn: logits and the block max at
  // t = 0..15, the reference update at 16, the weights at 17..32, their bf16
  // packing at 33. The input is pinned where the item starts and the result
  // where it ends, so the item's VALU work stays between the MFMAs around it.
  struct SoftState {
    float mblk, mref, psum, alpha;
    int moved;
  };
  auto soft_item = [&](int t, SoftState& ss, u32x4 (&pb)[2]) {
    if (t < 16) {
      float x = sn[t];
      pin_here(x);
      x = logit(x);
      pin_here(x);
      sn[t] = x;
      ss.mblk = fmaxf(ss.mblk, x);
    } else if (t == 16) {
      // Lane l ^ 32 holds the other 16 keys of the same head.
      float mb = ss.mblk;
      pin_here(mb);
      mb = wave_max_xor<32>(mb);
      const bool need = mb > m_run + kLazyTau;
      ss.moved = __builtin_amdgcn_readfirstlane(wave_any(need) ? 1 : 0);
      ss.alpha = need ? fast_exp2(m_run - mb) : 1.f;  // rows not moving keep scale 1
      l_run *= ss.alpha;
      m_run = need ? mb : m_run;
      ss.mref = m_run == -INFINITY ? 0.f : m_run;  // no visible key yet: weights 0
      pin_here(ss.mref);
    } else if (t <= 32) {
      const int r = t - 17;
      float x = sn[r];
      pin_here(x);
      float e = fast_exp2(x - ss.mref);
      pin_here(e);
      sn[r] = e;
      ss.psum += e;
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[u][i] = pack_bf16x2(sn[8 * u + 2 * i], sn[8 * u + 2 * i + 1]);
      pin_here(pb[0]);
      pin_here(pb[1]);
      l_run += ss.psum;
    }
  };
  auto publish = [&](const u32x4 (&pb)[2], const SoftState& ss) {
    sm.pex[wave][0][lane] = pb[0];
    sm.pex[wave][1][lane] = pb[1];
    if (lane < 32) sm.alpha[wave][lane] = ss.alpha;
    if (lane == 0) sm.rescale[wave] = ss.moved;
  };

  // O^T += V^T P^T(j) for dims 128*wave .. +127 of all 128 heads (k-step u
  // takes keys 16u + 4c + {0..3, 8..11}; each V^T operand feeds the four head
  // tiles), with the softmax items of the scores in sn after the MFMAs. (One
  // copy of this code serves every iteration: more copies in the loop body
  // make the register allocator spill.)
  auto pv_soft = [&](int j, u32x4 (&pb)[2], SoftState& ss) {
    // Per-stage bases as for K: the dims XOR (bits 6..9) commutes with adding
    // the stage address, and the 16-key step is the read's offset field.
    const uint32_t cur = stage_addr(j);
    const uint32_t vlb = cur + vlo, vhb = cur + vhi;
    auto vread = [&](int u, int d) -> u32x4 {
      const uint32_t dsel = (uint32_t)((kDtPerWave * wave + d) << 6);
      const uint32_t ub = (uint32_t)(u * 16 * kKvcBytes);
      const u32x2 v0 = lds_read_tr16(xor_here(vlb, dsel) + ub);
      const u32x2 v1 = lds_read_tr16(xor_here(vhb, dsel) + ub);
      return u32x4{v0[0], v0[1], v1[0], v1[1]};
    };
    // The flags, the first weights and the first V^T operand are read
    // together.
    const int4 flags = *reinterpret_cast<const int4*>(sm.rescale);
    u32x4 pbh[kWaves];
#pragma unroll
    for (int h = 0; h < kWaves; ++h) pbh[h] = sm.pex[h][0][lane];
    u32x4 vf = vread(0, 0);

    // Rescale the accumulators of head tiles whose reference moved (the
    // common case skips it all).
    const int rs_any = __builtin_amdgcn_readfirstlane(flags.x | flags.y | flags.z | flags.w);
    if (rs_any) {
#pragma unroll
      for (int h = 0; h < kWaves; ++h) {
        const int rs_h = h == 0 ? flags.x : h == 1 ? flags.y : h == 2 ? flags.z : flags.w;
        if (__builtin_amdgcn_readfirstlane(rs_h)) {
          const float al = sm.alpha[h][lane & 31];
#pragma unroll
          for (int d = 0; d < kDtPerWave; ++d) {
            floatx16 x = acc_read(d * kWaves + h, acc[d][h]);
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] *= al;
            acc_write(acc[d][h], x);
          }
          mfma_agpr_fence();
        }
      }
    }

#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1) {
#pragma unroll
        for (int h = 0; h < kWaves; ++h) pbh[h] = sm.pex[h][1][lane];
      }
#pragma unroll
      for (int d = 0; d < kDtPerWave; ++d) {
        const int n = u * kDtPerWave + d + 1;
        u32x4 vn = {0u, 0u, 0u, 0u};
        if (n < 2 * kDtPerWave) vn = vread(n / kDtPerWave, n % kDtPerWave);
        pin_after(vf);
#pragma unroll
        for (int h = 0; h < kWaves; ++h) {
          acc_mfma(acc[d][h], vf, pbh[h]);
          const int t = 4 * (kDtPerWave * u + d) + h;  // 0 .. 31
          soft_item(t, ss, pb);
          if (t == 31) {
            soft_item(32, ss, pb);
            soft_item(33, ss, pb);
          }
        }
        vf = vn;
      }
    }
  };

  // Iteration -1: S(0), its softmax and P(0).
  auto pre_stage = [&](int j, bool has_qk, bool& more, uint64_t& nkvc, uint64_t& nkpe) {
    // Stage j + 1 landed once this wave's loads of stage j + 2 are all that
    // is outstanding (the last iteration has none left). The barrier (after
    // this wave's LDS writes of P(j) have completed) makes every wave's part
    // visible, and every wave is past PV(j - 1): stage j - 1's buffer is free
    // for stage j + 3.
    if (has_qk && j + 2 < nst)
      wait_vmcnt<kDmaPerWave>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    more = j + kStages - 1 < nst;
    nkvc = 0;
    nkpe = 0;
    if (more) prep(j + kStages - 1, &nkvc, &nkpe);
  };
  auto soft_alone = [&](u32x4 (&pb)[2], SoftState& ss) {
#pragma unroll
    for (int t = 0; t < 34; ++t) soft_item(t, ss, pb);
  };
  if (nst > 0) {
    bool more;
    uint64_t nkvc, nkpe;
    pre_stage(-1, true, more, nkvc, nkpe);
    qk(stage_addr(0), stage_addr(kStages - 2), more, nkvc, nkpe);
    u32x4 pb[2];
    SoftState ss{-INFINITY, 0.f, 0.f, 1.f, 0};
    if (!(kb0 >= lo && kb0 + kBlk <= hi)) mask_pass(kb0);
    soft_alone(pb, ss);
    publish(pb, ss);
  }
#pragma unroll 1
  for (int j = 0; j < nst; ++j) {
    const bool has_qk = j + 1 < nst;
    bool more;
    uint64_t nkvc, nkpe;
    pre_stage(j, has_qk, more, nkvc, nkpe);
    u32x4 pb[2];
    SoftState ss{-INFINITY, 0.f, 0.f, 1.f, 0};
    const int kbn = kb0 + (j + 1) * kBlk;  // first key of stage j + 1
    if (has_qk) {
      qk(stage_addr(j + 1), stage_addr(j + kStages - 1), more, nkvc, nkpe);
      if (!(kbn >= lo && kbn + kBlk <= hi)) mask_pass(kbn);
    }
    // The last iteration has no next stage: its softmax items run on stale
    // scores and everything they produce is dropped.
    const float m_keep = m_run, l_keep = l_run;
    pv_soft(j, pb, ss);
    if (has_qk) {
      // Every wave is done reading P(j) and its rescale factors. (An early
      // exit from the loop here instead makes the register allocator spill.)
      wg_barrier();
      publish(pb, ss);
    } else {
      m_run = m_keep;
      l_run = l_keep;
    }
  }

  // ---- end of piece: every wave needs the row sums of all 128 heads.
  const float l_row = wave_sum_xor<32>(l_run);
  if (lane < 32) sm.lsum[wave][lane] = l_row;
  __syncthreads();
  if (slot >= a.slot_capacity) return;
  // Tile (d, h), register r: dims 128*wave + 32d + 8(r/4) + 4c + r%4 of head
  // 32h + lane%32.
#pragma unroll
  for (int h = 0; h < kWaves; ++h) {
    const int hh = hg * kHeadsPerWg + kWaveHeads * h + (lane & 31);
    const float lh = sm.lsum[h][lane & 31];
    const float inv = lh > 0.f ? a.v_scale / lh : 0.f;
    const bool ok = hh < a.num_heads;
    uint16_t* dst = slot >= 0 ? a.part_acc + ((int64_t)slot * a.num_heads + hh) * kDl
                              : (uint16_t*)a.out + ((int64_t)tok * a.num_heads + hh) * kDl;
#pragma unroll
    for (int d = 0; d < kDtPerWave; ++d) {
      const floatx16 x = acc_read(d * kWaves + h, acc[d][h]);
      if (!ok) continue;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<u32x2*>(dst + 128 * wave + 32 * d + 8 * qd + 4 * c) =
            u32x2{pack_bf16x2(x[4 * qd] * inv, x[4 * qd + 1] * inv),
                  pack_bf16x2(x[4 * qd + 2] * inv, x[4 * qd + 3] * inv)};
    }
  }
  // The head's own wave writes its (m, l) beside a partial.
  if (slot >= 0 && c == 0 && head_ok) {
    float* pm = a.part_ml + ((int64_t)slot * a.num_heads + head) * 2;
    pm[0] = m_run;
    pm[1] = l_row;
  }
}

template <bool CAP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_tile_kernel(MlaArgs a, int ps_log2) {
  __shared__ __attribute__((aligned(1024))) MlaSmem sm;
  const int w = blockIdx.x;
  const int p0 = a.wg_start[w], p1 = a.wg_start[w + 1];
  for (int p = p0; p < p1; ++p) {
    const int4 r0 = reinterpret_cast<const int4*>(a.pieces)[2 * p];
    const int4 r1 = reinterpret_cast<const int4*>(a.pieces)[2 * p + 1];
    process_piece<CAP>(a, r0, r1, sm, ps_log2);
    __syncthreads();
  }
}

// Combines the partials of each (head group, token) that was cut into
// several pieces: thread = (head, 8 dims); weight of piece i is
// l_i * 2^(m_i - M) on its normalised output.
__global__ void __launch_bounds__(kThreads) mla_merge_kernel(MlaArgs a) {
  const int item = blockIdx.x;
  const int T = a.max_num_tokens;
  const int hg = item / T;
  const int tok = item - hg * T;
  const int ns = num_seqs_clamped(a);
  const int Tu = ns > 0 ? clampi(a.cu_q_lens[ns], 0, T) : 0;
  if (tok >= Tu) return;
  const int first = a.tok_slot[2 * item];
  const int cnt = a.tok_slot[2 * item + 1];
  if (first < 0 || cnt <= 1 || first + cnt > a.slot_capacity) return;
  const int t = blockIdx.y * kThreads + threadIdx.x;
  const int head = hg * kHeadsPerWg + (t >> 6);
  const int d0 = (t & 63) * 8;
  if (head >= a.num_heads || (t >> 6) >= kHeadsPerWg) return;
  float M = -INFINITY;
  for (int i = 0; i < cnt; ++i)
    M = fmaxf(M, a.part_ml[((int64_t)(first + i) * a.num_heads + head) * 2]);
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int i = 0; i < cnt; ++i) {
      const float* pm = a.part_ml + ((int64_t)(first + i) * a.num_heads + head) * 2;
      const float w = fast_exp2(pm[0] - M) * pm[1];
      L += w;
      const u32x4 x =
          *reinterpret_cast<const u32x4*>(a.part_acc + ((int64_t)(first + i) * a.num_heads + head) * kDl + d0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo, hi;
        unpack_part(x[k], lo, hi, false);
        o[2 * k] += w * lo;
        o[2 * k + 1] += w * hi;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)tok * a.num_heads + head) * kDl + d0;
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(o[2 * k] * inv, o[2 * k + 1] * inv);
  *reinterpret_cast<u32x4*>(op) = w;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct MlaLayout {
  size_t counters, wg_start, kpre, tok_slot, pieces, part_ml, part_acc, total;
  int piece_capacity, slot_capacity;
};

MlaLayout mla_layout(int max_num_tokens, int num_heads) {
  const int HG = (num_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  MlaLayout L;
  L.piece_capacity = HG * max_num_tokens + kMlaGrid;
  L.slot_capacity = 2 * kMlaGrid;
  size_t off = 0;
  L.counters = off;
  off += align256(64 * sizeof(int32_t));
  L.wg_start = off;
  off += align256((kMlaGrid + 1) * sizeof(int32_t));
  L.kpre = off;
  off += align256((size_t)max_num_tokens * sizeof(long long));
  L.tok_slot = off;
  off += align256((size_t)HG * max_num_tokens * 2 * sizeof(int32_t));
  L.pieces = off;
  off += align256((size_t)L.piece_capacity * 32);
  L.part_ml = off;
  off += align256((size_t)L.slot_capacity * num_heads * 2 * sizeof(float));
  L.part_acc = off;
  off += align256((size_t)L.slot_capacity * num_heads * kDl * sizeof(uint16_t));
  L.total = off;
  return L;
}

}  // namespace

size_t mla_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_heads, int lkv_dim) {
  (void)max_num_seqs;
  (void)lkv_dim;
  return mla_layout(max_num_tokens, num_heads).total;
}

void mla_bind_workspace(MlaArgs& a, void* ws) {
  const MlaLayout L = mla_layout(a.max_num_tokens, a.num_heads);
  char* p = (char*)ws;
  a.counters = (int32_t*)(p + L.counters);
  a.wg_start = (int32_t*)(p + L.wg_start);
  a.kpre = (long long*)(p + L.kpre);
  a.tok_slot = (int32_t*)(p + L.tok_slot);
  a.pieces = (int32_t*)(p + L.pieces);
  a.part_ml = (float*)(p + L.part_ml);
  a.part_acc = (uint16_t*)(p + L.part_acc);
  a.piece_capacity = L.piece_capacity;
  a.slot_capacity = L.slot_capacity;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream) {
  int ps_log2 = 0;
  while ((1 << ps_log2) < a.page_size) ++ps_log2;
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  prof_begin(stream);
  if (a.soft_cap != 0.f)
    hipLaunchKernelGGL(mla_tile_kernel<true>, dim3(kMlaGrid), dim3(kThreads), 0, stream, a, ps_log2);
  else
    hipLaunchKernelGGL(mla_tile_kernel<false>, dim3(kMlaGrid), dim3(kThreads), 0, stream, a, ps_log2);
  prof_end(stream);
  const int hg = (a.num_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(hg * a.max_num_tokens, kHeadsPerWg * 64 / kThreads),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rpa
