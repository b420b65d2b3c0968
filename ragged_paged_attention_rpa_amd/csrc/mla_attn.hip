// MLA latent attention [MLA v1 page: mla_ragged_paged_attention,
// ref_mla_ragged_paged_attention, flash_attention] and sparse MLA-latent
// attention [Sparse page: sparse_mla_attention, _sparse_mla_kernel_chunked_hminor].
//
// Both attend one 576-wide latent row per key, shared by every head: the key
// is the whole row [kv_c (512) || k_pe (64)], the value its first 512 columns.
// Shared core:
//  * keys stream through LDS in blocks of 64 rows x 1152 bytes, moved by
//    global_load_lds_dwordx4 (no register staging) into two stages, so the
//    next block's loads are in flight while the current one is multiplied;
//  * 16-byte chunks of a row are XOR-swizzled by (row/2 mod 8) so that the
//    16 rows read by one MFMA operand fall in distinct LDS bank groups;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows from LDS, Q^T in VGPRs),
//    V^T for O^T += V^T P^T read straight out of the same rows with
//    ds_read_b64_tr_b16, so the value needs no second copy.
// MLA: one workgroup of 8 waves takes 128 heads of one query token (16 heads
// per wave) over a range of its keys; long decode ranges are split and merged
// with the rescaling algebra of the page's flash_attention.
// Sparse: one workgroup of 4 waves takes one query's 16 heads; each wave owns
// one 16-key tile of every block; the four partial softmax states are merged
// in LDS at the end. The key set is the query's selected units, each resolved
// through the page table [Sparse page: _src paged address computation].
#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

constexpr int kDl = 512;
constexpr int kDk = 576;
constexpr int kRowChunks = kDk * 2 / 16;              // 72 chunks of 16 B per latent row
constexpr int kBlk = 64;                              // keys per block (one per lane)
constexpr int kColStride = kBlk * 16 + 64;            // 1088: LDS bytes per chunk column
constexpr int kStageBytes = kRowChunks * kColStride;  // 78336
constexpr int kQSteps = kDk / 32;                     // 18 MFMA k-steps
constexpr int kDvTiles = kDl / 16;                    // 32 output tiles of 16 dims

// Zero row read by keys outside the visible range (1152 bytes of bf16 zeros).
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[kRowChunks * 16] = {0};

// LDS layout of a block: chunk-major. Column c (16 bytes of every key) starts
// at c * kColStride; key k sits at slot k in even columns and at slot
// (k + 4) mod 64 in odd columns. The column padding (64 B) and the rotation
// keep both operand reads below free of bank conflicts.
__device__ __forceinline__ uint32_t col_slot(int key, int c) {
  return (uint32_t)(c * kColStride + (((key + 4 * (c & 1)) & (kBlk - 1)) << 4));
}

// Latent row r: columns [0, 512) at a + r*sa, columns [512, 576) at b + r*sb.
struct RowSrc {
  const char* a;
  const char* b;
  int64_t sa, sb;
};

// This wave's share of one block: columns [wave*IPW, wave*IPW + IPW), one
// global_load_lds_dwordx4 each (64 keys x 16 bytes). Lane L loads key L in
// even columns and key (L - 4) mod 64 in odd columns; rows[k] (LDS) is the
// physical row of block key k, or -1 for a key that must read as zeros. Both
// row ids are read from LDS before the first DMA of the block; the
// addresses are then rebuilt per instruction with VALU arithmetic only.
template <int IPW>
__device__ __forceinline__ void issue_block(const RowSrc& src, uint32_t stage, int wave,
                                            const int* rows) {
  const int lane = threadIdx.x & 63;
  const int row_par[2] = {rows[lane], rows[(lane - 4) & (kBlk - 1)]};
#pragma unroll
  for (int ii = 0; ii < IPW; ++ii) {
    const int c = __builtin_amdgcn_readfirstlane(wave * IPW + ii);
    const int row = (c & 1) ? row_par[1] : row_par[0];
    const bool in_a = c < 64;
    const char* base = in_a ? src.a : src.b;
    const int64_t stride = in_a ? src.sa : src.sb;
    const int coff = (in_a ? c : c - 64) * 16;
    const char* g = row >= 0 ? base + (int64_t)row * stride + coff
                             : (const char*)kZeroRow + c * 16;
    dma_b128(g, __builtin_amdgcn_readfirstlane(stage + (uint32_t)c * kColStride));
  }
}

// Q^T operand of one wave: lane l holds head (l % 16) dims 32j + 8(l/16) .. +7.
__device__ __forceinline__ void load_q(u32x4* qv, const uint16_t* q_nope, const uint16_t* q_pe,
                                       bool ok) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int j = 0; j < kQSteps; ++j) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) {
      const int d = 32 * j + 8 * g;
      v = d < kDl ? *reinterpret_cast<const u32x4*>(q_nope + d)
                  : *reinterpret_cast<const u32x4*>(q_pe + (d - kDl));
    }
    qv[j] = v;
  }
}

// Lane base for the S^T A operand of key tile key0 (rows key0 + lane%16,
// columns 4j + lane/16): col_slot(...) minus the j-dependent 4j*kColStride.
__device__ __forceinline__ uint32_t k_base(int key0) {
  const int lane = threadIdx.x & 63;
  return col_slot(key0 + (lane & 15), lane >> 4);
}

// Lane base for the V^T A operand read with ds_read_b64_tr_b16 for keys
// k0 + 4(lane/16) .. +3 and dims 16dt + lane%16 (dt-dependent part removed).
__device__ __forceinline__ uint32_t v_base(int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int jj = lane & 15;
  const int h = (jj & 3) >> 1;
  return col_slot(k0 + 4 * g + (jj >> 2), h) + 8 * (jj & 1);
}

// S^T[key, head] for one 16-key tile and NH head tiles; each K operand read
// feeds NH MFMAs.
template <int NH>
__device__ __forceinline__ void score_tile(floatx4* out, uint32_t stage, uint32_t kb,
                                           const u32x4 (*qv)[kQSteps]) {
  const uint32_t base = stage + kb;
#pragma unroll
  for (int h = 0; h < NH; ++h) out[h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j0 = 0; j0 < kQSteps; j0 += 3) {
    u32x4 kf[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) kf[j] = lds_read_b128(base + 4 * (j0 + j) * kColStride);
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        out[h] = mfma_16x16x32(as_bf16x8(kf[j]), as_bf16x8(qv[h][j0 + j]), out[h]);
    sched_fence();
  }
}

// V^T operand for dims of tile dt (4 keys per lane group).
__device__ __forceinline__ u32x2 v_tr(uint32_t stage, uint32_t vb, int dt) {
  return lds_read_tr16(stage + vb + 2 * dt * kColStride);
}

// Score transform in the exp2 domain: scale, optional soft cap.
__device__ __forceinline__ float score_log2(float s, float sc, float cap) {
  if (cap != 0.f) return cap * tanh_def(s * sc / cap) * kLog2e;
  return s * sc * kLog2e;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int g_num_cus = 0;
int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

// =============================================================== MLA ========

constexpr int kMlaWaves = 8;
constexpr int kMlaThreads = kMlaWaves * 64;
constexpr int kMlaHT = 1;                             // 16-head tiles per wave
constexpr int kMlaHeads = kMlaWaves * 16 * kMlaHT;    // heads per workgroup (128)
constexpr int kMlaIPW = kRowChunks / kMlaWaves;       // 9 columns per wave
constexpr int kPageWin = 1024;                        // page ids cached in LDS
constexpr int kMlaMaxSplits = 16;
constexpr int kMlaMinChunk = 256;

struct MlaSeq {
  int cu0, q_len, kv_len, kv_cap;
};

__device__ __forceinline__ MlaSeq mla_seq(const MlaArgs& a, int seq) {
  MlaSeq s;
  s.cu0 = a.cu_q_lens[seq];
  s.q_len = a.cu_q_lens[seq + 1] - s.cu0;
  s.kv_len = a.kv_lens[seq];
  s.kv_cap = min(s.kv_len, a.pages_per_seq * a.page_size);
  return s;
}

// Visible key range of query token tok_rel of a sequence (causal + window).
__device__ __forceinline__ void mla_range(const MlaArgs& a, const MlaSeq& s, int tok_rel, int* lo,
                                          int* hi) {
  const int pos = s.kv_len - s.q_len + tok_rel;
  *lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;
  *hi = min(pos + 1, s.kv_cap);
}

__device__ __forceinline__ int mla_num_seqs(const MlaArgs& a) {
  return clampi(*a.num_seqs, 0, a.max_num_seqs);
}

__device__ __forceinline__ int mla_hgroups(const MlaArgs& a) {
  return (a.num_heads + kMlaHeads - 1) / kMlaHeads;
}

__device__ __forceinline__ int mla_nsplit(int n, int chunk) {
  return (n <= 0 || chunk <= 0) ? 1 : min(kMlaMaxSplits, (n + chunk - 1) / chunk);
}

// counters: [0] tile count, [1] work cursor, [2] split chunk, [64..] per-seq tile offsets
__global__ void __launch_bounds__(256) mla_plan_kernel(MlaArgs a, int tile_target) {
  __shared__ int sh[256];
  __shared__ unsigned long long s_total;
  __shared__ int s_max;
  const int tid = threadIdx.x;
  const int ns = mla_num_seqs(a);
  const int HG = mla_hgroups(a);
  if (tid == 0) {
    s_total = 0;
    s_max = 0;
  }
  __syncthreads();
  // Pass 1: total and largest decode key range.
  unsigned long long part = 0;
  int mx = 0;
  for (int i = tid; i < ns; i += 256) {
    const MlaSeq s = mla_seq(a, i);
    if (s.q_len == 1) {
      int lo, hi;
      mla_range(a, s, 0, &lo, &hi);
      const int n = max(0, hi - lo);
      part += n;
      mx = max(mx, n);
    }
  }
  atomicAdd(&s_total, part);
  atomicMax(&s_max, mx);
  __syncthreads();
  const unsigned long long per = (s_total + tile_target - 1) / (unsigned long long)max(1, tile_target);
  int chunk = (int)(per < (1ull << 30) ? per : (1ull << 30));
  chunk = max(chunk, (s_max + kMlaMaxSplits - 1) / kMlaMaxSplits);
  chunk = max(kMlaMinChunk, (chunk + kBlk - 1) / kBlk * kBlk);
  // Pass 2: per-sequence tile counts and offsets.
  int* off = a.counters + 64;
  int run = 0;
  for (int c0 = 0; c0 < ns; c0 += 256) {
    const int i = c0 + tid;
    int n = 0;
    if (i < ns) {
      const MlaSeq s = mla_seq(a, i);
      if (s.q_len == 1) {
        int lo, hi;
        mla_range(a, s, 0, &lo, &hi);
        n = mla_nsplit(hi - lo, chunk) * HG;
      } else if (s.q_len > 1) {
        n = s.q_len * HG;
      }
    }
    sh[tid] = n;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int x = tid >= o ? sh[tid - o] : 0;
      __syncthreads();
      sh[tid] += x;
      __syncthreads();
    }
    if (i < ns) off[i] = run + sh[tid] - n;
    run += sh[255];
    __syncthreads();
  }
  if (tid == 0) off[ns] = run;
  __threadfence();
  __syncthreads();
  const int total = min(run, a.tile_capacity);
  // Each thread writes one contiguous range of tiles (one search, then the
  // owning sequence advances as its offsets are passed).
  const int span = (total + 255) / 256;
  const int t0 = min(total, tid * span);
  const int t1 = min(total, t0 + span);
  int seq = -1, seq_begin = 0, seq_end = 0, q_len = 0;
  for (int t = t0; t < t1; ++t) {
    if (seq < 0 || t >= seq_end) {
      int lo = 0, hi = ns - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t)
          lo = mid;
        else
          hi = mid - 1;
      }
      seq = lo;
      seq_begin = off[seq];
      seq_end = off[seq + 1];
      q_len = a.cu_q_lens[seq + 1] - a.cu_q_lens[seq];
    }
    const int local = t - seq_begin;
    int4 tl;
    tl.x = seq;
    tl.w = local % HG;
    if (q_len == 1) {
      tl.y = 0;
      tl.z = local / HG;  // split
    } else {
      tl.y = local / HG;  // token
      tl.z = -1;
    }
    reinterpret_cast<int4*>(a.tiles)[t] = tl;
  }
  if (tid == 0) {
    a.counters[0] = total;
    a.counters[1] = 0;
    a.counters[2] = chunk;
  }
}

struct MlaShared {
  char stage[2][kStageBytes];
  int pages[kPageWin];
  int rows[kBlk];
  int tile;
};
static_assert(sizeof(MlaShared) <= 160 * 1024, "MLA LDS budget");

__device__ void mla_process_tile(const MlaArgs& a, int4 tl, MlaShared& sm, int ps_log2, int chunk) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int seq = tl.x;
  const MlaSeq s = mla_seq(a, seq);
  const int tok_rel = tl.y;
  const int split = tl.z;
  int lo_all, hi_all;
  mla_range(a, s, tok_rel, &lo_all, &hi_all);
  int lo = lo_all, hi = hi_all, nsplit = 1;
  if (split >= 0) {
    nsplit = mla_nsplit(hi_all - lo_all, chunk);
    lo = lo_all + split * chunk;
    hi = (split == nsplit - 1) ? hi_all : min(hi_all, lo + chunk);
  }
  const int tok = s.cu0 + tok_rel;
  const int head0 = tl.w * kMlaHeads + wave * 16 * kMlaHT;  // first head of this wave
  const bool wave_active = head0 < a.num_heads;

  u32x4 qv[kMlaHT][kQSteps];
#pragma unroll
  for (int h = 0; h < kMlaHT; ++h) {
    const int head = head0 + 16 * h + (lane & 15);
    load_q(qv[h], (const uint16_t*)a.ql_nope + ((int64_t)tok * a.num_heads + head) * a.lkv_dim,
           (const uint16_t*)a.q_pe + ((int64_t)tok * a.num_heads + head) * a.r_dim,
           head < a.num_heads);
  }

  floatx4 acc[kMlaHT][kDvTiles];
#pragma unroll
  for (int h = 0; h < kMlaHT; ++h)
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt) acc[h][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[kMlaHT], l_run[kMlaHT];
#pragma unroll
  for (int h = 0; h < kMlaHT; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }

  const int kb0 = (lo / kBlk) * kBlk;
  const int nblk = hi > kb0 ? cdiv_i(hi - kb0, kBlk) : 0;
  const int32_t* table = a.page_indices + (int64_t)seq * a.pages_per_seq;
  const int ps_mask = (1 << ps_log2) - 1;
  int pwin = kb0 >> ps_log2;
  for (int i = tid; i < kPageWin; i += kMlaThreads) {
    const int lp = pwin + i;
    sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
  }
  __syncthreads();

  RowSrc src;
  src.a = (const char*)a.cache_kv_c;
  src.b = (const char*)a.cache_k_pe;
  src.sa = (int64_t)a.kvc_stride * 2;
  src.sb = (int64_t)a.kpe_stride * 2;
  const uint32_t st0 = lds_addr(sm.stage[0]);
  const uint32_t st1 = lds_addr(sm.stage[1]);
  const int P = a.total_num_pages;

  // Rows of block b go to sm.rows (one thread per key), then this wave's DMA.
  auto issue = [&](int b, uint32_t st) {
    const int kb = kb0 + b * kBlk;
    // Refill the page window when this block runs past it.
    if (((kb + kBlk - 1) >> ps_log2) - pwin >= kPageWin) {
      wg_barrier();
      pwin = kb >> ps_log2;
      for (int i = tid; i < kPageWin; i += kMlaThreads) {
        const int lp = pwin + i;
        sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
      }
      __syncthreads();
    }
    if (tid < kBlk) {
      const int key = kb + tid;
      int row = -1;
      if (key >= lo && key < hi) {
        const int page = sm.pages[(key >> ps_log2) - pwin];
        if (page >= 0 && page < P) row = (page << ps_log2) + (key & ps_mask);
      }
      sm.rows[tid] = row;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    wg_barrier();
    issue_block<kMlaIPW>(src, st, wave, sm.rows);
  };

  const float sc = a.score_scale;
  const float cap = a.soft_cap;
  uint32_t kbase[4], vbase[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    kbase[t] = k_base(16 * t);
    vbase[t] = v_base(16 * t);
  }
  drain_vmem_before_loop();
  if (nblk > 0) issue(0, st0);
  for (int b = 0; b < nblk; ++b) {
    const uint32_t cur = (b & 1) ? st1 : st0;
    if (b + 1 < nblk) {
      issue(b + 1, (b & 1) ? st0 : st1);
      wait_vmcnt<kMlaIPW>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    if (wave_active) {
      const int kb = kb0 + b * kBlk;
      u32x4 pb[kMlaHT][2];
#pragma unroll
      for (int h = 0; h < kMlaHT; ++h) {
        pb[h][0] = u32x4{0u, 0u, 0u, 0u};
        pb[h][1] = u32x4{0u, 0u, 0u, 0u};
      }
      {
        floatx4 sv[4][kMlaHT];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) score_tile<kMlaHT>(sv[kt], cur, kbase[kt], qv);
#pragma unroll
        for (int h = 0; h < kMlaHT; ++h) {
          float mblk = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kb + 16 * kt + 4 * g + i;
              const float x =
                  (key >= lo && key < hi) ? score_log2(sv[kt][h][i], sc, cap) : -INFINITY;
              sv[kt][h][i] = x;
              mblk = fmaxf(mblk, x);
            }
          mblk = wave_max_xor(mblk, 16);
          mblk = wave_max_xor(mblk, 32);
          const bool need = mblk > m_run[h] + kLazyTau;
          if (wave_any(need)) {
            const float m_new = need ? mblk : m_run[h];
            const float alpha = need ? fast_exp2(m_run[h] - m_new) : 1.f;  // rows not moving keep scale 1
            l_run[h] *= alpha;
#pragma unroll
            for (int dt = 0; dt < kDvTiles; ++dt) {
              acc[h][dt][0] *= alpha;
              acc[h][dt][1] *= alpha;
              acc[h][dt][2] *= alpha;
              acc[h][dt][3] *= alpha;
            }
            m_run[h] = m_new;
          }
          if (m_run[h] != -INFINITY) {
            float psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                sv[kt][h][i] = fast_exp2(sv[kt][h][i] - m_run[h]);
                psum += sv[kt][h][i];
              }
            l_run[h] += psum;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              pb[h][ks][0] = pack_bf16x2(sv[2 * ks][h][0], sv[2 * ks][h][1]);
              pb[h][ks][1] = pack_bf16x2(sv[2 * ks][h][2], sv[2 * ks][h][3]);
              pb[h][ks][2] = pack_bf16x2(sv[2 * ks + 1][h][0], sv[2 * ks + 1][h][1]);
              pb[h][ks][3] = pack_bf16x2(sv[2 * ks + 1][h][2], sv[2 * ks + 1][h][3]);
            }
          }
        }
      }
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        u32x4 vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x2 v0 = v_tr(cur, vbase[2 * ks], dt);
          const u32x2 v1 = v_tr(cur, vbase[2 * ks + 1], dt);
          vf[ks] = u32x4{v0[0], v0[1], v1[0], v1[1]};
        }
#pragma unroll
        for (int h = 0; h < kMlaHT; ++h)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            acc[h][dt] = mfma_16x16x32(as_bf16x8(vf[ks]), as_bf16x8(pb[h][ks]), acc[h][dt]);
        sched_fence();
      }
    }
    wg_barrier();
  }

  if (!wave_active) return;
#pragma unroll
  for (int h = 0; h < kMlaHT; ++h) {
    const int head = head0 + 16 * h + (lane & 15);
    float l_row = wave_sum_xor(l_run[h], 16);
    l_row = wave_sum_xor(l_row, 32);
    if (head >= a.num_heads) continue;
    if (split >= 0 && nsplit > 1) {
      const int64_t pidx = (int64_t)seq * kMlaMaxSplits + split;
      float* pa = a.part_acc + (pidx * a.num_heads + head) * kDl;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt)
        *reinterpret_cast<floatx4*>(pa + 16 * dt + 4 * g) = acc[h][dt];
      if (g == 0) {
        float* pm = a.part_ml + (pidx * a.num_heads + head) * 2;
        pm[0] = m_run[h];
        pm[1] = l_row;
      }
      continue;
    }
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    uint16_t* op = (uint16_t*)a.out + ((int64_t)tok * a.num_heads + head) * kDl;
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[h][dt][0] * inv, acc[h][dt][1] * inv);
      w[1] = pack_bf16x2(acc[h][dt][2] * inv, acc[h][dt][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * g) = w;
    }
  }
}

__global__ void __launch_bounds__(kMlaThreads) mla_tile_kernel(MlaArgs a, int ps_log2) {
  __shared__ __attribute__((aligned(16))) MlaShared sm;
  const int count = a.counters[0];
  const int chunk = a.counters[2];
  for (;;) {
    if (threadIdx.x == 0) sm.tile = atomicAdd(&a.counters[1], 1);
    __syncthreads();
    const int ti = sm.tile;
    __syncthreads();
    if (ti >= count) break;
    const int4 tl = reinterpret_cast<const int4*>(a.tiles)[ti];
    mla_process_tile(a, tl, sm, ps_log2, chunk);
    __syncthreads();
  }
}

// Combines the split partials of decode sequences: thread = (head, 8 dims).
__global__ void __launch_bounds__(256) mla_merge_kernel(MlaArgs a) {
  const int seq = blockIdx.x;
  if (seq >= mla_num_seqs(a)) return;
  const MlaSeq s = mla_seq(a, seq);
  if (s.q_len != 1) return;
  int lo, hi;
  mla_range(a, s, 0, &lo, &hi);
  const int nsplit = mla_nsplit(hi - lo, a.counters[2]);
  if (nsplit <= 1) return;
  const int t = blockIdx.y * 256 + threadIdx.x;
  const int head = t >> 6;
  const int d0 = (t & 63) * 8;
  if (head >= a.num_heads) return;
  const int64_t pbase = (int64_t)seq * kMlaMaxSplits;
  float mv[kMlaMaxSplits];
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMlaMaxSplits; ++sp) {
    mv[sp] = sp < nsplit ? a.part_ml[((pbase + sp) * a.num_heads + head) * 2] : -INFINITY;
    M = fmaxf(M, mv[sp]);
  }
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMlaMaxSplits; ++sp) {
      if (sp >= nsplit) break;
      const float w = fast_exp2(mv[sp] - M);
      L += w * a.part_ml[((pbase + sp) * a.num_heads + head) * 2 + 1];
      const float* pa = a.part_acc + ((pbase + sp) * a.num_heads + head) * kDl + d0;
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(pa);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(pa + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] += w * x0[i];
        o[4 + i] += w * x1[i];
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)s.cu0 * a.num_heads + head) * kDl + d0;
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(op) = w;
}

// ============================================================ sparse ========

constexpr int kSpWaves = 4;
constexpr int kSpThreads = kSpWaves * 64;
constexpr int kSpIPW = kRowChunks / kSpWaves;         // 18 columns per wave
constexpr int kSpMaxUnits = 256;

struct SparseShared {
  char stage[2][kStageBytes];
  int unit_row[kSpMaxUnits];
  int unit_id[kSpMaxUnits];
  int rows[kBlk];
  uint8_t valid[2][kBlk];
};
static_assert(sizeof(SparseShared) <= 160 * 1024, "sparse LDS budget");

__global__ void __launch_bounds__(kSpThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_kernel(SparseArgs a) {
  __shared__ __attribute__((aligned(16))) SparseShared sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int qi = blockIdx.x;
  const int hbase = blockIdx.y * 16;
  const int head = hbase + (lane & 15);
  const bool head_ok = head < a.num_heads;
  const int pos = a.positions[qi];
  const int K = a.top_k;
  const int RB = a.read_block;
  const int ps = a.page_size;

  // Unit table: physical first row of each selected unit (-1 = padding or
  // outside the page table) [Sparse page: _src, paged branch].
  for (int k = tid; k < K; k += kSpThreads) {
    const int u = a.indices[(int64_t)qi * K + k];
    int row = -1;
    if (u >= 0) {
      const int64_t lt = (int64_t)u * RB;
      const int64_t lp = lt / ps;
      if (lp < a.ptw) {
        const int phys = a.page_table[lp];
        if (phys >= 0 && phys < a.total_num_pages) row = phys * ps + (int)(lt - lp * ps);
      }
    }
    sm.unit_row[k] = row;
    sm.unit_id[k] = u;
  }
  __syncthreads();

  u32x4 qv[kQSteps];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)qi * a.num_heads + head) * kDk;
    load_q(qv, qp, qp + kDl, head_ok);
  }
  floatx4 acc[kDvTiles];
#pragma unroll
  for (int dt = 0; dt < kDvTiles; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  RowSrc src;
  src.a = (const char*)a.kv;
  src.b = (const char*)a.kv + kDl * 2;
  src.sa = (int64_t)a.cache_dim * 2;
  src.sb = src.sa;
  const uint32_t st0 = lds_addr(sm.stage[0]);
  const uint32_t st1 = lds_addr(sm.stage[1]);
  const int total = K * RB;
  const int nblk = cdiv_i(total, kBlk);

  // Rows and validity of block b (one thread per key), then this wave's DMA.
  auto issue = [&](int b, uint32_t st, uint8_t* valid) {
    if (tid < kBlk) {
      const int kk = b * kBlk + tid;
      int row = -1;
      if (kk < total) {
        const int unit = kk / RB;
        const int r = kk - unit * RB;
        const int base = sm.unit_row[unit];
        const int kp = sm.unit_id[unit] * RB + r;
        if (base >= 0 && kp <= pos && kp < a.seq_len) row = base + r;
      }
      sm.rows[tid] = row;
      valid[tid] = row >= 0 ? 1 : 0;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    wg_barrier();
    issue_block<kSpIPW>(src, st, wave, sm.rows);
  };

  const float sc = a.score_scale;
  const uint32_t kbase = k_base(16 * wave);
  const uint32_t vbase = v_base(16 * wave);
  drain_vmem_before_loop();
  if (nblk > 0) issue(0, st0, sm.valid[0]);
  for (int b = 0; b < nblk; ++b) {
    const int cs = b & 1;
    const uint32_t cur = cs ? st1 : st0;
    if (b + 1 < nblk) {
      issue(b + 1, cs ? st0 : st1, sm.valid[cs ^ 1]);
      wait_vmcnt<kSpIPW>();
    } else {
      wait_vmcnt<0>();
    }
    // DMA of block b landed (vmcnt above); validity bytes written with ds_write.
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    wg_barrier();
    floatx4 sv;
    score_tile<1>(&sv, cur, kbase, &qv);
    float mblk = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = sm.valid[cs][16 * wave + 4 * g + i] != 0;
      const float x = ok ? score_log2(sv[i], sc, 0.f) : -INFINITY;
      sv[i] = x;
      mblk = fmaxf(mblk, x);
    }
    mblk = wave_max_xor(mblk, 16);
    mblk = wave_max_xor(mblk, 32);
    const bool need = mblk > m_run + kLazyTau;
    if (wave_any(need)) {
      const float m_new = need ? mblk : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;  // rows not moving keep scale 1
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        acc[dt][0] *= alpha;
        acc[dt][1] *= alpha;
        acc[dt][2] *= alpha;
        acc[dt][3] *= alpha;
      }
      m_run = m_new;
    }
    u32x2 pb = {0u, 0u};
    if (m_run != -INFINITY) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m_run);
      l_run += (p[0] + p[1] + p[2] + p[3]);
      pb[0] = pack_bf16x2(p[0], p[1]);
      pb[1] = pack_bf16x2(p[2], p[3]);
    }
#pragma unroll
    for (int dt0 = 0; dt0 < kDvTiles; dt0 += 4) {
      u32x2 vt[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) vt[d] = v_tr(cur, vbase, dt0 + d);
#pragma unroll
      for (int d = 0; d < 4; ++d) acc[dt0 + d] = mfma_16x16x16(vt[d], pb, acc[dt0 + d]);
      sched_fence();
    }
    wg_barrier();
  }
  // The four waves hold the softmax state of disjoint key tiles: merge in LDS.
  float l_row = wave_sum_xor(l_run, 16);
  l_row = wave_sum_xor(l_row, 32);
  __syncthreads();
  float* accs = reinterpret_cast<float*>(sm.stage[0]);             // [4][16][512]
  float* mls = accs + kSpWaves * 16 * kDl;                          // [4][16][2]
  const int hl = lane & 15;
#pragma unroll
  for (int dt = 0; dt < kDvTiles; ++dt)
    *reinterpret_cast<floatx4*>(accs + ((wave * 16 + hl) * kDl) + 16 * dt + 4 * g) = acc[dt];
  if (g == 0) {
    mls[(wave * 16 + hl) * 2] = m_run;
    mls[(wave * 16 + hl) * 2 + 1] = l_row;
  }
  __syncthreads();
  const int h = tid >> 4;          // head within the group
  const int d0 = (tid & 15) * 32;  // 32 dims per thread
  if (hbase + h >= a.num_heads) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kSpWaves; ++w) M = fmaxf(M, mls[(w * 16 + h) * 2]);
  float wt[kSpWaves];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kSpWaves; ++w) {
    wt[w] = M == -INFINITY ? 0.f : fast_exp2(mls[(w * 16 + h) * 2] - M);
    L += wt[w] * mls[(w * 16 + h) * 2 + 1];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* op = a.out + ((int64_t)qi * a.num_heads + hbase + h) * kDl + d0;
#pragma unroll
  for (int d = 0; d < 32; d += 4) {
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kSpWaves; ++w) {
      const floatx4 x = *reinterpret_cast<const floatx4*>(accs + (w * 16 + h) * kDl + d0 + d);
      o[0] += wt[w] * x[0];
      o[1] += wt[w] * x[1];
      o[2] += wt[w] * x[2];
      o[3] += wt[w] * x[3];
    }
    o[0] *= inv;
    o[1] *= inv;
    o[2] *= inv;
    o[3] *= inv;
    *reinterpret_cast<floatx4*>(op + d) = o;
  }
}

}  // namespace

size_t mla_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_heads, int lkv_dim,
                           int* tile_capacity, int* max_splits) {
  const int HG = (num_heads + kMlaHeads - 1) / kMlaHeads;
  const int64_t cap = (int64_t)HG * ((int64_t)max_num_tokens + (int64_t)max_num_seqs * kMlaMaxSplits);
  if (tile_capacity) *tile_capacity = (int)cap;
  if (max_splits) *max_splits = kMlaMaxSplits;
  const int64_t nparts = (int64_t)max_num_seqs * kMlaMaxSplits;
  size_t bytes = align256((64 + (size_t)max_num_seqs + 1) * sizeof(int32_t));
  bytes += align256((size_t)cap * 16);
  bytes += align256((size_t)nparts * num_heads * 2 * sizeof(float));
  bytes += align256((size_t)nparts * num_heads * (size_t)lkv_dim * sizeof(float));
  return bytes;
}

void mla_bind_workspace(MlaArgs& a, void* ws) {
  int cap = 0, ms = 0;
  mla_workspace_bytes(a.max_num_seqs, a.max_num_tokens, a.num_heads, a.lkv_dim, &cap, &ms);
  a.tile_capacity = cap;
  a.max_splits = ms;
  char* p = (char*)ws;
  a.counters = (int32_t*)p;
  p += align256((64 + (size_t)a.max_num_seqs + 1) * sizeof(int32_t));
  a.tiles = (int32_t*)p;
  p += align256((size_t)cap * 16);
  const int64_t nparts = (int64_t)a.max_num_seqs * kMlaMaxSplits;
  a.part_ml = (float*)p;
  p += align256((size_t)nparts * a.num_heads * 2 * sizeof(float));
  a.part_acc = (float*)p;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream) {
  int ps_log2 = 0;
  while ((1 << ps_log2) < a.page_size) ++ps_log2;
  const int target = 2 * num_cus();
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(256), 0, stream, a, target);
  const int grid = max(1, min(a.tile_capacity, num_cus()));
  prof_begin(stream);
  hipLaunchKernelGGL(mla_tile_kernel, dim3(grid), dim3(kMlaThreads), 0, stream, a, ps_log2);
  prof_end(stream);
  const int ygrid = (a.num_heads * 64 + 255) / 256;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(a.max_num_seqs, ygrid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const SparseArgs& a, hipStream_t stream) {
  if (a.top_k > kSpMaxUnits) return hipErrorInvalidValue;
  const int hg = (a.num_heads + 15) / 16;
  prof_begin(stream);
  hipLaunchKernelGGL(sparse_mla_kernel, dim3(a.num_queries, hg), dim3(kSpThreads), 0, stream, a);
  prof_end(stream);
  return hipGetLastError();
}

}  // namespace rpa
