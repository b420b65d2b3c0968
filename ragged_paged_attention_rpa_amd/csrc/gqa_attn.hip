// GQA ragged paged attention on gfx950 [RPA v2 page: ragged_paged_attention,
// ref_ragged_paged_attention, flash_attention].
//
// Three launches on one stream, no host synchronisation:
//   1. gqa_plan_kernel   one workgroup turns the ragged metadata into a work
//                        list of tiles (prefill-class tiles first, then
//                        decode-class splits) and resets the work cursor;
//   2. gqa_tile_kernel   a persistent grid pops tiles off the list. A tile is
//                        (sequence, kv head, block of query tokens, key range);
//                        its rows are (query token, q head of the kv head's
//                        group) pairs, 16 per wave. Keys stream through LDS in
//                        blocks of 64 straight from the pages named by the page
//                        table; S^T = K Q^T and O^T += V^T P^T run on
//                        v_mfma_f32_16x16x32_bf16 with an online softmax in
//                        the exp2 domain;
//   3. gqa_merge_kernel  combines the (m, l, acc) partials of split decode
//                        sequences with the rescaling algebra of the page's
//                        flash_attention (alpha = e^{m_i - m*}).
// The per-row arithmetic follows the page: scale, optional soft cap, mask
// (causal offset kv_len - q_len, optional sliding window), softmax, P V.
#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

constexpr int kD = 128;                   // head dim of the MFMA path
constexpr int kBN = 64;                   // keys per LDS block
constexpr int kThreads = 256;             // 4 waves
constexpr int kKStride = kD * 2 + 16;     // LDS bytes per key row of K (padded)
constexpr int kVStride = kBN * 2 + 8;     // LDS bytes per dim row of V^T (padded)
constexpr int kKBytes = kBN * kKStride;   // 17408
constexpr int kVBytes = kD * kVStride;    // 17408
constexpr int kPartRows = 16;             // rows of a decode-class tile
constexpr int kNegBig = -1000000000;

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Split of a decode sequence's visible key range of n keys into at most
// max_splits chunks of at least split_keys keys (chunks are multiples of 64).
__host__ __device__ inline void split_plan(int n, int split_keys, int max_splits, int* nsplit,
                                           int* chunk) {
  if (n <= 0) {
    *nsplit = 1;
    *chunk = 0;
    return;
  }
  int c = split_keys;
  int ns = (n + c - 1) / c;
  if (ns > max_splits) {
    c = (((n + max_splits - 1) / max_splits) + 63) / 64 * 64;
    ns = (n + c - 1) / c;
  }
  *nsplit = ns;
  *chunk = c;
}

struct SeqInfo {
  int cu0, q_len, kv_len, kv_cap;
};

__device__ __forceinline__ SeqInfo seq_info(const GqaArgs& a, int seq) {
  SeqInfo s;
  s.cu0 = a.cu_q_lens[seq];
  s.q_len = a.cu_q_lens[seq + 1] - s.cu0;
  s.kv_len = a.kv_lens[seq];
  s.kv_cap = min(s.kv_len, a.pages_per_seq * a.page_size);
  return s;
}

// Visible key range [lo, hi) of all queries of a decode-class sequence.
__device__ __forceinline__ void decode_range(const GqaArgs& a, const SeqInfo& s, int* lo,
                                             int* hi) {
  const int first = s.kv_len - s.q_len;
  *lo = a.geo.window > 0 ? max(0, first - a.geo.window + 1) : 0;
  *hi = s.kv_cap;
}

__device__ __forceinline__ int num_seqs_clamped(const GqaArgs& a) {
  return clampi(*a.num_seqs, 0, a.max_num_seqs);
}

__device__ __forceinline__ bool is_decode_class(const GqaArgs& a, int q_len) {
  return q_len >= 1 && q_len <= a.geo.qdec;
}

// Tiles a sequence contributes: (prefill-class, decode-class).
__device__ __forceinline__ void seq_tile_counts(const GqaArgs& a, int seq, int* n_pre,
                                                int* n_dec) {
  const SeqInfo s = seq_info(a, seq);
  *n_pre = 0;
  *n_dec = 0;
  if (s.q_len <= 0) return;
  if (is_decode_class(a, s.q_len)) {
    int lo, hi, ns, ch;
    decode_range(a, s, &lo, &hi);
    split_plan(hi - lo, a.geo.split_keys, a.geo.max_splits, &ns, &ch);
    *n_dec = ns * a.num_kv_heads;
  } else {
    *n_pre = cdiv_i(s.q_len, a.geo.bq) * a.num_kv_heads;
  }
}

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int x = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[kThreads - 1];
  __syncthreads();
  return incl - v;
}

// seq_off layout in the workspace: [0, ns] prefill offsets, then [0, ns] decode offsets.
__device__ __forceinline__ int* seq_offsets(const GqaArgs& a) { return a.counters + 64; }

__device__ __forceinline__ int upper_bound_seq(const int* off, int n, int t) {
  // largest i in [0, n) with off[i] <= t
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kThreads) gqa_plan_kernel(GqaArgs a) {
  __shared__ int sh[kThreads];
  const int tid = threadIdx.x;
  const int ns = num_seqs_clamped(a);
  int* pre_off = seq_offsets(a);
  int* dec_off = pre_off + (a.max_num_seqs + 1);
  int run_pre = 0, run_dec = 0;
  for (int c0 = 0; c0 < ns; c0 += kThreads) {
    const int i = c0 + tid;
    int np = 0, nd = 0;
    if (i < ns) seq_tile_counts(a, i, &np, &nd);
    int tp, td;
    const int op = block_excl_scan(np, sh, &tp);
    const int od = block_excl_scan(nd, sh, &td);
    if (i < ns) {
      pre_off[i] = run_pre + op;
      dec_off[i] = run_dec + od;
    }
    run_pre += tp;
    run_dec += td;
  }
  if (tid == 0) {
    pre_off[ns] = run_pre;
    dec_off[ns] = run_dec;
  }
  __threadfence();
  __syncthreads();
  const int total = min(run_pre + run_dec, a.tile_capacity);
  const int H = a.num_kv_heads;
  for (int t = tid; t < total; t += kThreads) {
    Tile tl;
    if (t < run_pre) {
      const int seq = upper_bound_seq(pre_off, ns, t);
      const int q_len = a.cu_q_lens[seq + 1] - a.cu_q_lens[seq];
      const int nqb = cdiv_i(q_len, a.geo.bq);
      const int local = t - pre_off[seq];
      tl.seq = seq;
      tl.kvh = local / nqb;
      tl.qtok0 = (local % nqb) * a.geo.bq;
      tl.split = -1;
    } else {
      const int u = t - run_pre;
      const int seq = upper_bound_seq(dec_off, ns, u);
      const int local = u - dec_off[seq];
      tl.seq = seq;
      tl.kvh = local % H;
      tl.qtok0 = 0;
      tl.split = local / H;
    }
    a.tiles[t] = tl;
  }
  if (tid == 0) {
    a.counters[0] = total;
    a.counters[1] = 0;
  }
}

// ------------------------------------------------------------ tile kernel --

// Register staging of one 64-key block of K and V rows of one kv head.
// bf16: 32 lanes per key (16 B each, 512 B = K row then V row), 8 steps.
// fp8:  16 lanes per key (16 B each, 256 B), 4 steps.
template <int KV_DT>
struct KvStage {
  static constexpr int kLanesPerKey = KV_DT == DT_BF16 ? 32 : 16;
  static constexpr int kKeysPerStep = kThreads / kLanesPerKey;
  static constexpr int kSteps = kBN / kKeysPerStep;
  u32x4 buf[kSteps];
};

template <int KV_DT>
__device__ __forceinline__ void stage_load(KvStage<KV_DT>& st, const GqaArgs& a, int seq, int kvh,
                                           int kb, int lo, int hi, int ps_log2) {
  constexpr int LPK = KvStage<KV_DT>::kLanesPerKey;
  constexpr int KPS = KvStage<KV_DT>::kKeysPerStep;
  const int tid = threadIdx.x;
  const int kk = tid / LPK;
  const int c = tid % LPK;
  const int eb = KV_DT == DT_BF16 ? 2 : 1;
  const int64_t token_stride = (int64_t)2 * a.num_kv_heads * kD * eb;  // bytes per token row
  const char* kv = (const char*)a.kv;
  const int32_t* table = a.page_indices + (int64_t)seq * a.pages_per_seq;
#pragma unroll
  for (int s = 0; s < KvStage<KV_DT>::kSteps; ++s) {
    const int key = kb + s * KPS + kk;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key >= lo && key < hi) {
      const int page = table[key >> ps_log2];
      if (page >= 0 && page < a.total_num_pages) {
        const int64_t row = ((int64_t)page << ps_log2) + (key & ((1 << ps_log2) - 1));
        const char* p = kv + row * token_stride + (int64_t)(2 * kvh) * kD * eb + c * 16;
        v = *reinterpret_cast<const u32x4*>(p);
      }
    }
    st.buf[s] = v;
  }
}

template <int KV_DT>
__device__ __forceinline__ void stage_store(const KvStage<KV_DT>& st, char* k_lds, char* v_lds) {
  constexpr int LPK = KvStage<KV_DT>::kLanesPerKey;
  constexpr int KPS = KvStage<KV_DT>::kKeysPerStep;
  const int tid = threadIdx.x;
  const int kk = tid / LPK;
  const int c = tid % LPK;
#pragma unroll
  for (int s = 0; s < KvStage<KV_DT>::kSteps; ++s) {
    const int key = s * KPS + kk;
    const u32x4 v = st.buf[s];
    if (KV_DT == DT_BF16) {
      if (c < 16) {
        *reinterpret_cast<u32x4*>(k_lds + key * kKStride + c * 16) = v;
      } else {
        const int d0 = (c - 16) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<uint16_t*>(v_lds + (d0 + 2 * i) * kVStride + key * 2) =
              (uint16_t)(v[i] & 0xffffu);
          *reinterpret_cast<uint16_t*>(v_lds + (d0 + 2 * i + 1) * kVStride + key * 2) =
              (uint16_t)(v[i] >> 16);
        }
      }
    } else {
      if (c < 8) {
        const u32x2 b0 = fp8x4_to_bf16x4(v[0]);
        const u32x2 b1 = fp8x4_to_bf16x4(v[1]);
        const u32x2 b2 = fp8x4_to_bf16x4(v[2]);
        const u32x2 b3 = fp8x4_to_bf16x4(v[3]);
        const u32x4 w0 = {b0[0], b0[1], b1[0], b1[1]};
        const u32x4 w1 = {b2[0], b2[1], b3[0], b3[1]};
        *reinterpret_cast<u32x4*>(k_lds + key * kKStride + c * 32) = w0;
        *reinterpret_cast<u32x4*>(k_lds + key * kKStride + c * 32 + 16) = w1;
      } else {
        const int d0 = (c - 8) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x2 b = fp8x4_to_bf16x4(v[i]);
          *reinterpret_cast<uint16_t*>(v_lds + (d0 + 4 * i + 0) * kVStride + key * 2) =
              (uint16_t)(b[0] & 0xffffu);
          *reinterpret_cast<uint16_t*>(v_lds + (d0 + 4 * i + 1) * kVStride + key * 2) =
              (uint16_t)(b[0] >> 16);
          *reinterpret_cast<uint16_t*>(v_lds + (d0 + 4 * i + 2) * kVStride + key * 2) =
              (uint16_t)(b[1] & 0xffffu);
          *reinterpret_cast<uint16_t*>(v_lds + (d0 + 4 * i + 3) * kVStride + key * 2) =
              (uint16_t)(b[1] >> 16);
        }
      }
    }
  }
}

template <int KV_DT>
__device__ void process_tile(const GqaArgs& a, const Tile& tile, char* k_lds, char* v_lds,
                             int ps_log2) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = a.geo.group;
  const int seq = tile.seq;
  const int kvh = tile.kvh;
  const SeqInfo s = seq_info(a, seq);

  int qtok0, ntok, lo, hi;
  int nsplit = 1;
  if (tile.split >= 0) {
    int lo_all, hi_all, chunk;
    decode_range(a, s, &lo_all, &hi_all);
    split_plan(hi_all - lo_all, a.geo.split_keys, a.geo.max_splits, &nsplit, &chunk);
    qtok0 = 0;
    ntok = s.q_len;
    lo = lo_all + tile.split * chunk;
    hi = min(hi_all, lo + chunk);
  } else {
    qtok0 = tile.qtok0;
    ntok = min(a.geo.bq, s.q_len - qtok0);
    const int first = s.kv_len - s.q_len + qtok0;
    lo = a.geo.window > 0 ? max(0, first - a.geo.window + 1) : 0;
    hi = min(first + ntok, s.kv_cap);
  }
  const int first_pos = s.kv_len - s.q_len + qtok0;
  const int nrows = ntok * G;
  const bool wave_active = wave * 16 < nrows;

  // This lane's row (for the S^T columns and the O^T columns).
  const int r = wave * 16 + (lane & 15);
  const bool row_ok = r < nrows;
  const int qpos = row_ok ? first_pos + r / G : kNegBig;
  const int W = a.geo.window;

  // Q^T operand: row r, dims 32j + 8*(lane/16) .. +7.
  u32x4 qv[4];
  {
    const int tok = s.cu0 + qtok0 + (row_ok ? r / G : 0);
    const int head = kvh * G + (row_ok ? r % G : 0);
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)tok * a.num_q_heads + head) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + 32 * j + 8 * (lane >> 4));
      qv[j] = v;
    }
  }

  floatx4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const float cap = a.soft_cap;
  const float sc = cap != 0.f ? a.score_scale : a.score_scale * kLog2e;

  const int kb0 = lo > 0 ? (lo / kBN) * kBN : 0;
  const int nblk = hi > kb0 ? cdiv_i(hi - kb0, kBN) : 0;

  KvStage<KV_DT> st;
  if (nblk > 0) {
    stage_load<KV_DT>(st, a, seq, kvh, kb0, lo, hi, ps_log2);
    stage_store<KV_DT>(st, k_lds, v_lds);
  }
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    const int kb = kb0 + b * kBN;
    if (b + 1 < nblk) stage_load<KV_DT>(st, a, seq, kvh, kb + kBN, lo, hi, ps_log2);

    if (wave_active) {
      // S^T[key, row] for the 4 key tiles of the block.
      floatx4 sv[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        floatx4 c = {0.f, 0.f, 0.f, 0.f};
        const char* krow = k_lds + (16 * kt + (lane & 15)) * kKStride + 16 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + 64 * j);
          c = mfma_16x16x32(as_bf16x8(kf), as_bf16x8(qv[j]), c);
        }
        sv[kt] = c;
      }
      // Scale, soft cap, mask (log2 domain).
      float mblk = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 16 * kt + 4 * (lane >> 4) + i;
          float x = sv[kt][i] * sc;
          if (cap != 0.f) x = cap * tanh_def(x / cap) * kLog2e;
          const bool vis = key >= lo && key < hi && key <= qpos && (W <= 0 || key > qpos - W);
          x = vis ? x : -INFINITY;
          sv[kt][i] = x;
          mblk = fmaxf(mblk, x);
        }
      }
      mblk = wave_max_xor(mblk, 16);
      mblk = wave_max_xor(mblk, 32);
      const float m_new = fmaxf(m_run, mblk);
      float alpha = 1.f;
      u32x4 pb[2];
      if (m_new == -INFINITY) {
        pb[0] = u32x4{0u, 0u, 0u, 0u};
        pb[1] = u32x4{0u, 0u, 0u, 0u};
      } else {
        alpha = fast_exp2(m_run - m_new);
        float psum = 0.f;
        float p[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kt][i] = fast_exp2(sv[kt][i] - m_new);
            psum += p[kt][i];
          }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          pb[ks][0] = pack_bf16x2(p[2 * ks][0], p[2 * ks][1]);
          pb[ks][1] = pack_bf16x2(p[2 * ks][2], p[2 * ks][3]);
          pb[ks][2] = pack_bf16x2(p[2 * ks + 1][0], p[2 * ks + 1][1]);
          pb[ks][3] = pack_bf16x2(p[2 * ks + 1][2], p[2 * ks + 1][3]);
        }
      }
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        acc[dt][0] *= alpha;
        acc[dt][1] *= alpha;
        acc[dt][2] *= alpha;
        acc[dt][3] *= alpha;
      }
      // O^T[d, row] += V^T[d, key] P^T[key, row].
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const char* vrow = v_lds + (16 * dt + (lane & 15)) * kVStride + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow + 64 * ks);
          const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + 64 * ks + 32);
          const u32x4 vf = {v0[0], v0[1], v1[0], v1[1]};
          acc[dt] = mfma_16x16x32(as_bf16x8(vf), as_bf16x8(pb[ks]), acc[dt]);
        }
      }
    }
    __syncthreads();
    if (b + 1 < nblk) {
      stage_store<KV_DT>(st, k_lds, v_lds);
      __syncthreads();
    }
  }

  if (!wave_active) return;
  // Row normaliser: the four lanes holding a row each summed a quarter of it.
  float l_row = wave_sum_xor(l_run, 16);
  l_row = wave_sum_xor(l_row, 32);

  if (tile.split >= 0 && nsplit > 1) {
    // Partial (m, l, unnormalised acc) for the merge kernel.
    const int64_t pidx = ((int64_t)seq * a.num_kv_heads + kvh) * a.geo.max_splits + tile.split;
    if (row_ok) {
      float* pa = a.part_acc + (pidx * kPartRows + r) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<floatx4*>(pa + 16 * dt + 4 * (lane >> 4)) = acc[dt];
      if (lane < 16) {
        float* pm = a.part_ml + (pidx * kPartRows + r) * 2;
        pm[0] = m_run;
        pm[1] = l_row;
      }
    }
    return;
  }
  if (!row_ok) return;
  const float inv = l_row > 0.f ? a.v_scale / l_row : 0.f;
  const int tok = s.cu0 + qtok0 + r / G;
  const int head = kvh * G + r % G;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)tok * a.num_q_heads + head) * kD;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w;
    w[0] = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
    w[1] = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * (lane >> 4)) = w;
  }
}

template <int KV_DT>
__global__ void __launch_bounds__(kThreads, 2) gqa_tile_kernel(GqaArgs a, int ps_log2) {
  __shared__ __attribute__((aligned(16))) char smem[kKBytes + kVBytes];
  __shared__ int s_tile;
  const int count = a.counters[0];
  for (;;) {
    if (threadIdx.x == 0) s_tile = atomicAdd(&a.counters[1], 1);
    __syncthreads();
    const int ti = s_tile;
    __syncthreads();
    if (ti >= count) break;
    const Tile tile = a.tiles[ti];
    process_tile<KV_DT>(a, tile, smem, smem + kKBytes, ps_log2);
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kThreads) gqa_merge_kernel(GqaArgs a) {
  const int seq = blockIdx.x / a.num_kv_heads;
  const int kvh = blockIdx.x % a.num_kv_heads;
  if (seq >= num_seqs_clamped(a)) return;
  const SeqInfo s = seq_info(a, seq);
  if (!is_decode_class(a, s.q_len)) return;
  int lo, hi, nsplit, chunk;
  decode_range(a, s, &lo, &hi);
  split_plan(hi - lo, a.geo.split_keys, a.geo.max_splits, &nsplit, &chunk);
  if (nsplit <= 1) return;
  const int G = a.geo.group;
  const int nrows = s.q_len * G;
  const int r = threadIdx.x >> 4;        // row
  const int d0 = (threadIdx.x & 15) * 8; // 8 dims per thread
  if (r >= nrows) return;
  const int64_t pbase = ((int64_t)seq * a.num_kv_heads + kvh) * a.geo.max_splits;
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, a.part_ml[((pbase + sp) * kPartRows + r) * 2]);
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* pm = a.part_ml + ((pbase + sp) * kPartRows + r) * 2;
      const float w = fast_exp2(pm[0] - M);
      L += w * pm[1];
      const float* pa = a.part_acc + ((pbase + sp) * kPartRows + r) * kD + d0;
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(pa);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(pa + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] += w * x0[i];
        o[4 + i] += w * x1[i];
      }
    }
  }
  const float inv = L > 0.f ? a.v_scale / L : 0.f;
  const int tok = s.cu0 + r / G;
  const int head = kvh * G + r % G;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)tok * a.num_q_heads + head) * kD + d0;
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(op) = w;
}

// ----------------------------------------------------------- VALU generic --
// One wave per (query token, q head); keys one at a time. Serves fp32 queries,
// head dims other than 128 and non-power-of-two page sizes.
template <typename T>
__device__ __forceinline__ float load_as_f32(const void* base, int64_t idx, int dt) {
  if (dt == DT_F32) return reinterpret_cast<const float*>(base)[idx];
  if (dt == DT_BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  const uint8_t b = reinterpret_cast<const uint8_t*>(base)[idx];
  float f[4];
  fp8x4_to_f32((uint32_t)b, f);
  return f[0];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__global__ void __launch_bounds__(64) gqa_generic_kernel(GqaArgs a) {
  const int tok = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int ns = num_seqs_clamped(a);
  const int seq = find_seq(a.cu_q_lens, ns, tok);
  if (seq < 0) return;
  const SeqInfo s = seq_info(a, seq);
  const int G = a.geo.group;
  const int kvh = h / G;
  const int D = a.head_dim;
  const int pos = s.kv_len - s.q_len + (tok - s.cu0);
  const int W = a.geo.window;
  const int lo = W > 0 ? max(0, pos - W + 1) : 0;
  const int hi = min(pos + 1, s.kv_cap);
  constexpr int kMaxChunks = 8;  // head_dim <= 512
  float qf[kMaxChunks], acc[kMaxChunks];
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    const int d = lane + 64 * k;
    qf[k] = d < D ? load_as_f32<float>(a.q, ((int64_t)tok * a.num_q_heads + h) * D + d, a.q_dtype)
                  : 0.f;
    acc[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int64_t ch = 2 * a.num_kv_heads;
  for (int key = lo; key < hi; ++key) {
    const int page = a.page_indices[(int64_t)seq * a.pages_per_seq + key / a.page_size];
    if (page < 0 || page >= a.total_num_pages) continue;
    const int64_t row = (int64_t)page * a.page_size + key % a.page_size;
    const int64_t kbase = (row * ch + 2 * kvh) * D;
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) {
      const int d = lane + 64 * k;
      if (d < D) part += qf[k] * load_as_f32<float>(a.kv, kbase + d, a.kv_dtype);
    }
    float x = wave_sum(part) * a.score_scale;
    if (a.soft_cap != 0.f) x = a.soft_cap * tanhf(x / a.soft_cap);
    const float m_new = fmaxf(m, x);
    const float alpha = expf(m - m_new);
    const float p = expf(x - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) {
      const int d = lane + 64 * k;
      const float v = d < D ? load_as_f32<float>(a.kv, kbase + D + d, a.kv_dtype) : 0.f;
      acc[k] = acc[k] * alpha + p * v;
    }
    m = m_new;
  }
  const float inv = l > 0.f ? a.v_scale / l : 0.f;
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    const int d = lane + 64 * k;
    if (d >= D) continue;
    const int64_t o = ((int64_t)tok * a.num_q_heads + h) * D + d;
    if (a.q_dtype == DT_F32)
      reinterpret_cast<float*>(a.out)[o] = acc[k] * inv;
    else
      reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(acc[k] * inv);
  }
}

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

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

GqaGeometry gqa_geometry(int num_q_heads, int num_kv_heads, int window) {
  GqaGeometry g;
  g.group = num_q_heads / num_kv_heads;
  g.qdec = g.group <= 16 ? 16 / g.group : 0;
  g.bq = g.group <= 64 ? 64 / g.group : 1;
  g.split_keys = 512;
  g.max_splits = 16;
  g.window = window;
  return g;
}

bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim, int group) {
  return q_dtype == DT_BF16 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && head_dim == kD &&
         group >= 1 && group <= 64;
}

size_t gqa_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_q_heads,
                           int num_kv_heads, int head_dim, int window, int* tile_capacity) {
  const GqaGeometry g = gqa_geometry(num_q_heads, num_kv_heads, window);
  const int64_t cap = (int64_t)num_kv_heads *
                      ((int64_t)max_num_tokens / g.bq + max_num_seqs +
                       (int64_t)max_num_seqs * g.max_splits);
  if (tile_capacity) *tile_capacity = (int)cap;
  const int64_t nparts = (int64_t)max_num_seqs * num_kv_heads * g.max_splits;
  size_t bytes = 0;
  bytes += align256((64 + 2 * ((size_t)max_num_seqs + 1)) * sizeof(int32_t));  // counters + offsets
  bytes += align256((size_t)cap * sizeof(Tile));
  bytes += align256((size_t)nparts * kPartRows * 2 * sizeof(float));
  bytes += align256((size_t)nparts * kPartRows * (size_t)head_dim * sizeof(float));
  return bytes;
}

void gqa_bind_workspace(GqaArgs& a, void* ws) {
  int cap = 0;
  gqa_workspace_bytes(a.max_num_seqs, a.max_num_tokens, a.num_q_heads, a.num_kv_heads,
                      a.head_dim, a.geo.window, &cap);
  a.tile_capacity = cap;
  char* p = (char*)ws;
  a.counters = (int32_t*)p;
  p += align256((64 + 2 * ((size_t)a.max_num_seqs + 1)) * sizeof(int32_t));
  a.tiles = (Tile*)p;
  p += align256((size_t)cap * sizeof(Tile));
  const int64_t nparts = (int64_t)a.max_num_seqs * a.num_kv_heads * a.geo.max_splits;
  a.part_ml = (float*)p;
  p += align256((size_t)nparts * kPartRows * 2 * sizeof(float));
  a.part_acc = (float*)p;
}

hipError_t launch_gqa(const GqaArgs& a, hipStream_t stream) {
  int ps_log2 = 0;
  while ((1 << ps_log2) < a.page_size) ++ps_log2;
  hipLaunchKernelGGL(gqa_plan_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  const int grid = max(1, min(a.tile_capacity, num_cus() * 4));
  prof_begin(stream);
  if (a.kv_dtype == DT_BF16)
    hipLaunchKernelGGL(gqa_tile_kernel<DT_BF16>, dim3(grid), dim3(kThreads), 0, stream, a,
                       ps_log2);
  else
    hipLaunchKernelGGL(gqa_tile_kernel<DT_FP8>, dim3(grid), dim3(kThreads), 0, stream, a,
                       ps_log2);
  prof_end(stream);
  if (a.geo.qdec > 0)
    hipLaunchKernelGGL(gqa_merge_kernel, dim3(a.max_num_seqs * a.num_kv_heads), dim3(kThreads),
                       0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gqa_generic(const GqaArgs& a, hipStream_t stream) {
  if (a.max_num_tokens <= 0) return hipSuccess;
  prof_begin(stream);
  hipLaunchKernelGGL(gqa_generic_kernel, dim3(a.max_num_tokens, a.num_q_heads), dim3(64), 0,
                     stream, a);
  prof_end(stream);
  return hipGetLastError();
}

}  // namespace rpa
