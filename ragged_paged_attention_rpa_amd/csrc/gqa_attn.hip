// GQA ragged paged attention on gfx950 [RPA v2 page: ragged_paged_attention,
// ref_ragged_paged_attention, flash_attention].
//
// Launches, with no host synchronisation:
//   1. gqa_plan_kernel   turns the ragged metadata into a work list of tiles
//                        (prefill-class tiles first, then decode-class
//                        splits) and resets the work cursors;
//   2. gqa_prefill_kernel (gqa_prefill.hip) takes the prefill-class tiles
//                        when it applies (page size >= 8, positive scale);
//   3. gqa_tile_kernel   a persistent grid pops the remaining tiles. A tile is
//                        (sequence, kv head, block of query tokens, key range);
//                        its rows are (query token, q head of the kv head's
//                        group) pairs, 16 per wave. Keys stream through LDS in
//                        blocks of 64 straight from the pages named by the page
//                        table; S^T = K Q^T and O^T += V^T P^T run on
//                        v_mfma_f32_16x16x32_bf16 with an online softmax in
//                        the exp2 domain. For an fp8 pool whose prefill-class
//                        tiles went to the prefill kernel, gqa_decode8_kernel
//                        takes its place (128-key raw blocks widened in
//                        registers);
//   4. gqa_merge_kernel  combines the (m, l, output) partials of split decode
//                        sequences with the rescaling algebra of the page's
//                        flash_attention (alpha = e^{m_i - m*}).
// Launches 3 and 4 go to a library-owned side stream, forked after 1 and
// joined before the call returns, when the batch has room for a prefill share
// (they then run beside launch 2); otherwise everything is on the caller's
// stream.
// The per-row arithmetic follows the page: scale, optional soft cap, mask
// (causal offset kv_len - q_len, optional sliding window), softmax, P V.
#include <mutex>

#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

constexpr int kD = 128;                   // head dim of the MFMA path
constexpr int kBN = 64;                   // keys per LDS block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPartRows = 16;             // rows of a decode-class tile
constexpr int kNegBig = -1000000000;
constexpr int kMaxSplits = 16;            // cap on splits of one decode sequence

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

// Block-wide exclusive scan of one int per thread: wave scans by shuffles,
// then the four wave totals through LDS.
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    before += w < wave ? sh[w] : 0;
    all += sh[w];
  }
  *total = all;
  __syncthreads();
  return before + x - v;
}

// seq_off layout in the workspace: [0, ns] prefill offsets, then [0, ns] offsets of the
// decode splits but the last, then [0, ns] offsets of the last splits.
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

// Batches of up to this many sequences keep the planner's tile offsets in LDS.
constexpr int kPlanLdsSeqs = 4096;
constexpr int kPlanWgs = 32;

__global__ void __launch_bounds__(kThreads) gqa_plan_kernel(GqaArgs a) {
  __shared__ int sh[kThreads];
  __shared__ int off_lds[3 * (kPlanLdsSeqs + 1)];
  const int tid = threadIdx.x;
  const int ns = num_seqs_clamped(a);
  const bool in_lds = ns <= kPlanLdsSeqs;
  const int H = a.num_kv_heads;
  // Tile order: prefill-class tiles, then every decode split but the last of
  // its sequence (full length), then the last splits (the remainders, mostly
  // shorter), so a persistent grid ends on short tiles.
  int* pre_off = in_lds ? off_lds : seq_offsets(a);
  const int stride = in_lds ? kPlanLdsSeqs + 1 : a.max_num_seqs + 1;
  int* full_off = pre_off + stride;
  int* last_off = full_off + stride;
  int run_pre = 0, run_full = 0, run_last = 0;
  for (int c0 = 0; c0 < ns; c0 += kThreads) {
    const int i = c0 + tid;
    int np = 0, nd = 0;
    if (i < ns) seq_tile_counts(a, i, &np, &nd);
    const int nl = nd > 0 ? H : 0;
    int tp, tf, tl;
    const int op = block_excl_scan(np, sh, &tp);
    const int of = block_excl_scan(nd - nl, sh, &tf);
    const int ol = block_excl_scan(nl, sh, &tl);
    if (i < ns) {
      pre_off[i] = run_pre + op;
      full_off[i] = run_full + of;
      last_off[i] = run_last + ol;
    }
    run_pre += tp;
    run_full += tf;
    run_last += tl;
  }
  if (tid == 0) {
    pre_off[ns] = run_pre;
    full_off[ns] = run_full;
    last_off[ns] = run_last;
  }
  if (!in_lds) __threadfence();
  __syncthreads();
  const int total = min(run_pre + run_full + run_last, a.tile_capacity);
  // With the offsets in LDS every workgroup has computed them and writes its
  // share of the tiles; otherwise workgroup 0 writes them all. Each thread
  // writes one contiguous range: one search for its first tile, then the
  // owning sequence advances as the offsets are passed.
  const int nwg = in_lds ? (int)gridDim.x : 1;
  if ((int)blockIdx.x >= nwg) return;
  const int per_wg = (total + nwg - 1) / nwg;
  const int w0 = min(total, (int)blockIdx.x * per_wg);
  const int w1 = min(total, w0 + per_wg);
  const int per = (w1 - w0 + kThreads - 1) / kThreads;
  const int t0 = min(w1, w0 + tid * per);
  const int t1 = min(w1, t0 + per);
  if (t0 < t1) {
    int seq = -1, seq_begin = 0, seq_end = 0, nqb = 1;
    for (int t = t0; t < t1; ++t) {
      Tile tl;
      if (t < run_pre) {
        if (seq < 0 || t >= seq_end) {
          seq = upper_bound_seq(pre_off, ns, t);
          seq_begin = pre_off[seq];
          seq_end = pre_off[seq + 1];
          const int q_len = a.cu_q_lens[seq + 1] - a.cu_q_lens[seq];
          nqb = cdiv_i(q_len, a.geo.bq);
        }
        const int local = t - seq_begin;
        tl.seq = seq;
        tl.kvh = local / nqb;
        // Query blocks in descending order: within a (sequence, kv head) the
        // blocks with the most keys are taken first, so the last tiles a
        // workgroup picks up are the short ones.
        tl.qtok0 = (nqb - 1 - local % nqb) * a.geo.bq;
        tl.split = -1;
      } else if (t < run_pre + run_full) {
        const int u = t - run_pre;
        if (seq < 0 || t == run_pre || u >= seq_end) {  // first full split or next sequence
          seq = upper_bound_seq(full_off, ns, u);
          seq_begin = full_off[seq];
          seq_end = full_off[seq + 1];
        }
        const int local = u - seq_begin;
        tl.seq = seq;
        tl.kvh = local % H;
        tl.qtok0 = 0;
        tl.split = local / H;
      } else {
        const int u = t - run_pre - run_full;
        if (seq < 0 || t == run_pre + run_full || u >= seq_end) {  // first last split or next sequence
          seq = upper_bound_seq(last_off, ns, u);
          seq_begin = last_off[seq];
          seq_end = last_off[seq + 1];
          int lo, hi, ch;
          decode_range(a, seq_info(a, seq), &lo, &hi);
          split_plan(hi - lo, a.geo.split_keys, a.geo.max_splits, &nqb, &ch);
        }
        tl.seq = seq;
        tl.kvh = u - seq_begin;
        tl.qtok0 = 0;
        tl.split = nqb - 1;  // nqb holds the sequence's split count here
      }
      a.tiles[t] = tl;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    const int npre = min(run_pre, total);
    a.counters[0] = total;
    a.counters[1] = a.pre_kernel ? npre : 0;  // this file's kernel starts past them
    a.counters[3] = a.pre_kernel ? npre : 0;
    for (int x = 0; x < kXcds; ++x) a.counters[kXcdCursor0 + x] = 0;
  }
}

// ------------------------------------------------------------ tile kernel --
//
// Keys move through LDS in blocks of 64. A DMA instruction
// (global_load_lds_dwordx4) moves 1 KB of consecutive global bytes, two keys
// of a bf16 pool (K then V of one kv head: 512 bytes each) or four keys of an
// fp8 pool (256 bytes each): wide contiguous requests stream much faster
// than the 64-keys-by-16-bytes pattern of one column per instruction. A block
// is stored key-major, 512 bytes per key; inside a key the 16-byte column q
// (0..15 K dims 8q.., 16..31 V dims 8(q-16)..) sits at q ^ swz(key), which
// makes the K reads (eight keys, one column) and the transposed V reads
// (four keys, two columns) hit distinct banks. The DMA applies the swizzle
// by choosing which global column each lane fetches. fp8 blocks land raw
// (256 bytes per key, column rc at rc ^ (key & 15)) and a conversion pass
// widens them into the bf16 layout.
//
// Two compute modes share the block pipeline:
//  * rows <= 16 (decode): every wave takes the same rows and one 16-key tile
//    of each block, keeping its own softmax state; the four states are merged
//    in LDS at the end;
//  * rows > 16 (prefill): wave w takes rows 16w .. 16w+15 against all 64 keys.

constexpr int kKeyBytes = 512;                       // K + V of one key, bf16
constexpr int kRawKeyBytes = 256;                    // K + V of one key, fp8
constexpr int kStageBytes = kBN * kKeyBytes;         // 32768
constexpr int kRawStageBytes = kBN * kRawKeyBytes;   // 16384
constexpr int kTileBytes = 16 * kKeyBytes;           // one 16-key MFMA tile
constexpr int kPageWin = 512;                        // page ids of the tile cached in LDS
constexpr int kStages = 2;                           // DMA stages per workgroup

__device__ __attribute__((aligned(16))) const uint8_t kZeroKV[512] = {0};

template <int KV_DT, int NST>
struct TileSmem {
  // bf16: NST DMA stages. fp8: NST raw DMA stages plus one converted stage.
  char stage[KV_DT == DT_BF16 ? NST * kStageBytes : NST * kRawStageBytes + kStageBytes];
  int pages[kPageWin];
  int tile;
};

// Column swizzle of a key (only its low four bits matter, so every 16-key
// tile has the same pattern). It maps the low four key bits one-to-one, gives
// eight consecutive keys distinct low three bits (K reads: eight keys, one
// column) and, for the transposed V reads (four keys of a quad, two columns
// each), distinct bits 0..2 within a quad and distinct bit 3 between the two
// quads of an aligned group of eight, so neither read conflicts with 32 or 64
// LDS banks.
__device__ __forceinline__ int swz(int key) {
  return ((key & 3) << 1) | ((key >> 2) & 1) | ((((key >> 2) ^ (key >> 3)) & 1) << 3);
}

// Raw fp8 blocks: column rc (0..15) of key k sits at rc ^ (k & 15).
__device__ __forceinline__ uint32_t raw_col(int key, int rc) {
  return (uint32_t)(key * kRawKeyBytes + ((rc ^ (key & 15)) << 4));
}

// Byte offset of logical column q of block key `key`.
__device__ __forceinline__ uint32_t key_col(int key, int q) {
  return (uint32_t)(key * kKeyBytes + ((q ^ swz(key)) << 4));
}

// K operand of tile 0 for k-step 0: key lane%16, column lane/16. Column
// lane/16 + 4j is at k_base() ^ (j << 6); tile t is kTileBytes * t further.
__device__ __forceinline__ uint32_t k_base() {
  const int lane = threadIdx.x & 63;
  return key_col(lane & 15, lane >> 4);
}
// Transposed-V operand of tile 0, dims 0..15: in each 16-lane group g, lanes
// 4r..4r+3 read 8 bytes each of key 4g + r. Dims 16dt.. are at v_base() ^ (dt << 5).
__device__ __forceinline__ uint32_t v_base() {
  const int lane = threadIdx.x & 63;
  const int jj = lane & 15;
  return key_col(4 * (lane >> 4) + (jj >> 2), 16 + ((jj & 3) >> 1)) + 8 * (jj & 1);
}

// S^T for one 16-key tile over head_dim 128 (4 k-steps); kx[j] = k_base() ^ (j << 6).
__device__ __forceinline__ floatx4 score16(uint32_t tile, const uint32_t* kx, const u32x4* qv) {
  u32x4 kf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kf[j] = lds_read_b128(tile + kx[j]);
  floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) c = mfma_16x16x32(as_bf16x8(kf[j]), as_bf16x8(qv[j]), c);
  return c;
}

// V^T operand of dims 16dt .. 16dt+15 for 4 keys per lane group; vx = v_base() ^ (dt << 5).
__device__ __forceinline__ u32x2 vtr(uint32_t tile, uint32_t vx) {
  return lds_read_tr16(tile + vx);
}

struct TileCtx {
  int seq, kvh, qtok0, ntok, lo, hi, nsplit, first_pos, nrows;
  int new_start, cu0;  // first position of the step's new tokens, the sequence's first token
};

__device__ __forceinline__ TileCtx tile_ctx(const GqaArgs& a, const Tile& tile, const SeqInfo& s) {
  TileCtx t;
  t.seq = tile.seq;
  t.kvh = tile.kvh;
  t.nsplit = 1;
  if (tile.split >= 0) {
    int lo_all, hi_all, chunk;
    decode_range(a, s, &lo_all, &hi_all);
    split_plan(hi_all - lo_all, a.geo.split_keys, a.geo.max_splits, &t.nsplit, &chunk);
    t.qtok0 = 0;
    t.ntok = s.q_len;
    t.lo = lo_all + tile.split * chunk;
    t.hi = min(hi_all, t.lo + chunk);
  } else {
    t.qtok0 = tile.qtok0;
    t.ntok = min(a.geo.bq, s.q_len - t.qtok0);
    const int first = s.kv_len - s.q_len + t.qtok0;
    t.lo = a.geo.window > 0 ? max(0, first - a.geo.window + 1) : 0;
    t.hi = min(first + t.ntok, s.kv_cap);
  }
  t.first_pos = s.kv_len - s.q_len + t.qtok0;
  t.nrows = t.ntok * a.geo.group;
  t.new_start = a.new_kv != nullptr ? s.kv_len - s.q_len : 0x7fffffff;
  t.cu0 = s.cu0;
  return t;
}

// Waits until at most `ahead` blocks of this wave's DMA are outstanding
// (each block is kIPW instructions).
template <int kIPW>
__device__ __forceinline__ void wait_blocks_ahead(int ahead) {
  if (ahead <= 0)
    wait_vmcnt<0>();
  else if (ahead == 1)
    wait_vmcnt<kIPW>();
  else if (ahead == 2)
    wait_vmcnt<2 * kIPW>();
  else
    wait_vmcnt<3 * kIPW>();
}

// Writes a tile's result: with the keys split over the four waves their
// softmax states are merged first (through `scratch`, LDS the key pipeline no
// longer uses: 4*16*(kD + 2) floats); then either a split partial (m, l, acc)
// or the normalised output rows.
__device__ __forceinline__ void finish_tile(const GqaArgs& a, const Tile& tile, const TileCtx& t,
                                            const SeqInfo& s, floatx4 (&acc)[8], float m_run,
                                            float l_run, bool keysplit, bool wave_active,
                                            bool row_ok, int r, float* scratch) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int G = a.geo.group;
  // Row normaliser of this wave: the four lanes of a row each summed a quarter.
  float l_row = wave_sum_xor<16>(l_run);
  l_row = wave_sum_xor<32>(l_row);
  float m_row = m_run;
  if (keysplit) {
    // Merge the four waves' states (disjoint key tiles) through LDS.
    float* accs = scratch;            // [4][16][128]
    float* mls = accs + 4 * 16 * kD;  // [4][16][2]
    const int hl = lane & 15;
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<floatx4*>(accs + (wave * 16 + hl) * kD + 16 * dt + 4 * g) = acc[dt];
    if (g == 0) {
      mls[(wave * 16 + hl) * 2] = m_run;
      mls[(wave * 16 + hl) * 2 + 1] = l_row;
    }
    __syncthreads();
    if (wave != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mls[(w * 16 + hl) * 2]);
    float wt[4];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = M == -INFINITY ? 0.f : fast_exp2(mls[(w * 16 + hl) * 2] - M);
      L += wt[w] * mls[(w * 16 + hl) * 2 + 1];
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const floatx4 x = *reinterpret_cast<const floatx4*>(accs + (w * 16 + hl) * kD + 16 * dt + 4 * g);
        o[0] += wt[w] * x[0];
        o[1] += wt[w] * x[1];
        o[2] += wt[w] * x[2];
        o[3] += wt[w] * x[3];
      }
      acc[dt] = o;
    }
    m_row = M;
    l_row = L;
  } else if (!wave_active) {
    return;
  }

  if (tile.split >= 0 && t.nsplit > 1) {
    const int64_t pidx = ((int64_t)t.seq * a.num_kv_heads + t.kvh) * a.geo.max_splits + tile.split;
    if (row_ok) {
      // The split's output normalised by its own row sum (pack_part: fp16
      // for fp8 pools, bf16 for bf16 pools), with (m, l) in fp32.
      uint16_t* pa = a.part_acc + (pidx * kPartRows + r) * kD;
      const float inv_l = l_row > 0.f ? 1.f / l_row : 0.f;
      const bool f16 = a.kv_dtype != DT_BF16;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<u32x2*>(pa + 16 * dt + 4 * g) =
            u32x2{pack_part(acc[dt][0] * inv_l, acc[dt][1] * inv_l, f16),
                  pack_part(acc[dt][2] * inv_l, acc[dt][3] * inv_l, f16)};
      if (g == 0) {
        float* pm = a.part_ml + (pidx * kPartRows + r) * 2;
        pm[0] = m_row;
        pm[1] = l_row;
      }
    }
    return;
  }
  if (!row_ok) return;
  const float inv = l_row > 0.f ? a.v_scale / l_row : 0.f;
  const int tok = s.cu0 + t.qtok0 + r / G;
  const int head = t.kvh * G + r % G;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)tok * a.num_q_heads + head) * kD;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w;
    w[0] = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
    w[1] = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * g) = w;
  }
}

// Log2-domain logits of a raw score s = q.k: s * scale * log2(e), or with
// the soft cap c, c * tanh(s * scale / c) * log2(e). The exact capped form
// takes tanh(z) as 1 - 2 / (e^{2z} + 1) with the hardware exp2 and
// reciprocal, i.e. c2 - c3 / (2^{s * c1} + 1); the series form (CapSeries)
// serves a wave whose scores all lie within its range.
struct LogitConsts {
  float c1, c2, c3;
  CapSeries cs;
};

template <bool CAP>
__device__ __forceinline__ LogitConsts logit_consts(const GqaArgs& a) {
  LogitConsts k;
  k.c1 = CAP ? 2.f * kLog2e * a.score_scale / a.soft_cap : a.score_scale * kLog2e;
  k.c2 = a.soft_cap * kLog2e;
  k.c3 = 2.f * a.soft_cap * kLog2e;
  k.cs = CAP ? cap_series(a.soft_cap, a.score_scale) : CapSeries{0.f, 0.f, 0.f, 0.f, 0.f};
  return k;
}

// The logits of the NT groups of four raw scores a wave holds, in place.
// With the cap, one branch for the whole wave: the series when no score
// exceeds its range (lanes masked afterwards count too, except NaN, which
// the maximum ignores), else the exact form.
template <bool CAP, int NT>
__device__ __forceinline__ void to_logits(floatx4* sv, const LogitConsts& k) {
  if constexpr (!CAP) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[t][i] *= k.c1;
  } else {
    float am = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(sv[t][i]));
    if (!wave_any(am > k.cs.smax3)) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[t][i] = cap_series3_eval(k.cs, sv[t][i], 0.f);
    } else if (!wave_any(am > k.cs.smax)) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[t][i] = cap_series_eval(k.cs, sv[t][i], 0.f);
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sv[t][i] = k.c2 - k.c3 * __builtin_amdgcn_rcpf(fast_exp2(sv[t][i] * k.c1) + 1.f);
    }
  }
}

template <int KV_DT, int NST, bool CAP>
__device__ void process_tile(const GqaArgs& a, const Tile& tile, TileSmem<KV_DT, NST>& sm,
                             int ps_log2) {
  // DMA instructions per wave per block (1 KB each, four waves).
  constexpr int kIPW = (KV_DT == DT_BF16 ? kStageBytes : kRawStageBytes) / 1024 / kWaves;
  constexpr int kEB = KV_DT == DT_BF16 ? 2 : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int g = lane >> 4;
  const int G = a.geo.group;
  const SeqInfo s = seq_info(a, tile.seq);
  const TileCtx t = tile_ctx(a, tile, s);
  const bool keysplit = t.nrows <= 16;
  const int W = a.geo.window;

  // This lane's row: in key-split mode all waves hold rows 0..15.
  const int r = (keysplit ? 0 : wave * 16) + (lane & 15);
  const bool row_ok = r < t.nrows;
  const bool wave_active = keysplit || wave * 16 < t.nrows;
  const int qpos = row_ok ? t.first_pos + r / G : kNegBig;

  u32x4 qv[4];
  {
    const int tok = s.cu0 + t.qtok0 + (row_ok ? r / G : 0);
    const int head = t.kvh * G + (row_ok ? r % G : 0);
    const int64_t q0 = ((int64_t)tok * a.num_q_heads + head) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = load_q8(a.q, q0 + 32 * j + 8 * g, a.q_dtype);
      qv[j] = v;
    }
  }

  floatx4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int kb0 = (t.lo / kBN) * kBN;
  const int nblk = t.hi > kb0 ? cdiv_i(t.hi - kb0, kBN) : 0;
  const int32_t* table = a.page_indices + (int64_t)t.seq * a.pages_per_seq;
  const int ps_mask = (1 << ps_log2) - 1;
  int pwin = kb0 >> ps_log2;
  for (int i = tid; i < kPageWin; i += kThreads) {
    const int lp = pwin + i;
    sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
  }
  __syncthreads();

  const int64_t token_bytes = (int64_t)2 * a.num_kv_heads * kD * kEB;
  const char* kv_head = (const char*)a.kv + (int64_t)(2 * t.kvh) * kD * kEB;
  const char* new_head = (const char*)a.new_kv + (int64_t)(2 * t.kvh) * kD * kEB;
  const uint32_t sbase = lds_addr(sm.stage);
  const uint32_t dma_stride = KV_DT == DT_BF16 ? kStageBytes : kRawStageBytes;
  const uint32_t conv = sbase + NST * kRawStageBytes;  // fp8: converted stage

  auto issue = [&](int b) {
    const int kb = kb0 + b * kBN;
    if (((kb + kBN - 1) >> ps_log2) - pwin >= kPageWin) {
      wg_barrier();
      pwin = kb >> ps_log2;
      for (int i = tid; i < kPageWin; i += kThreads) {
        const int lp = pwin + i;
        sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
      }
      __syncthreads();
    }
    // Row address of block key 16*wave + lane%16 (the same in each 16-lane
    // group); every DMA instruction below takes its keys' rows by readlane.
    const int key = kb + 16 * wave + (lane & 15);
    const char* row = (const char*)kZeroKV;
    bool cache_row = false;  // key's row is a valid pool row
    if (key >= t.lo && key < t.hi) {
      if (key >= t.new_start) {
        row = new_head + (int64_t)(t.cu0 + key - t.new_start) * token_bytes;
      } else {
        const int page = sm.pages[(key >> ps_log2) - pwin];
        if (page >= 0 && page < a.total_num_pages) {
          row = kv_head + (((int64_t)page << ps_log2) + (key & ps_mask)) * token_bytes;
          cache_row = true;
        }
      }
    }
    const uint32_t rlo = (uint32_t)(uintptr_t)row;
    const uint32_t rhi = (uint32_t)((uintptr_t)row >> 32);
    const uint32_t st = sbase + (uint32_t)(b % NST) * dma_stride;
    constexpr int kKeysPerDma = KV_DT == DT_BF16 ? 2 : 4;
    constexpr int kKeysLog2 = KV_DT == DT_BF16 ? 1 : 2;
    const int sub = KV_DT == DT_BF16 ? lane >> 5 : lane >> 4;  // key of this lane in the DMA
    // When all 16 keys are pool rows and a page holds a whole instruction's
    // keys (they are kKeysPerDma-aligned), those keys are consecutive rows:
    // one scalar base (the first key's row) plus a per-lane offset.
    if (ps_log2 >= kKeysLog2 && __builtin_amdgcn_ballot_w64(!cache_row) == 0) {
#pragma unroll
      for (int ii = 0; ii < kIPW; ++ii) {
        const uint32_t l = __builtin_amdgcn_readlane(rlo, kKeysPerDma * ii);
        const uint32_t h = __builtin_amdgcn_readlane(rhi, kKeysPerDma * ii);
        const char* base = (const char*)(((uint64_t)h << 32) | l);
        const int kk = kKeysPerDma * ii + sub;  // key within this wave's 16
        const uint32_t col = KV_DT == DT_BF16 ? (uint32_t)(((lane & 31) ^ swz(kk)) << 4)
                                              : (uint32_t)(((lane & 15) ^ kk) << 4);
        const int c = wave * kIPW + ii;  // 1 KB slot of the stage
        dma_b128_s(base, (uint32_t)sub * (uint32_t)token_bytes + col,
                   __builtin_amdgcn_readfirstlane(st + (uint32_t)c * 1024), keysplit);
      }
      return;
    }
#pragma unroll
    for (int ii = 0; ii < kIPW; ++ii) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < kKeysPerDma; ++k) {
        const uint32_t l = __builtin_amdgcn_readlane(rlo, kKeysPerDma * ii + k);
        const uint32_t h = __builtin_amdgcn_readlane(rhi, kKeysPerDma * ii + k);
        lo = sub == k ? l : lo;
        hi = sub == k ? h : hi;
      }
      const char* base = (const char*)(((uint64_t)hi << 32) | lo);
      const int kk = kKeysPerDma * ii + sub;  // key within this wave's 16
      const char* src = KV_DT == DT_BF16 ? base + (((lane & 31) ^ swz(kk)) << 4)
                                         : base + (((lane & 15) ^ kk) << 4);
      const int c = wave * kIPW + ii;  // 1 KB slot of the stage
      dma_b128(src, __builtin_amdgcn_readfirstlane(st + (uint32_t)c * 1024), keysplit);
    }
  };

  const LogitConsts lk = logit_consts<CAP>(a);
  // Keys [klo, khi) of this wave's share of a block are visible to every row
  // of the wave (rows past the tile's end do not count): the mask can be skipped.
  auto all_visible = [&](int klo, int khi) -> bool {
    const bool ok = !row_ok || (klo >= t.lo && khi <= t.hi && khi - 1 <= qpos &&
                                (W <= 0 || klo > qpos - W));
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
  };
  uint32_t kx[4], vx[8];
  {
    const uint32_t kb_ = k_base(), vb_ = v_base();
#pragma unroll
    for (int j = 0; j < 4; ++j) kx[j] = kb_ ^ (uint32_t)(j << 6);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vx[dt] = vb_ ^ (uint32_t)(dt << 5);
  }

  drain_vmem_before_loop();
  // Prologue: the first NST-1 blocks in flight.
  for (int b = 0; b < NST - 1 && b < nblk; ++b) issue(b);
  for (int b = 0; b < nblk; ++b) {
    if (b + NST - 1 < nblk) issue(b + NST - 1);
    // Blocks issued after block b: min(NST-1, nblk-1-b).
    wait_blocks_ahead<kIPW>(min(NST - 1, nblk - 1 - b));
    // bf16 decode tiles: each wave moves and reads only its own 16 keys of a
    // block (its own 8 KB of the stage), so its vmcnt wait is all it needs.
    // Prefill-class tiles share every key, and fp8 blocks are widened by all
    // waves together: those synchronise the workgroup.
    const bool shared = !keysplit || KV_DT != DT_BF16;
    if (shared) wg_barrier();
    uint32_t cur = sbase + (uint32_t)(b % NST) * dma_stride;
    if (KV_DT != DT_BF16) {
      // Widen the raw block: thread tid takes raw column tid/16 (16 fp8
      // values: bf16 columns 2(tid/16) and 2(tid/16) + 1) of keys tid%16 + 16i,
      // so sixteen consecutive lanes touch sixteen keys.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = (tid & 15) + 16 * i, rc = tid >> 4;
        const u32x4 w = lds_read_b128(cur + raw_col(key, rc));
        const u32x2 b0 = kv8x4_to_bf16x4<KV_DT>(w[0]);
        const u32x2 b1 = kv8x4_to_bf16x4<KV_DT>(w[1]);
        const u32x2 b2 = kv8x4_to_bf16x4<KV_DT>(w[2]);
        const u32x2 b3 = kv8x4_to_bf16x4<KV_DT>(w[3]);
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
            (__attribute__((address_space(3))) char*)(uintptr_t)(conv + key_col(key, 2 * rc))) =
            u32x4{b0[0], b0[1], b1[0], b1[1]};
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
            (__attribute__((address_space(3))) char*)(uintptr_t)(conv + key_col(key, 2 * rc + 1))) =
            u32x4{b2[0], b2[1], b3[0], b3[1]};
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
      wg_barrier();
      cur = conv;
    }
    const int kb = kb0 + b * kBN;
    if (keysplit) {
      // One 16-key tile per wave; PV on v_mfma_f32_16x16x16_bf16.
      floatx4 sv = score16(cur + kTileBytes * wave, kx, qv);
      to_logits<CAP, 1>(&sv, lk);
      float mblk = -INFINITY;
      if (all_visible(kb + 16 * wave, kb + 16 * wave + 16)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mblk = fmaxf(mblk, sv[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 16 * wave + 4 * g + i;
          const bool vis =
              key >= t.lo && key < t.hi && key <= qpos && (W <= 0 || key > qpos - W);
          sv[i] = vis ? sv[i] : -INFINITY;
          mblk = fmaxf(mblk, sv[i]);
        }
      }
      mblk = wave_max_xor<16>(mblk);
      mblk = wave_max_xor<32>(mblk);
      const bool need = mblk > m_run + kLazyTau;
      if (wave_any(need)) {
        const float m_new = need ? mblk : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;  // rows not moving keep scale 1
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
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
        l_run += p[0] + p[1] + p[2] + p[3];
        pb[0] = pack_bf16x2(p[0], p[1]);
        pb[1] = pack_bf16x2(p[2], p[3]);
      }
      u32x2 vt[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vt[dt] = vtr(cur + kTileBytes * wave, vx[dt]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] = mfma_16x16x16(vt[dt], pb, acc[dt]);
    } else if (wave_active) {
      floatx4 sv[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sv[kt] = score16(cur + kTileBytes * kt, kx, qv);
      to_logits<CAP, 4>(sv, lk);
      float mblk = -INFINITY;
      if (all_visible(kb, kb + kBN)) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mblk = fmaxf(mblk, sv[kt][i]);
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb + 16 * kt + 4 * g + i;
            const bool vis =
                key >= t.lo && key < t.hi && key <= qpos && (W <= 0 || key > qpos - W);
            sv[kt][i] = vis ? sv[kt][i] : -INFINITY;
            mblk = fmaxf(mblk, sv[kt][i]);
          }
      }
      mblk = wave_max_xor<16>(mblk);
      mblk = wave_max_xor<32>(mblk);
      const bool need = mblk > m_run + kLazyTau;
      if (wave_any(need)) {
        const float m_new = need ? mblk : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;  // rows not moving keep scale 1
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          acc[dt][0] *= alpha;
          acc[dt][1] *= alpha;
          acc[dt][2] *= alpha;
          acc[dt][3] *= alpha;
        }
        m_run = m_new;
      }
      u32x4 pb[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
      if (m_run != -INFINITY) {
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[kt][i] = fast_exp2(sv[kt][i] - m_run);
            psum += sv[kt][i];
          }
        l_run += psum;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          pb[ks][0] = pack_bf16x2(sv[2 * ks][0], sv[2 * ks][1]);
          pb[ks][1] = pack_bf16x2(sv[2 * ks][2], sv[2 * ks][3]);
          pb[ks][2] = pack_bf16x2(sv[2 * ks + 1][0], sv[2 * ks + 1][1]);
          pb[ks][3] = pack_bf16x2(sv[2 * ks + 1][2], sv[2 * ks + 1][3]);
        }
      }
#pragma unroll
      for (int dt0 = 0; dt0 < 8; dt0 += 4) {
        u32x4 vf[4][2];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const u32x2 v0 = vtr(cur + kTileBytes * (2 * ks), vx[dt0 + d]);
            const u32x2 v1 = vtr(cur + kTileBytes * (2 * ks + 1), vx[dt0 + d]);
            vf[d][ks] = u32x4{v0[0], v0[1], v1[0], v1[1]};
          }
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            acc[dt0 + d] = mfma_16x16x32(as_bf16x8(vf[d][ks]), as_bf16x8(pb[ks]), acc[dt0 + d]);
        sched_fence();
      }
    }
    if (shared) wg_barrier();
  }

  finish_tile(a, tile, t, s, acc, m_run, l_run, keysplit, wave_active, row_ok, r,
              reinterpret_cast<float*>(sm.stage));
}

template <int KV_DT, int NST, bool CAP>
__global__ void __launch_bounds__(kThreads) gqa_tile_kernel(GqaArgs a, int ps_log2) {
  __shared__ __attribute__((aligned(16))) TileSmem<KV_DT, NST> sm;
  const int count = a.counters[0];
  for (;;) {
    if (threadIdx.x == 0) sm.tile = atomicAdd(&a.counters[1], 1);
    __syncthreads();
    const int ti = sm.tile;
    __syncthreads();
    if (ti >= count) break;
    const Tile tile = a.tiles[ti];
    process_tile<KV_DT, NST, CAP>(a, tile, sm, ps_log2);
    __syncthreads();
  }
}

// ------------------------------------------------------- fp8 decode kernel --
//
// Decode-class tiles of an fp8 pool whenever the prefill-class tiles go to the
// prefill kernel, so every tile here has at most 16 rows. Blocks of 128 keys
// land raw (256 bytes per key, 32 KB, two stages) and are never widened in
// LDS: wave w owns keys 32w .. 32w+31 of each block as two 16-key score tiles
// and widens its own operands in registers (v_cvt_scalef32_pk_bf16_fp8,
// exact). K comes from ds_read_b64 (eight dims of one key per lane). The two
// score tiles leave keys 4g..4g+3 and 16+4g..16+4g+3 in lane group g, which is
// exactly the B operand (P^T) of one 16x16x32 PV MFMA per 16 value dims, and
// V^T for it comes from the raw rows through ds_read_b64_tr_b8 (eight keys of
// one dim per lane). Each wave moves and reads only its own keys, so the
// waves run without workgroup barriers. Against the 64-key path this doubles
// the bytes in flight per workgroup and drops the widening pass.
constexpr int kBN8 = 128;                          // keys per block
constexpr int kRaw8Stage = kBN8 * kRawKeyBytes;    // 32768
constexpr int kStages8 = 2;
constexpr int kIPW8 = kRaw8Stage / 1024 / kWaves;  // DMA instructions per wave per block (8)
constexpr int kWaveKeys8 = kBN8 / kWaves;          // keys per wave per block (32)

struct Dec8Smem {
  char stage[kStages8 * kRaw8Stage];
  int pages[kPageWin];
  int tile;
};
static_assert(4 * 16 * (kD + 2) * sizeof(float) <= sizeof(Dec8Smem::stage), "merge scratch");

// Raw column rc (16 bytes: 0..7 K dims 16rc.., 8..15 V dims 16(rc-8)..) of key
// k of a wave's 32 sits at rc ^ sw8(k). sw8 is one-to-one on each 16-key score
// tile (the K reads) and on the keys {4g..4g+3, 16+4g..16+4g+3 : g = 2h, 2h+1}
// that half h of the wave names in a transposed V read, so neither read has
// bank conflicts.
__device__ __forceinline__ int sw8(int key) { return (key & 15) ^ (((key >> 4) & 1) << 3); }

// S^T(16 keys x 16 rows) += K(16 x 128) Q^T(128 x 16) on one fp8 MFMA
// (v_mfma_f32_16x16x128_f8f6f4, both operands OCP E4M3, no block scaling).
// Lane l holds row l%16 of either operand over one 32-byte slice of the
// contraction; the two operands only have to use the same slice per lane (a
// dot product does not depend on the order of its terms), and the output
// layout is that of the 16x16x32 bf16 form.
__device__ __forceinline__ floatx4 mfma_16x16x128_fp8(const u32x4 (&a)[2], const u32x4 (&b)[2],
                                                      const floatx4& c) {
  typedef int intx8 __attribute__((ext_vector_type(8)));
  const intx8 av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                    (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
  const intx8 bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                    (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
}

// QF8: fp8 queries over an fp8 pool: the scores run on the fp8 MFMA straight
// from the raw K rows (a product of two E4M3 values is exact in fp32, as it
// is after widening both to bf16); otherwise K is widened to bf16.
template <int KV_DT, bool CAP, bool QF8>
__device__ void process_decode8(const GqaArgs& a, const Tile& tile, Dec8Smem& sm, int ps_log2) {
  static_assert(!QF8 || KV_DT == DT_FP8, "fp8 scores need an fp8 pool");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int g = lane >> 4;
  const int G = a.geo.group;
  const SeqInfo s = seq_info(a, tile.seq);
  const TileCtx t = tile_ctx(a, tile, s);
  const int W = a.geo.window;
  // Every wave holds rows 0..15 (query token, q head) of the tile.
  const int r = lane & 15;
  const bool row_ok = r < t.nrows;
  const int qpos = row_ok ? t.first_pos + r / G : kNegBig;

  // Q^T: bf16 (widened on load) for four 16x16x32 k-steps, or with QF8 the
  // raw fp8 bytes of dims 32g .. 32g + 31 for one 16x16x128 step.
  u32x4 qv[QF8 ? 2 : 4];
  {
    const int tok = s.cu0 + t.qtok0 + (row_ok ? r / G : 0);
    const int head = t.kvh * G + (row_ok ? r % G : 0);
    const int64_t q0 = ((int64_t)tok * a.num_q_heads + head) * kD;
    if constexpr (QF8) {
      const u32x4* qp = reinterpret_cast<const u32x4*>((const uint8_t*)a.q + q0 + 32 * g);
#pragma unroll
      for (int j = 0; j < 2; ++j) qv[j] = row_ok ? qp[j] : u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok) v = load_q8(a.q, q0 + 32 * j + 8 * g, a.q_dtype);
        qv[j] = v;
      }
    }
  }

  floatx4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int kb0 = (t.lo / kBN8) * kBN8;
  const int nblk = t.hi > kb0 ? cdiv_i(t.hi - kb0, kBN8) : 0;
  const int32_t* table = a.page_indices + (int64_t)t.seq * a.pages_per_seq;
  const int ps_mask = (1 << ps_log2) - 1;
  int pwin = kb0 >> ps_log2;
  for (int i = tid; i < kPageWin; i += kThreads) {
    const int lp = pwin + i;
    sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
  }
  __syncthreads();

  const int64_t token_bytes = (int64_t)2 * a.num_kv_heads * kD;
  const char* kv_head = (const char*)a.kv + (int64_t)(2 * t.kvh) * kD;
  const char* new_head = (const char*)a.new_kv + (int64_t)(2 * t.kvh) * kD;
  const uint32_t sbase = lds_addr(sm.stage);

  // Block b: wave w moves its own 32 keys, four per instruction (lane L takes
  // 16 bytes of key L/16: raw column (L%16) ^ sw8(key), so LDS position L%16
  // of the key holds that column).
  auto issue = [&](int b) {
    const int kb = kb0 + b * kBN8;
    if (((kb + kBN8 - 1) >> ps_log2) - pwin >= kPageWin) {
      wg_barrier();
      pwin = kb >> ps_log2;
      for (int i = tid; i < kPageWin; i += kThreads) {
        const int lp = pwin + i;
        sm.pages[i] = lp < a.pages_per_seq ? table[lp] : -1;
      }
      __syncthreads();
    }
    const int key = kb + kWaveKeys8 * wave + (lane & 31);
    const char* row = (const char*)kZeroKV;
    bool cache_row = false;  // key's row is a valid pool row
    if (key >= t.lo && key < t.hi) {
      if (key >= t.new_start) {
        row = new_head + (int64_t)(t.cu0 + key - t.new_start) * token_bytes;
      } else {
        const int page = sm.pages[(key >> ps_log2) - pwin];
        if (page >= 0 && page < a.total_num_pages) {
          row = kv_head + (((int64_t)page << ps_log2) + (key & ps_mask)) * token_bytes;
          cache_row = true;
        }
      }
    }
    const uint32_t rlo = (uint32_t)(uintptr_t)row;
    const uint32_t rhi = (uint32_t)((uintptr_t)row >> 32);
    const uint32_t st = sbase + (uint32_t)(b % kStages8) * kRaw8Stage +
                        (uint32_t)wave * (kWaveKeys8 * kRawKeyBytes);
    const int sub = lane >> 4;
    // When all 32 keys are pool rows, the four keys of one instruction
    // (4-aligned, so on one page: pages hold at least 8 keys) are consecutive
    // rows: one scalar base (the first key's row) plus a per-lane offset.
    // (This kernel runs only beside the prefill kernel, whose page size is at
    // least 8.)
    if (__builtin_amdgcn_ballot_w64(!cache_row) == 0) {
#pragma unroll
      for (int ii = 0; ii < kIPW8; ++ii) {
        const uint32_t l = __builtin_amdgcn_readlane(rlo, 4 * ii);
        const uint32_t h = __builtin_amdgcn_readlane(rhi, 4 * ii);
        const char* base = (const char*)(((uint64_t)h << 32) | l);
        const uint32_t voff = (uint32_t)sub * (uint32_t)token_bytes +
                              (uint32_t)(((lane & 15) ^ sw8(4 * ii + sub)) << 4);
        dma_b128_s(base, voff, __builtin_amdgcn_readfirstlane(st + (uint32_t)ii * 1024), true);
      }
      return;
    }
#pragma unroll
    for (int ii = 0; ii < kIPW8; ++ii) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t l = __builtin_amdgcn_readlane(rlo, 4 * ii + k);
        const uint32_t h = __builtin_amdgcn_readlane(rhi, 4 * ii + k);
        lo = sub == k ? l : lo;
        hi = sub == k ? h : hi;
      }
      const char* base = (const char*)(((uint64_t)hi << 32) | lo);
      dma_b128(base + (((lane & 15) ^ sw8(4 * ii + sub)) << 4),
               __builtin_amdgcn_readfirstlane(st + (uint32_t)ii * 1024), true);
    }
  };

  const LogitConsts lk = logit_consts<CAP>(a);

  // K operand (tile tt, k-step j) at ka ^ (j << 5 | tt << 7) + tt * 16 rows:
  // key tt*16 + lane%16, dims 8(g + 4j) .. +7 = half g&1 of raw column 2j + g/2.
  const int km = lane & 15;
  const uint32_t ka = (uint32_t)(km * kRawKeyBytes + (((lane >> 5) ^ km) << 4) + 8 * (g & 1));
  // QF8 K operand (tile tt, 16-byte half hh) at ka8 ^ (tt << 7 | hh << 4) + tt
  // * 16 rows: key tt*16 + km, raw column 2g + hh (sw8 of that key is km ^ 8tt).
  const uint32_t ka8 = (uint32_t)(km * kRawKeyBytes + (((2 * g) ^ km) << 4));
  // V^T operand of dims 16dt.. at va ^ (dt << 4): lanes 2r, 2r+1 of group g
  // name key slot r, i.e. key 4g + r (r < 4) or 16 + 4g + r - 4.
  const int vslot = (lane & 15) >> 1;
  const int vkey = vslot < 4 ? 4 * g + vslot : 16 + 4 * g + (vslot - 4);
  const uint32_t va = (uint32_t)(vkey * kRawKeyBytes + ((8 ^ sw8(vkey)) << 4) + 8 * (lane & 1));

  drain_vmem_before_loop();
  if (nblk > 0) issue(0);
  for (int b = 0; b < nblk; ++b) {
    if (b + 1 < nblk) issue(b + 1);
    // Each wave moves and reads only its own 32 keys (its 8 KB of the stage),
    // so its own vmcnt wait suffices: no workgroup barrier per block.
    wait_blocks_ahead<kIPW8>(min(1, nblk - 1 - b));
    const uint32_t cur = sbase + (uint32_t)(b % kStages8) * kRaw8Stage +
                         (uint32_t)wave * (kWaveKeys8 * kRawKeyBytes);
    const int kw = kb0 + b * kBN8 + kWaveKeys8 * wave;  // first key of this wave's share
    floatx4 sv[2];
    u32x2 vr[8];
    if constexpr (QF8) {
      u32x4 k8[2][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          k8[tt][hh] = lds_read_b128(cur + (ka8 ^ (uint32_t)((tt << 7) | (hh << 4))) +
                                     (uint32_t)(tt * 16 * kRawKeyBytes));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vr[dt] = lds_read_tr8(cur + (va ^ (uint32_t)(dt << 4)));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        sv[tt] = mfma_16x16x128_fp8(k8[tt], qv, floatx4{0.f, 0.f, 0.f, 0.f});
    } else {
      u32x2 kr[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          kr[tt][j] = lds_read_b64(cur + (ka ^ (uint32_t)((j << 5) | (tt << 7))) +
                                   (uint32_t)(tt * 16 * kRawKeyBytes));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vr[dt] = lds_read_tr8(cur + (va ^ (uint32_t)(dt << 4)));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sv[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sv[tt] = mfma_16x16x32(as_bf16x8(kv8x8_to_bf16x8<KV_DT>(kr[tt][j])), as_bf16x8(qv[j]),
                                 sv[tt]);
      }
    }
    // sv[tt][i] of lane group g is key kw + 16tt + 4g + i of row lane%16.
    to_logits<CAP, 2>(sv, lk);
    float mblk = -INFINITY;
    const bool all_vis =
        __builtin_amdgcn_ballot_w64(row_ok && !(kw >= t.lo && kw + kWaveKeys8 <= t.hi &&
                                                kw + kWaveKeys8 - 1 <= qpos &&
                                                (W <= 0 || kw > qpos - W))) == 0;
    if (all_vis) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mblk = fmaxf(mblk, sv[tt][i]);
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kw + 16 * tt + 4 * g + i;
          const bool vis =
              key >= t.lo && key < t.hi && key <= qpos && (W <= 0 || key > qpos - W);
          sv[tt][i] = vis ? sv[tt][i] : -INFINITY;
          mblk = fmaxf(mblk, sv[tt][i]);
        }
    }
    mblk = wave_max_xor<16>(mblk);
    mblk = wave_max_xor<32>(mblk);
    const bool need = mblk > m_run + kLazyTau;
    if (wave_any(need)) {
      const float m_new = need ? mblk : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;  // rows not moving keep scale 1
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        acc[dt][0] *= alpha;
        acc[dt][1] *= alpha;
        acc[dt][2] *= alpha;
        acc[dt][3] *= alpha;
      }
      m_run = m_new;
    }
    u32x4 pb = {0u, 0u, 0u, 0u};
    if (m_run != -INFINITY) {
      float psum = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[tt][i] = fast_exp2(sv[tt][i] - m_run);
          psum += sv[tt][i];
        }
      l_run += psum;
      pb[0] = pack_bf16x2(sv[0][0], sv[0][1]);
      pb[1] = pack_bf16x2(sv[0][2], sv[0][3]);
      pb[2] = pack_bf16x2(sv[1][0], sv[1][1]);
      pb[3] = pack_bf16x2(sv[1][2], sv[1][3]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      acc[dt] = mfma_16x16x32(as_bf16x8(kv8x8_to_bf16x8<KV_DT>(vr[dt])), as_bf16x8(pb), acc[dt]);
  }

  finish_tile(a, tile, t, s, acc, m_run, l_run, true, true, row_ok, r,
              reinterpret_cast<float*>(sm.stage));
}

template <int KV_DT, bool CAP, bool QF8>
__global__ void __launch_bounds__(kThreads) gqa_decode8_kernel(GqaArgs a, int ps_log2) {
  __shared__ __attribute__((aligned(1024))) Dec8Smem sm;
  const int count = a.counters[0];
  for (;;) {
    if (threadIdx.x == 0) sm.tile = atomicAdd(&a.counters[1], 1);
    __syncthreads();
    const int ti = sm.tile;
    __syncthreads();
    if (ti >= count) break;
    const Tile tile = a.tiles[ti];
    process_decode8<KV_DT, CAP, QF8>(a, tile, sm, ps_log2);
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kThreads) gqa_merge_kernel(GqaArgs a) {
  const int seq = blockIdx.x / a.num_kv_heads;
  const int kvh = blockIdx.x % a.num_kv_heads;
  if (seq >= num_seqs_clamped(a)) return;
  const SeqInfo s = seq_info(a, seq);
  if (a.new_kv != nullptr) {
    // The step's new K and V rows of this kv head go to their pool slots. The
    // attention kernels of this call read those keys from new_kv, never from
    // these slots, so the copy needs no ordering against them.
    const int eb = a.kv_dtype == DT_BF16 ? 2 : 1;
    const int chunks = 2 * kD * eb / 16;  // 16-byte pieces of one K+V row pair
    const int64_t ch = 2 * a.num_kv_heads;
    for (int i = threadIdx.x; i < s.q_len * chunks; i += kThreads) {
      const int j = i / chunks, q = i - j * chunks;
      const int pos = s.kv_len - s.q_len + j;
      const int lp = pos / a.page_size;
      const int page = (pos >= 0 && lp < a.pages_per_seq)
                           ? a.page_indices[(int64_t)seq * a.pages_per_seq + lp] : -1;
      if (page < 0 || page >= a.total_num_pages) continue;
      const int64_t slot = (int64_t)page * a.page_size + pos % a.page_size;
      const u32x4* sp = reinterpret_cast<const u32x4*>(
          (const char*)a.new_kv + (((int64_t)(s.cu0 + j) * ch + 2 * kvh) * kD) * eb);
      u32x4* dp = reinterpret_cast<u32x4*>((char*)a.kv_out + ((slot * ch + 2 * kvh) * kD) * eb);
      dp[q] = sp[q];
    }
  }
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
  float mv[kMaxSplits];
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    mv[sp] = sp < nsplit ? a.part_ml[((pbase + sp) * kPartRows + r) * 2] : -INFINITY;
    M = fmaxf(M, mv[sp]);
  }
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      if (sp < nsplit) {
        // Weight l_sp * 2^(m_sp - M) on the split's normalised output.
        const float w = fast_exp2(mv[sp] - M) * a.part_ml[((pbase + sp) * kPartRows + r) * 2 + 1];
        L += w;
        const uint16_t* pa = a.part_acc + ((pbase + sp) * kPartRows + r) * kD + d0;
        const u32x4 x = *reinterpret_cast<const u32x4*>(pa);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float lo, hi;
          unpack_part(x[i], lo, hi, a.kv_dtype != DT_BF16);
          o[2 * i] += w * lo;
          o[2 * i + 1] += w * hi;
        }
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
  if (dt == DT_INT4) {
    // Element idx: nibble idx % 2 of byte idx / 2, two's complement.
    const uint32_t b = reinterpret_cast<const uint8_t*>(base)[idx >> 1];
    const int v = (int)((idx & 1) ? (b >> 4) : (b & 15u));
    return (float)(v >= 8 ? v - 16 : v);
  }
  const uint8_t b = reinterpret_cast<const uint8_t*>(base)[idx];
  float f[4];
  if (dt == DT_INT8)
    i8x4_to_f32((uint32_t)b, f);
  else
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
  const int new_start = a.new_kv != nullptr ? s.kv_len - s.q_len : 0x7fffffff;
  for (int key = lo; key < hi; ++key) {
    // The step's new tokens come from new_kv, the rest from the pool.
    const void* src = a.new_kv;
    int64_t kbase = ((int64_t)(s.cu0 + key - new_start) * ch + 2 * kvh) * D;
    if (key < new_start) {
      const int page = a.page_indices[(int64_t)seq * a.pages_per_seq + key / a.page_size];
      if (page < 0 || page >= a.total_num_pages) continue;
      const int64_t row = (int64_t)page * a.page_size + key % a.page_size;
      src = a.kv;
      kbase = (row * ch + 2 * kvh) * D;
    }
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) {
      const int d = lane + 64 * k;
      if (d < D) part += qf[k] * load_as_f32<float>(src, kbase + d, a.kv_dtype);
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
      const float v = d < D ? load_as_f32<float>(src, kbase + D + d, a.kv_dtype) : 0.f;
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
  // The first q head of each kv head copies this token's K and V rows to the
  // token's pool slot; no key read in this launch comes from that slot.
  if (a.new_kv != nullptr && h % G == 0) {
    const int lp = pos / a.page_size;
    const int page = lp < a.pages_per_seq ? a.page_indices[(int64_t)seq * a.pages_per_seq + lp] : -1;
    if (page >= 0 && page < a.total_num_pages) {
      // Bytes of one head's row (INT4: two values per byte, head_dim even).
      const int64_t hb = a.kv_dtype == DT_INT4 ? D / 2
                         : (int64_t)D * (a.kv_dtype == DT_F32 ? 4 : a.kv_dtype == DT_BF16 ? 2 : 1);
      const int64_t slot = (int64_t)page * a.page_size + pos % a.page_size;
      const uint8_t* sp = (const uint8_t*)a.new_kv + ((int64_t)tok * ch + 2 * kvh) * hb;
      uint8_t* dp = (uint8_t*)a.kv_out + (slot * ch + 2 * kvh) * hb;
      for (int64_t i = lane; i < 2 * hb; i += 64) dp[i] = sp[i];
    }
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

GqaGeometry gqa_geometry(int num_q_heads, int num_kv_heads, int window, int split_keys) {
  GqaGeometry g;
  g.group = num_q_heads / num_kv_heads;
  g.qdec = g.group <= 16 ? 16 / g.group : 0;
  g.bq = g.group <= 64 ? 64 / g.group : 1;
  // Decode split target from the tile table or the caller (a multiple of 64;
  // the split count is capped at kMaxSplits, so the workspace does not depend
  // on it).
  g.split_keys = split_keys;
  g.max_splits = kMaxSplits;
  g.window = window;
  return g;
}

bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim, int group) {
  return (q_dtype == DT_BF16 || q_dtype == DT_FP8) &&
         (kv_dtype == DT_BF16 || kv_dtype == DT_FP8 || kv_dtype == DT_INT8) && head_dim == kD &&
         group >= 1 && group <= 64;
}

size_t gqa_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_q_heads,
                           int num_kv_heads, int head_dim, int window, int* tile_capacity) {
  const GqaGeometry g = gqa_geometry(num_q_heads, num_kv_heads, window, 1024);  // size: split cap only
  const int64_t cap = (int64_t)num_kv_heads *
                      ((int64_t)max_num_tokens / g.bq + max_num_seqs +
                       (int64_t)max_num_seqs * g.max_splits);
  if (tile_capacity) *tile_capacity = (int)cap;
  const int64_t nparts = (int64_t)max_num_seqs * num_kv_heads * g.max_splits;
  size_t bytes = 0;
  bytes += align256((64 + 3 * ((size_t)max_num_seqs + 1)) * sizeof(int32_t));  // counters + offsets
  bytes += align256((size_t)cap * sizeof(Tile));
  bytes += align256((size_t)nparts * kPartRows * 2 * sizeof(float));
  bytes += align256((size_t)nparts * kPartRows * (size_t)head_dim * sizeof(uint16_t));
  return bytes;
}

void gqa_bind_workspace(GqaArgs& a, void* ws) {
  int cap = 0;
  gqa_workspace_bytes(a.max_num_seqs, a.max_num_tokens, a.num_q_heads, a.num_kv_heads,
                      a.head_dim, a.geo.window, &cap);
  a.tile_capacity = cap;
  char* p = (char*)ws;
  a.counters = (int32_t*)p;
  p += align256((64 + 3 * ((size_t)a.max_num_seqs + 1)) * sizeof(int32_t));
  a.tiles = (Tile*)p;
  p += align256((size_t)cap * sizeof(Tile));
  const int64_t nparts = (int64_t)a.max_num_seqs * a.num_kv_heads * a.geo.max_splits;
  a.part_ml = (float*)p;
  p += align256((size_t)nparts * kPartRows * 2 * sizeof(float));
  a.part_acc = (uint16_t*)p;
}

// Library-owned side stream per device (default priority) with its fork and
// join events. When the prefill kernel runs on a batch with room for a real
// prefill share, the decode-class launch goes to the side stream, so its
// workgroups take CUs as the prefill kernel's workgroups run out of tiles
// instead of waiting for the last one. The fork and join cost ~20 us, more
// than the prefill kernel's tail on a batch of decodes, so batches whose token
// capacity leaves fewer than kOverlapMinTokens tokens beyond one per sequence
// stay on one stream (the results are the same either way).
constexpr int64_t kOverlapMinTokens = 2048;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;

// Fork: work later enqueued on the returned stream starts after what `stream`
// holds now. Returns nullptr (caller stays on one stream) if it cannot be set up.
SideStream* side_fork(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  // A caller's stream of another device keeps everything on that stream.
  hipDevice_t sdev = dev;
  if (stream != nullptr && (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev))
    return nullptr;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    // Never create the stream while the caller's stream is being captured
    // (creating a stream mid-capture is not a capturable operation): such a
    // call stays on one stream; the side stream appears on the first call
    // made outside a capture.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (stream != nullptr && hipStreamIsCapturing(stream, &cs) != hipSuccess) return nullptr;
    if (cs != hipStreamCaptureStatusNone) return nullptr;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) {
      ss.s = nullptr;
      return nullptr;
    }
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(ss.s);
      ss.s = nullptr;
      return nullptr;
    }
  }
  // Record and wait under the lock: another caller's fork cannot slip between.
  if (hipEventRecord(ss.fork, stream) != hipSuccess ||
      hipStreamWaitEvent(ss.s, ss.fork, 0) != hipSuccess)
    return nullptr;
  return &ss;
}

hipError_t side_join(SideStream* ss, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_side_mu);
  hipError_t e = hipEventRecord(ss->join, ss->s);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, ss->join, 0);
  return e;
}

hipError_t launch_gqa(const GqaArgs& a, hipStream_t stream) {
  int ps_log2 = 0;
  while ((1 << ps_log2) < a.page_size) ++ps_log2;
  // Up to kPlanLdsSeqs sequences, several planner workgroups share the tile
  // writes (each computes the offsets itself); beyond that, one workgroup.
  const int plan_wgs = a.max_num_seqs <= kPlanLdsSeqs ? kPlanWgs : 1;
  hipLaunchKernelGGL(gqa_plan_kernel, dim3(plan_wgs), dim3(kThreads), 0, stream, a);
  // Two workgroups per CU, each with two stages: one block computing while
  // the next streams in (deeper pipelines at one workgroup per CU measured
  // slower: the compute of a block is then exposed).
  const int grid = max(1, min(a.tile_capacity, num_cus() * 2));
  prof_begin(stream);
  hipStream_t dstream = stream;
  SideStream* side = nullptr;
  if (a.pre_kernel) {
    if (!a.single_stream && (int64_t)a.max_num_tokens - a.max_num_seqs >= kOverlapMinTokens)
      side = side_fork(stream);
    if (side) dstream = side->s;
    // Prefill-class tiles on the eight-wave kernel (one workgroup per CU).
    prof_kernel_begin(stream, 0);
    const hipError_t e = launch_gqa_prefill(a, ps_log2, num_cus(), stream);
    if (e != hipSuccess) {
      // Join the fork even on failure: a capture with an unjoined fork
      // cannot end.
      if (side) (void)side_join(side, stream);
      return e;
    }
    prof_kernel_end(stream, 0);
  }
  prof_kernel_begin(dstream, 1);
  const bool cap = a.soft_cap != 0.f;
#define RPA_TILE_LAUNCH(DT, CAP)                                                         \
  hipLaunchKernelGGL((gqa_tile_kernel<DT, kStages, CAP>), dim3(grid), dim3(kThreads), 0, \
                     dstream, a, ps_log2)
  if (a.kv_dtype == DT_BF16) {
    if (cap)
      RPA_TILE_LAUNCH(DT_BF16, true);
    else
      RPA_TILE_LAUNCH(DT_BF16, false);
  } else if (a.pre_kernel) {
    // Only decode-class tiles are left for this launch: the one-byte decode
    // kernel.
#define RPA_DEC8_LAUNCH(DT, CAP, QF8)                                                      \
  hipLaunchKernelGGL((gqa_decode8_kernel<DT, CAP, QF8>), dim3(grid), dim3(kThreads), 0, \
                     dstream, a, ps_log2)
    if (a.kv_dtype == DT_INT8) {
      if (cap)
        RPA_DEC8_LAUNCH(DT_INT8, true, false);
      else
        RPA_DEC8_LAUNCH(DT_INT8, false, false);
    } else if (a.q_dtype == DT_FP8) {
      if (cap)
        RPA_DEC8_LAUNCH(DT_FP8, true, true);
      else
        RPA_DEC8_LAUNCH(DT_FP8, false, true);
    } else {
      if (cap)
        RPA_DEC8_LAUNCH(DT_FP8, true, false);
      else
        RPA_DEC8_LAUNCH(DT_FP8, false, false);
    }
#undef RPA_DEC8_LAUNCH
  } else if (a.kv_dtype == DT_INT8) {
    if (cap)
      RPA_TILE_LAUNCH(DT_INT8, true);
    else
      RPA_TILE_LAUNCH(DT_INT8, false);
  } else {
    if (cap)
      RPA_TILE_LAUNCH(DT_FP8, true);
    else
      RPA_TILE_LAUNCH(DT_FP8, false);
  }
#undef RPA_TILE_LAUNCH
  prof_kernel_end(dstream, 1);
  if (a.geo.qdec > 0 || a.new_kv != nullptr)
    hipLaunchKernelGGL(gqa_merge_kernel, dim3(a.max_num_seqs * a.num_kv_heads), dim3(kThreads),
                       0, dstream, a);
  hipError_t e = hipGetLastError();
  if (side) {
    const hipError_t j = side_join(side, stream);
    if (e == hipSuccess) e = j;
  }
  prof_end(stream);
  return e;
}

// Scratch of rpa_forward_noalloc: the work list, counters and split partials
// of callers that cannot allocate. Every device the library runs on holds its
// own copy until the process ends, and every call on a device shares it (the
// planner rewrites the counters each call; calls that overlap on one device
// race). In host code `scratch` is only a host-side stand-in for the symbol:
// its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
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
