// Sparse MLA-latent attention [Sparse page: sparse_mla_attention,
// _sparse_mla_kernel_chunked_hminor]: each query attends its own top-k set of
// page units of a fused latent pool. The key is a whole latent row
// [kv_c (512) || k_pe (64)], shared by every head; the value its first 512
// columns.
//  * keys stream through LDS in blocks of 64 rows, moved by
//    global_load_lds_dwordx4 (no register staging) into two stages, so the
//    next block's loads are in flight while the current one is multiplied.
//    One instruction moves the 1 KB latent part of one row; one more moves
//    the 128-byte rope parts of eight rows, so every request is a long run
//    of consecutive bytes;
//  * a block is stored row-major (latent parts, then rope parts); the 16-byte
//    chunks of a row are XOR-swizzled by the row, so the rows read by one
//    MFMA operand fall in distinct LDS banks;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows from LDS, Q^T in VGPRs),
//    V^T for O^T += V^T P^T read straight out of the same rows with
//    ds_read_b64_tr_b16, so the value needs no second copy.
// One workgroup of 4 waves takes one query's 16 heads; each wave owns one
// 16-key tile of every block; the four partial softmax states are merged in
// LDS at the end. The key set is the query's selected units, each resolved
// through the page table [Sparse page: _src paged address computation].
// (The dense MLA path is in mla_decode.hip.)
#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

constexpr int kDl = 512;
constexpr int kDk = 576;
constexpr int kBlk = 64;                                     // keys per block
constexpr int kKvcBytes = kDl * 2;                           // 1024: latent part of a row
constexpr int kKpeBytes = (kDk - kDl) * 2;                   // 128: rope part of a row
constexpr int kKpeOff = kBlk * kKvcBytes;                    // rope parts follow the latent parts
constexpr int kStageBytes = kBlk * (kKvcBytes + kKpeBytes);  // 73728
constexpr int kTileKvc = 16 * kKvcBytes;                     // latent parts of a 16-key tile
constexpr int kTileKpe = 16 * kKpeBytes;                     // rope parts of a 16-key tile
constexpr int kDmaPer8 = 9;                                  // DMA instructions per 8 keys
constexpr int kQSteps = kDk / 32;                            // 18 MFMA k-steps
constexpr int kDvTiles = kDl / 16;                           // 32 output tiles of 16 dims

// Zero row read by keys outside the visible range (1152 bytes of bf16 zeros).
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[kKvcBytes + kKpeBytes] = {0};

// Chunk q (0..63) of a row's latent part sits at q ^ swz(row) (row = key
// within the block; only its low four bits matter): one-to-one on sixteen
// consecutive rows, distinct low three bits on eight, distinct bits 0..2
// within an aligned quad and distinct bit 3 between the two quads of an
// aligned eight, which keeps the K reads (one chunk of 8 or 16 rows) and the
// transposed V reads (two chunks of 4 rows per lane group) conflict free.
__device__ __forceinline__ int swz(int key) {
  return ((key & 3) << 1) | ((key >> 2) & 1) | ((((key >> 2) ^ (key >> 3)) & 1) << 3);
}
// Rope chunk q (0..7) sits at q ^ swz_pe(row): one-to-one on eight
// consecutive rows and on the eight rows of either parity among sixteen.
__device__ __forceinline__ int swz_pe(int key) { return ((key >> 1) & 7) ^ ((key & 1) << 2); }

// Latent row r: columns [0, 512) at a + r*sa, columns [512, 576) at b + r*sb.
struct RowSrc {
  const char* a;
  const char* b;
  int64_t sa, sb;
};

// DMA instruction k (0..8) of block keys [8*grp, 8*grp + 8): k < 8 moves
// the latent part of key 8*grp + k (64 lanes x 16 bytes), k = 8 the rope
// parts of all eight keys (8 keys x 8 lanes). `row` is the physical row of
// block key 8*grp + lane/8, or -1 for a key that reads as zeros; a latent
// instruction takes its row by readlane and uses it as a scalar base with a
// per-lane 32-bit offset.
__device__ __forceinline__ void issue_key_dma(const RowSrc& src, uint32_t stage, int grp, int row,
                                              int k) {
  const int lane = threadIdx.x & 63;
  if (k < 8) {
    const int r = __builtin_amdgcn_readlane(row, 8 * k);
    const int key = 8 * grp + k;
    const char* base = r >= 0 ? src.a + (int64_t)r * src.sa : (const char*)kZeroRow;
    dma_b128_s(base, xor_here((uint32_t)lane << 4, (uint32_t)(swz(key) << 4)),
               __builtin_amdgcn_readfirstlane(stage + (uint32_t)key * kKvcBytes));
  } else {
    const int key = 8 * grp + (lane >> 3);
    const char* base =
        row >= 0 ? src.b + (int64_t)row * src.sb : (const char*)kZeroRow + kKvcBytes;
    dma_b128(base + (((lane & 7) ^ swz_pe(key)) << 4),
             __builtin_amdgcn_readfirstlane(stage + (uint32_t)(kKpeOff + grp * 1024)));
  }
}

// Q^T operand of one wave, lane l = head l%16. The contraction order is free
// as long as K uses the same one: k-step j < 16 covers latent chunk
// 16*(l/16) + j (dims 128(l/16) + 8j ..+7), k-step 16 + m rope chunk
// 2*(l/16) + m.
__device__ __forceinline__ void load_q(u32x4* qv, const uint16_t* q_nope, const uint16_t* q_pe,
                                       bool ok) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    qv[j] = ok ? *reinterpret_cast<const u32x4*>(q_nope + 128 * g + 8 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int m = 0; m < 2; ++m)
    qv[16 + m] = ok ? *reinterpret_cast<const u32x4*>(q_pe + 16 * g + 8 * m) : u32x4{0u, 0u, 0u, 0u};
}

// S^T A operand, key tile 0 (row lane%16): latent k-step j at k_lat() ^ (j << 4),
// rope k-step 16 + m at k_rope() ^ (m << 4); tile t is t*kTileKvc (t*kTileKpe)
// further. Stage bases are multiples of 1024, so the XOR may follow the add.
__device__ __forceinline__ uint32_t k_lat() {
  const int lane = threadIdx.x & 63;
  const int kk = lane & 15;
  return (uint32_t)(kk * kKvcBytes + 256 * (lane >> 4) + (swz(kk) << 4));
}
__device__ __forceinline__ uint32_t k_rope() {
  const int lane = threadIdx.x & 63;
  const int kk = lane & 15;
  return (uint32_t)(kKpeOff + kk * kKpeBytes + (((2 * (lane >> 4)) ^ swz_pe(kk)) << 4));
}
// V^T A operand read with ds_read_b64_tr_b16, key tile 0: in lane group g,
// lanes 4r..4r+3 read 8 bytes each of row 4g + r; dims 16dt .. are at
// v_lat() ^ (dt << 5).
__device__ __forceinline__ uint32_t v_lat() {
  const int lane = threadIdx.x & 63;
  const int jj = lane & 15;
  const int key = 4 * (lane >> 4) + (jj >> 2);
  return (uint32_t)(key * kKvcBytes + ((((jj & 3) >> 1) ^ swz(key)) << 4) + 8 * (jj & 1));
}

// S^T[key, head] for NT 16-key tiles and NH 16-head tiles; lat/rope are the
// lane operand addresses of the first tile (stage included). Each K read
// feeds NH MFMAs; the NT tiles give independent accumulation chains. The K
// reads run AH k-steps ahead of their MFMAs (an LDS round trip takes several
// MFMAs).
template <int NT, int NH, int AH>
__device__ __forceinline__ void score_tiles(floatx4 (&sv)[NT][NH], uint32_t lat, uint32_t rope,
                                            const u32x4 (&qv)[NH][kQSteps]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int h = 0; h < NH; ++h) sv[t][h] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto kread = [&](int j, int t) -> u32x4 {
    return j < 16 ? lds_read_b128((lat ^ (uint32_t)(j << 4)) + t * kTileKvc)
                  : lds_read_b128((rope ^ (uint32_t)((j - 16) << 4)) + t * kTileKpe);
  };
  u32x4 ring[AH][NT];
#pragma unroll
  for (int j = 0; j < AH; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) ring[j][t] = kread(j, t);
#pragma unroll
  for (int j = 0; j < kQSteps; ++j) {
    u32x4 kf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kf[t] = ring[j % AH][t];
      pin_after(kf[t]);  // later reads stay behind this step's operands
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        sv[t][h] = mfma_16x16x32(as_bf16x8(kf[t]), as_bf16x8(qv[h][j]), sv[t][h]);
    if (j + AH < kQSteps) {
#pragma unroll
      for (int t = 0; t < NT; ++t) ring[j % AH][t] = kread(j + AH, t);
    }
  }
}

// Score transform in the exp2 domain: scale, optional soft cap.
__device__ __forceinline__ float score_log2(float s, float sc, float cap) {
  if (cap != 0.f) return cap * tanh_def(s * sc / cap) * kLog2e;
  return s * sc * kLog2e;
}


// ============================================================ sparse ========

constexpr int kSpWaves = 4;
constexpr int kSpThreads = kSpWaves * 64;
constexpr int kSpGroups = kBlk / 8 / kSpWaves;         // 8-key DMA groups per wave (2)
constexpr int kSpIPW = kSpGroups * kDmaPer8;           // DMA instructions per wave per block
constexpr int kSpMaxUnits = 256;
constexpr int kSpAhead = 6;                            // K k-steps read ahead of their MFMAs
constexpr int kSpVAhead = 8;                           // V^T tiles read ahead of their MFMAs

struct SparseShared {
  char stage[2][kStageBytes];
  int unit_row[kSpMaxUnits];
  int unit_id[kSpMaxUnits];
};
static_assert(sizeof(SparseShared) <= 160 * 1024, "sparse LDS budget");

__global__ void __launch_bounds__(kSpThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_kernel(SparseArgs a) {
  __shared__ __attribute__((aligned(1024))) SparseShared sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int g = lane >> 4;
  const int qi = blockIdx.x;
  const int hbase = blockIdx.y * 16;
  const int head = hbase + (lane & 15);
  const bool head_ok = head < a.num_heads;
  const int pos = a.positions[qi];
  const int K = a.top_k;
  const int RB = a.read_block;
  const int ps = a.page_size;

  // Causal bound and page-table base of this query: the call's seq_len and 0
  // for one sequence; for packed requests those of request rid, the number
  // of cu_q_lens[1..num_seqs] at or below qi clipped to the last request
  // [Sparse page: prefill_write_and_attend_ragged, sparse_mla_attention].
  int kv_bound = a.seq_len;
  int64_t tbase = 0;
  if (a.cu_q_lens != nullptr) {
    int lo = 0, hi = a.num_seqs;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_q_lens[mid + 1] <= qi)
        lo = mid + 1;
      else
        hi = mid;
    }
    const int rid = min(lo, a.num_seqs - 1);
    kv_bound = a.seq_lens[rid];
    tbase = a.cu_kv_lens[rid] / ps;
  }

  // Unit table: physical first row of each selected unit (-1 = padding or
  // outside the page table) [Sparse page: _src, paged branch].
  for (int k = tid; k < K; k += kSpThreads) {
    const int u = a.indices[(int64_t)qi * K + k];
    int row = -1;
    if (u >= 0) {
      const int64_t lt = (int64_t)u * RB;
      const int64_t lp = lt / ps;
      const int64_t li = tbase + lp;
      if (li >= 0 && li < a.ptw) {
        const int phys = a.page_table[li];
        if (phys >= 0 && phys < a.total_num_pages) row = phys * ps + (int)(lt - lp * ps);
      }
    }
    sm.unit_row[k] = row;
    sm.unit_id[k] = u;
  }
  __syncthreads();

  u32x4 qv[1][kQSteps];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)qi * a.num_heads + head) * kDk;
    load_q(qv[0], qp, qp + kDl, head_ok);
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

  // Rows of this wave's two 8-key DMA groups of block b (keys 16*wave .. +15,
  // the keys it also multiplies): lane l resolves key 8*gi + l/8 of group gi.
  // The validity of a group's keys comes back as a lane mask (bit 8i: key i).
  auto prep_rows = [&](int b, int* rows, uint64_t* vmask) {
#pragma unroll
    for (int gi = 0; gi < kSpGroups; ++gi) {
      const int kk = b * kBlk + 16 * wave + 8 * gi + (lane >> 3);
      int row = -1;
      if (kk < total) {
        const int unit = kk / RB;
        const int r = kk - unit * RB;
        const int base = sm.unit_row[unit];
        const int kp = sm.unit_id[unit] * RB + r;
        if (base >= 0 && kp <= pos && kp < kv_bound) row = base + r;
      }
      rows[gi] = row;
      vmask[gi] = __builtin_amdgcn_ballot_w64(row >= 0);
    }
  };

  const float sc = a.score_scale;
  const uint32_t klat = k_lat() + wave * kTileKvc;
  const uint32_t krope = k_rope() + wave * kTileKpe;
  const uint32_t vlat = v_lat() + wave * kTileKvc;
  // Validity masks of the blocks in the two stages.
  uint64_t vm_st[2][kSpGroups] = {{0, 0}, {0, 0}};
  // Block b goes to stage b % 2 as soon as every wave is done with block
  // b - 2 there, so while a block is multiplied the next one is in flight,
  // and while a wave waits for that one the block after it is too.
  auto issue_block = [&](int b, uint32_t stage) {
    int rows[kSpGroups];
    prep_rows(b, rows, vm_st[b & 1]);
#pragma unroll
    for (int j = 0; j < kSpIPW; ++j)
      issue_key_dma(src, stage, kSpGroups * wave + j / kDmaPer8, rows[j / kDmaPer8], j % kDmaPer8);
  };
  drain_vmem_before_loop();
  if (nblk > 0) issue_block(0, st0);
  if (nblk > 1) issue_block(1, st1);
  for (int b = 0; b < nblk; ++b) {
    const uint32_t cur = (b & 1) ? st1 : st0;
    // Block b has landed once only block b + 1's loads (if any) are
    // outstanding; the barrier makes every wave's part of it visible.
    if (b + 1 < nblk)
      wait_vmcnt<kSpIPW>();
    else
      wait_vmcnt<0>();
    wg_barrier();
    uint64_t vm_cur[kSpGroups];
    vm_cur[0] = vm_st[b & 1][0];
    vm_cur[1] = vm_st[b & 1][1];
    floatx4 sv2[1][1];
    score_tiles<1, 1, kSpAhead>(sv2, (cur + klat), (cur + krope), qv);
    floatx4 sv = sv2[0][0];
    // Keys 4g + i of this wave's tile: group g/2, bit 8*(4(g&1) + i) of its mask.
    const uint64_t vm = (g >> 1) ? vm_cur[1] : vm_cur[0];
    float mblk = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = ((vm >> (8 * (4 * (g & 1) + i))) & 1ull) != 0;
      const float x = ok ? score_log2(sv[i], sc, 0.f) : -INFINITY;
      sv[i] = x;
      mblk = fmaxf(mblk, x);
    }
    mblk = wave_max_xor<16>(mblk);
    mblk = wave_max_xor<32>(mblk);
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
    {
      // V^T tiles read kSpVAhead tiles ahead of their MFMAs.
      u32x2 vr[kSpVAhead];
#pragma unroll
      for (int d = 0; d < kSpVAhead; ++d) vr[d] = lds_read_tr16((cur + vlat) ^ (uint32_t)(d << 5));
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        u32x2 x = vr[dt % kSpVAhead];
        pin_after(x);
        acc[dt] = mfma_16x16x16(x, pb, acc[dt]);
        if (dt + kSpVAhead < kDvTiles)
          vr[dt % kSpVAhead] = lds_read_tr16(xor_here(cur + vlat, (uint32_t)((dt + kSpVAhead) << 5)));
      }
    }
    if (b + 2 < nblk) {
      // Every wave is done reading stage cur: block b + 2 takes it.
      wg_barrier();
      issue_block(b + 2, cur);
    }
  }
  // The four waves hold the softmax state of disjoint key tiles: merge in LDS.
  float l_row = wave_sum_xor<16>(l_run);
  l_row = wave_sum_xor<32>(l_row);
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

hipError_t launch_sparse_mla(const SparseArgs& a, hipStream_t stream) {
  if (a.top_k > kSpMaxUnits) return hipErrorInvalidValue;
  const int hg = (a.num_heads + 15) / 16;
  prof_begin(stream);
  hipLaunchKernelGGL(sparse_mla_kernel, dim3(a.num_queries, hg), dim3(kSpThreads), 0, stream, a);
  prof_end(stream);
  return hipGetLastError();
}

}  // namespace rpa
