/*
 * CPU oracle for ragged paged attention — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library. The product path (the HIP library and its Python
 * binding) never calls it and shares no code with it: this file has its own
 * dtype decoders, its own page-table walk and its own masks.
 *
 * Every function is the plain definition written out in fp64, one output row
 * (one query token x one query head) at a time:
 *   gather the row's visible keys through the page table, score them in fp64,
 *   optionally soft-cap, take a max-subtracted softmax over the visible keys
 *   only, and sum the values with those weights.
 *
 * Pages cited (by the short names used throughout this repository):
 *   "RPA v2 page"   tpu-inference 0.12.0, ragged_paged_attention/v2/kernel.py
 *   "MLA v1 page"   tpu-inference 0.11.1, mla/v1/kernel.py
 *   "Sparse page"   sglang-jax, kernels/dsa/sparse_mla_prefill.py
 *
 * Readings taken where the pages leave a step open (each is listed with its
 * reason in the design notes):
 *   - masked keys are excluded from the softmax; on valid input this equals
 *     the pages' finite mask value (replace or add) because every query row
 *     sees at least its own position;
 *   - dequantisation k*k_scale and v*v_scale is exact here (the pages round
 *     it to the query dtype; with power-of-two scales that rounding is exact);
 *   - softmax weights stay fp64 (the pages round them to the value dtype
 *     before the value product);
 *   - the output is fp64; the caller rounds to the output dtype if it wants.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * (dense library attention, hand-derived golden values, closed forms and
 * invariants). No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8_E4M3 = 2, OR_INT8 = 3, OR_INT4 = 4 };
enum { OR_LAYOUT_COMBINED_GQA = 0, OR_LAYOUT_MLA_SPLIT = 1, OR_LAYOUT_MLA_FUSED = 2 };

/* ---- storage decoders (own implementations, from the format definitions) ---- */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
static double dec_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP FP8 E4M3 "fn" variant: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, subnormals for exponent field 0. */
static double dec_e4m3fn(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int m = b & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case OR_FP8_E4M3: return dec_e4m3fn(((const uint8_t*)base)[idx]);
    /* two's-complement byte: the integer it encodes (dequantised by the caller's scale) */
    case OR_INT8: return (double)((const int8_t*)base)[idx];
    /* two values per byte along the innermost index, element 2i in the low
     * four bits of byte i, each a two's-complement nibble -8..7
     * [RPA v2 page: strided_load_kv, eight 4-bit values per 32-bit word] */
    case OR_INT4: {
      const uint8_t b = ((const uint8_t*)base)[idx / 2];
      const int v = (idx % 2 == 0) ? (b & 0xF) : (b >> 4);
      return (double)(v < 8 ? v : v - 16);
    }
  }
  return NAN;
}

static int dtype_bytes(int dtype) {
  return dtype == OR_F32 ? 4 : dtype == OR_BF16 ? 2 : (dtype == OR_FP8_E4M3 || dtype == OR_INT8) ? 1 : 0;
}

/* Visibility of key position t to a query at position p
 * [RPA v2 page: ref_ragged_paged_attention, causal and sliding-window mask;
 *  MLA v1 page: ref_mla_ragged_paged_attention]:
 * masked when t > p, or, with a window W > 0, when t <= p - W. */
static int key_visible(int64_t t, int64_t p, int window) {
  if (t > p) return 0;
  if (window > 0 && t <= p - window) return 0;
  return 1;
}

/* Soft cap: cap * tanh(s / cap), applied after the scale and before the mask
 * [RPA v2 page: ref_ragged_paged_attention]. cap == 0 means "no cap". */
static double apply_cap(double s, double cap) {
  return cap != 0.0 ? cap * tanh(s / cap) : s;
}

/* Softmax-weighted sum over n scored keys; returns the normaliser. Weights are
 * exp(s - max) over the keys given (all of which are visible). */
static double softmax_normaliser(const double* s, int64_t n, double* w) {
  double mx = -INFINITY, sum = 0.0;
  for (int64_t i = 0; i < n; ++i)
    if (s[i] > mx) mx = s[i];
  for (int64_t i = 0; i < n; ++i) {
    w[i] = exp(s[i] - mx);
    sum += w[i];
  }
  return sum;
}

/* Finds the sequence that owns packed query token `tok` by scanning cu_q_lens. */
static int owner_seq(const int32_t* cu_q_lens, int num_seqs, int tok) {
  for (int i = 0; i < num_seqs; ++i)
    if (tok >= cu_q_lens[i] && tok < cu_q_lens[i + 1]) return i;
  return -1;
}

/*
 * GQA ragged paged attention [RPA v2 page: ref_ragged_paged_attention].
 *
 * q        [num_tokens, num_q_heads, head_dim]            (q_dtype)
 * kv_pages [total_num_pages, page_size, 2*num_kv_heads, head_dim] (kv_dtype);
 *          combined head 2h holds K of kv head h, 2h+1 holds V.
 * page_indices [max_num_seqs, pages_per_seq] flattened; kv_lens, cu_q_lens
 * as on the page; num_seqs is the dynamic sequence count.
 * Query r of sequence i sits at position kv_len - q_len + r.
 * q head h reads kv head h / (num_q_heads / num_kv_heads).
 * Stored values are dequantised exactly before use: K by k_scale, V by
 * v_scale, Q by q_scale (the RPA v2 page scales K and V this way; q_scale is
 * the MLA v1 page's scale on the scores, which equals scaling Q).
 * token_list (optional, n_list entries): compute only those packed tokens.
 * out [num_tokens, num_q_heads, head_dim] fp64; rows not computed are left
 * as they were.
 * Returns 0, or a negative code for input the definition does not cover.
 */
int oracle_rpa(const void* q, int q_dtype, int num_tokens, int num_q_heads, int head_dim,
               const void* kv_pages, int kv_dtype, int total_num_pages, int page_size,
               int num_kv_heads, const int32_t* kv_lens, const int32_t* page_indices,
               int pages_per_seq, const int32_t* cu_q_lens, int num_seqs, double sm_scale,
               int sliding_window, double soft_cap, double k_scale, double v_scale,
               double q_scale, const int32_t* token_list, int n_list, double* out) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  if (kv_dtype == OR_INT4 && head_dim % 2 != 0) return -5;
  const int group = num_q_heads / num_kv_heads;
  const int ch = 2 * num_kv_heads;
  for (int i = 0; i < num_seqs; ++i) {
    int ql = cu_q_lens[i + 1] - cu_q_lens[i];
    if (ql < 0 || ql > kv_lens[i]) return -2;
    if ((kv_lens[i] + page_size - 1) / page_size > pages_per_seq) return -3;
    if (cu_q_lens[i + 1] > num_tokens) return -4;
  }
  const int n_rows_tok = token_list ? n_list : (num_seqs > 0 ? cu_q_lens[num_seqs] : 0);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int a = 0; a < n_rows_tok; ++a) {
    for (int h = 0; h < num_q_heads; ++h) {
      const int tok = token_list ? token_list[a] : a;
      const int i = owner_seq(cu_q_lens, num_seqs, tok);
      if (i < 0) continue;
      const int64_t q_len = cu_q_lens[i + 1] - cu_q_lens[i];
      const int64_t kv_len = kv_lens[i];
      const int64_t pos = kv_len - q_len + (tok - cu_q_lens[i]);
      const int kvh = h / group;
      double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
      double* w = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
      int64_t* key_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(kv_len > 0 ? kv_len : 1));
      int64_t n = 0;
      for (int64_t t = 0; t < kv_len; ++t) {
        if (!key_visible(t, pos, sliding_window)) continue;
        const int32_t page = page_indices[(int64_t)i * pages_per_seq + t / page_size];
        if (page < 0 || page >= total_num_pages) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        const int64_t row = (int64_t)page * page_size + t % page_size; /* token row in pool */
        double dot = 0.0;
        const int64_t kbase = (row * ch + 2 * kvh) * head_dim;
        const int64_t qbase = ((int64_t)tok * num_q_heads + h) * head_dim;
        for (int d = 0; d < head_dim; ++d)
          dot += (load_elem(q, q_dtype, qbase + d) * q_scale) *
                 (load_elem(kv_pages, kv_dtype, kbase + d) * k_scale);
        s[n] = apply_cap(dot * sm_scale, soft_cap);
        key_row[n] = row;
        ++n;
      }
      double* o = out + ((int64_t)tok * num_q_heads + h) * head_dim;
      for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
      if (n > 0) {
        const double norm = softmax_normaliser(s, n, w);
        for (int64_t k = 0; k < n; ++k) {
          const int64_t vbase = (key_row[k] * ch + 2 * kvh + 1) * head_dim;
          for (int d = 0; d < head_dim; ++d)
            o[d] += w[k] * (load_elem(kv_pages, kv_dtype, vbase + d) * v_scale);
        }
        for (int d = 0; d < head_dim; ++d) o[d] /= norm;
      }
      free(s);
      free(w);
      free(key_row);
    }
  }
  return bad ? -5 : 0;
}

/*
 * MLA latent attention over an already-updated cache
 * [MLA v1 page: ref_mla_ragged_paged_attention, after update_kv_cache].
 *
 * ql_nope [num_tokens, num_heads, lkv_dim], q_pe [num_tokens, num_heads, r_dim]
 * cache_kv_c [total_num_pages, page_size, kvc_stride] (first lkv_dim used)
 * cache_k_pe [total_num_pages, page_size, kpe_stride] (first r_dim used)
 * Every head shares the one latent per token (MQA):
 *   K_t = [kv_c_t || k_pe_t] (lkv_dim + r_dim), V_t = kv_c_t (lkv_dim).
 * For the fused pool (one array [P, ps, stride] holding [kv_c || k_pe || 0])
 * pass the same pointer for both caches with kpe_col = lkv_dim; otherwise
 * kpe_col = 0.
 * Scales as the page's kernel applies them: scores times sm_scale, k_scale
 * and q_scale (before the cap), the value sum times v_scale.
 */
int oracle_mla(const void* ql_nope, const void* q_pe, int dtype, int num_tokens, int num_heads,
               int lkv_dim, int r_dim, const void* cache_kv_c, int kvc_stride,
               const void* cache_k_pe, int kpe_stride, int kpe_col, int total_num_pages,
               int page_size, const int32_t* kv_lens, const int32_t* page_indices,
               int pages_per_seq, const int32_t* cu_q_lens, int num_seqs, double sm_scale,
               int sliding_window, double soft_cap, double q_scale, double k_scale,
               double v_scale, const int32_t* token_list, int n_list, double* out) {
  for (int i = 0; i < num_seqs; ++i) {
    int ql = cu_q_lens[i + 1] - cu_q_lens[i];
    if (ql < 0 || ql > kv_lens[i]) return -2;
    if ((kv_lens[i] + page_size - 1) / page_size > pages_per_seq) return -3;
    if (cu_q_lens[i + 1] > num_tokens) return -4;
  }
  const int n_rows_tok = token_list ? n_list : (num_seqs > 0 ? cu_q_lens[num_seqs] : 0);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int a = 0; a < n_rows_tok; ++a) {
    for (int h = 0; h < num_heads; ++h) {
      const int tok = token_list ? token_list[a] : a;
      const int i = owner_seq(cu_q_lens, num_seqs, tok);
      if (i < 0) continue;
      const int64_t q_len = cu_q_lens[i + 1] - cu_q_lens[i];
      const int64_t kv_len = kv_lens[i];
      const int64_t pos = kv_len - q_len + (tok - cu_q_lens[i]);
      double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
      double* w = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
      int64_t* key_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(kv_len > 0 ? kv_len : 1));
      int64_t n = 0;
      const int64_t qn = ((int64_t)tok * num_heads + h) * lkv_dim;
      const int64_t qr = ((int64_t)tok * num_heads + h) * r_dim;
      for (int64_t t = 0; t < kv_len; ++t) {
        if (!key_visible(t, pos, sliding_window)) continue;
        const int32_t page = page_indices[(int64_t)i * pages_per_seq + t / page_size];
        if (page < 0 || page >= total_num_pages) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        const int64_t row = (int64_t)page * page_size + t % page_size;
        double dot = 0.0;
        for (int d = 0; d < lkv_dim; ++d)
          dot += load_elem(ql_nope, dtype, qn + d) *
                 load_elem(cache_kv_c, dtype, row * kvc_stride + d);
        for (int d = 0; d < r_dim; ++d)
          dot += load_elem(q_pe, dtype, qr + d) *
                 load_elem(cache_k_pe, dtype, row * kpe_stride + kpe_col + d);
        s[n] = apply_cap(dot * sm_scale * k_scale * q_scale, soft_cap);
        key_row[n] = row;
        ++n;
      }
      double* o = out + ((int64_t)tok * num_heads + h) * lkv_dim;
      for (int d = 0; d < lkv_dim; ++d) o[d] = 0.0;
      if (n > 0) {
        const double norm = softmax_normaliser(s, n, w);
        for (int64_t k = 0; k < n; ++k)
          for (int d = 0; d < lkv_dim; ++d)
            o[d] += w[k] * load_elem(cache_kv_c, dtype, key_row[k] * kvc_stride + d);
        for (int d = 0; d < lkv_dim; ++d) o[d] = o[d] * v_scale / norm;
      }
      free(s);
      free(w);
      free(key_row);
    }
  }
  return bad ? -5 : 0;
}

/*
 * Sparse MLA-latent attention over a fused paged latent pool
 * [Sparse page: _sparse_mla_kernel_chunked_hminor, validity bias and online
 *  softmax; sparse_mla_attention, paged single-sequence and packed-ragged
 *  modes; prefill_write_and_attend_ragged for the token -> request map].
 *
 * q        [S, H, dk]  (dk = dv + rope, e.g. 512 + 64)
 * kv_cache [total_num_pages, page_size, cache_dim]; token (page P, offset o)
 *          is row P*page_size + o; its first dk columns are the latent, the
 *          value is the first dv columns.
 * page_table [ptw]: logical page -> physical page.
 * indices [S, K]: unit ids (one unit = read_block consecutive logical tokens),
 *          -1 = padding. The key set of query s is the multiset
 *          { u*RB + r : k < K, u = indices[s,k] >= 0, r < RB,
 *            u*RB + r <= positions[s], u*RB + r < seq_len };
 *          duplicate units count once per occurrence.
 * out [S, H, dv] fp64; an empty key set gives zeros.
 *
 * Packed-ragged mode (cu_q_lens != NULL): the S queries are the packed tokens
 * of num_seqs requests. Token s belongs to request
 *   rid = min(#{ j in 1..num_seqs : cu_q_lens[j] <= s }, num_seqs - 1)
 * (a right-sided search of s in cu_q_lens[1:], clipped), its causal bound is
 * seq_lens[rid] in place of seq_len, and its unit ids are local to the
 * request: logical page lp is page_table[cu_kv_lens[rid] / page_size + lp],
 * page_table being the packed table of ptw entries.
 */
int oracle_sparse_mla(const void* q, int dtype, int S, int H, int dk, int dv,
                      const void* kv_cache, int total_num_pages, int page_size, int cache_dim,
                      const int32_t* page_table, int ptw, const int32_t* indices, int K,
                      int read_block, const int32_t* positions, int seq_len, double sm_scale,
                      const int32_t* cu_q_lens, const int32_t* seq_lens,
                      const int32_t* cu_kv_lens, int num_seqs,
                      const int32_t* query_list, int n_list, double* out) {
  if (read_block <= 0 || page_size % read_block != 0) return -1;
  if (dk > cache_dim || dv > dk) return -1;
  if (cu_q_lens && (num_seqs <= 0 || !seq_lens || !cu_kv_lens)) return -1;
  const int n_q = query_list ? n_list : S;
  const int64_t max_keys = (int64_t)K * read_block;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int a = 0; a < n_q; ++a) {
    for (int h = 0; h < H; ++h) {
      const int si = query_list ? query_list[a] : a;
      const int64_t qpos = positions[si];
      int64_t kv_bound = seq_len, table_base = 0;
      if (cu_q_lens) {
        int rid = 0;
        for (int j = 1; j <= num_seqs; ++j) rid += cu_q_lens[j] <= si;
        if (rid > num_seqs - 1) rid = num_seqs - 1;
        kv_bound = seq_lens[rid];
        table_base = cu_kv_lens[rid] / page_size;
      }
      double* s = (double*)malloc(sizeof(double) * (size_t)(max_keys > 0 ? max_keys : 1));
      double* w = (double*)malloc(sizeof(double) * (size_t)(max_keys > 0 ? max_keys : 1));
      int64_t* key_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_keys > 0 ? max_keys : 1));
      int64_t n = 0;
      const int64_t qb = ((int64_t)si * H + h) * dk;
      for (int k = 0; k < K; ++k) {
        const int32_t u = indices[(int64_t)si * K + k];
        if (u < 0) continue;
        for (int r = 0; r < read_block; ++r) {
          const int64_t kp = (int64_t)u * read_block + r; /* logical token */
          if (kp > qpos || kp >= kv_bound) continue;
          const int64_t lp = table_base + kp / page_size;
          if (lp < 0 || lp >= ptw) {
#pragma omp atomic write
            bad = 1;
            continue;
          }
          const int32_t page = page_table[lp];
          if (page < 0 || page >= total_num_pages) {
#pragma omp atomic write
            bad = 1;
            continue;
          }
          const int64_t row = (int64_t)page * page_size + kp % page_size;
          double dot = 0.0;
          for (int d = 0; d < dk; ++d)
            dot += load_elem(q, dtype, qb + d) * load_elem(kv_cache, dtype, row * cache_dim + d);
          s[n] = dot * sm_scale;
          key_row[n] = row;
          ++n;
        }
      }
      double* o = out + ((int64_t)si * H + h) * dv;
      for (int d = 0; d < dv; ++d) o[d] = 0.0;
      if (n > 0) {
        const double norm = softmax_normaliser(s, n, w);
        for (int64_t k = 0; k < n; ++k)
          for (int d = 0; d < dv; ++d)
            o[d] += w[k] * load_elem(kv_cache, dtype, key_row[k] * cache_dim + d);
        for (int d = 0; d < dv; ++d) o[d] /= norm;
      }
      free(s);
      free(w);
      free(key_row);
    }
  }
  return bad ? -5 : 0;
}

/*
 * Scatter of new tokens into the paged caches, as a plain byte copy
 * [MLA v1 page: update_kv_cache; Sparse page: prefill_write_and_attend
 *  self-write with -1 slots dropped].
 *
 * Destination of new token j of sequence i (page-table mode):
 *   pos = kv_len - q_len + j, page = page_indices[i*pages_per_seq + pos/ps],
 *   slot = page*ps + pos%ps.
 * Slot-list mode (slot_loc != NULL): token t goes to slot slot_loc[t]; a
 * negative slot is skipped. Tokens are visited sequence-major, so when two
 * tokens name one slot the later one wins.
 *
 * layout COMBINED_GQA: new_a = K [T, heads, dim_a], new_b = V [T, heads, dim_a];
 *   cache_a [P, ps, 2*heads, dim_a]: K to combined head 2h, V to 2h+1.
 * layout MLA_SPLIT: new_a = kv_c [T, dim_a], new_b = k_pe [T, dim_b];
 *   cache_a [P, ps, stride_a], cache_b [P, ps, stride_b]; columns past the
 *   new data are written with zeros (the page pads k_pe up to 128).
 * layout MLA_FUSED: cache_a [P, ps, stride_a] receives [kv_c || k_pe || 0].
 */
int oracle_kv_update(int layout, const void* new_a, const void* new_b, void* cache_a,
                     void* cache_b, int dtype, int total_num_pages, int page_size, int heads,
                     int dim_a, int dim_b, int stride_a, int stride_b, const int32_t* kv_lens,
                     const int32_t* page_indices, int pages_per_seq, const int32_t* cu_q_lens,
                     int num_seqs, const int32_t* slot_loc, int num_tokens) {
  /* Bytes per element; INT4 rows (combined layout only, even dim_a) take
   * dim_a / 2 bytes, two values per byte. */
  const int eb = dtype_bytes(dtype);
  if (eb == 0 && !(dtype == OR_INT4 && layout == OR_LAYOUT_COMBINED_GQA && dim_a % 2 == 0))
    return -1;
  const int64_t row_a = dtype == OR_INT4 ? dim_a / 2 : (int64_t)dim_a * eb;
  const int64_t n_slots = (int64_t)total_num_pages * page_size;
  const int n_tok = slot_loc ? num_tokens : (num_seqs > 0 ? cu_q_lens[num_seqs] : 0);
  for (int t = 0; t < n_tok; ++t) {
    int64_t slot;
    if (slot_loc) {
      slot = slot_loc[t];
      if (slot < 0) continue;
    } else {
      const int i = owner_seq(cu_q_lens, num_seqs, t);
      if (i < 0) continue;
      const int64_t q_len = cu_q_lens[i + 1] - cu_q_lens[i];
      const int64_t pos = kv_lens[i] - q_len + (t - cu_q_lens[i]);
      if (pos < 0) return -2;
      if (pos / page_size >= pages_per_seq) return -3;
      const int32_t page = page_indices[(int64_t)i * pages_per_seq + pos / page_size];
      if (page < 0 || page >= total_num_pages) return -5;
      slot = (int64_t)page * page_size + pos % page_size;
    }
    if (slot >= n_slots) return -5;
    if (layout == OR_LAYOUT_COMBINED_GQA) {
      for (int h = 0; h < heads; ++h) {
        memcpy((char*)cache_a + (slot * 2 * heads + 2 * h) * row_a,
               (const char*)new_a + ((int64_t)t * heads + h) * row_a, (size_t)row_a);
        memcpy((char*)cache_a + (slot * 2 * heads + 2 * h + 1) * row_a,
               (const char*)new_b + ((int64_t)t * heads + h) * row_a, (size_t)row_a);
      }
    } else if (layout == OR_LAYOUT_MLA_SPLIT) {
      char* da = (char*)cache_a + slot * stride_a * eb;
      char* db = (char*)cache_b + slot * stride_b * eb;
      memset(da, 0, (size_t)stride_a * eb);
      memcpy(da, (const char*)new_a + (int64_t)t * dim_a * eb, (size_t)dim_a * eb);
      memset(db, 0, (size_t)stride_b * eb);
      memcpy(db, (const char*)new_b + (int64_t)t * dim_b * eb, (size_t)dim_b * eb);
    } else if (layout == OR_LAYOUT_MLA_FUSED) {
      char* da = (char*)cache_a + slot * stride_a * eb;
      memset(da, 0, (size_t)stride_a * eb);
      memcpy(da, (const char*)new_a + (int64_t)t * dim_a * eb, (size_t)dim_a * eb);
      memcpy(da + (size_t)dim_a * eb, (const char*)new_b + (int64_t)t * dim_b * eb,
             (size_t)dim_b * eb);
    } else {
      return -1;
    }
  }
  return 0;
}

/* Threads an OpenMP region of this library uses (for reporting). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Decoders exported for the pins (tests check them against the format
 * definitions' own worked values). */
double oracle_decode_bf16(uint16_t h) { return dec_bf16(h); }
double oracle_decode_e4m3fn(uint8_t b) { return dec_e4m3fn(b); }
