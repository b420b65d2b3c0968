/*
 * rpa.h — C ABI of librpa.so: ragged paged attention on MI355X (gfx950).
 *
 * Four operations, each an asynchronous launch sequence on the caller's HIP
 * stream:
 *   rpa_forward        GQA attention over a packed ragged batch whose K/V live
 *                      in a shared pool of fixed-size pages
 *                      [RPA v2 page: ragged_paged_attention, ref_ragged_paged_attention];
 *   mla_rpa_forward    the MLA latent variant, scatter of the new tokens then
 *                      attention [MLA v1 page: mla_ragged_paged_attention,
 *                      update_kv_cache, ref_mla_ragged_paged_attention];
 *   kv_cache_update    the scatter of new tokens into page/row slots alone
 *                      [MLA v1 page: update_kv_cache; Sparse page:
 *                      prefill_write_and_attend self-write];
 *   sparse_mla_forward attention of each query over its own top-k set of page
 *                      units of the latent pool [Sparse page:
 *                      sparse_mla_attention, _sparse_mla_kernel_chunked_hminor].
 *
 * Pages are cited by short name: "RPA v2 page" (tpu-inference
 * ragged_paged_attention v2 kernel), "MLA v1 page" (tpu-inference MLA ragged
 * paged attention v1 kernel), "Sparse page" (sglang-jax sparse MLA prefill
 * kernel).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is DEVICE memory owned by the caller; the library
 *    never keeps a pointer past the call and never allocates on these paths.
 *    Scratch space is the caller's `workspace` (size from *_workspace_size).
 *  - Layouts are dense row-major in the index order written; element types
 *    are given by rpa_dtype (bf16 = upper half of binary32; fp8 = OCP E4M3FN).
 *  - Calls are asynchronous on `stream` (NULL = the default stream). Unless
 *    rpa_opts.debug_validate is set, no call synchronises with the host.
 *  - rpa_forward on a batch whose token capacity leaves room for a prefill
 *    share runs its decode-class launch on a library-owned stream of the
 *    current device (created on the first such call made outside a stream
 *    capture, default priority, kept until the process ends), forked from
 *    `stream` with an event and joined back into it before the call returns:
 *    to the caller all of the call's work is ordered on `stream`, and the call
 *    can be captured into a graph like any other (a call captured before the
 *    side stream exists stays on `stream`). The side stream is shared by all
 *    callers and threads of a device: calls from several host threads are
 *    serialised on it, and capturing on one thread while another thread
 *    issues eager calls on the same device is not supported.
 *  - On any error the call returns a non-zero rpa_status, launches nothing,
 *    and rpa_last_error() describes the first problem found (thread-local).
 *  - Outputs are written in the query dtype for rpa_forward/mla_rpa_forward
 *    and in fp32 for sparse_mla_forward; results are deterministic (a fixed
 *    reduction order that does not depend on scheduling).
 */
#ifndef RPA_H_
#define RPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (HIP declares `typedef struct ihipStream_t* hipStream_t`). */
struct ihipStream_t;
typedef struct ihipStream_t* rpa_stream_t;

typedef enum {
  RPA_OK = 0,
  RPA_E_INVALID = 1,     /* a value is out of its allowed range */
  RPA_E_SHAPE = 2,       /* sizes disagree with each other */
  RPA_E_DTYPE = 3,       /* element type not accepted for this argument */
  RPA_E_UNSUPPORTED = 4, /* valid input this build does not implement */
  RPA_E_WORKSPACE = 5,   /* workspace missing or smaller than required */
  RPA_E_HIP = 6          /* the HIP runtime reported an error */
} rpa_status;

/* RPA_INT4: signed 4-bit integers (two's complement, -8..7), two per byte
 * along the innermost index, element 2i in the low nibble of byte i; a row
 * of head_dim values takes head_dim / 2 bytes [RPA v2 page:
 * strided_load_kv, eight values per 32-bit word]. KV pools of rpa_forward
 * only. */
typedef enum { RPA_F32 = 0, RPA_BF16 = 1, RPA_FP8_E4M3 = 2, RPA_INT8 = 3, RPA_INT4 = 4 } rpa_dtype;

typedef enum {
  RPA_LAYOUT_COMBINED_GQA = 0, /* [P, ps, 2*Hkv, D]: K of kv head h at 2h, V at 2h+1 */
  RPA_LAYOUT_MLA_SPLIT = 1,    /* kv_c [P, ps, stride_a] and k_pe [P, ps, stride_b] */
  RPA_LAYOUT_MLA_FUSED = 2     /* one pool [P, ps, stride_a] holding [kv_c || k_pe || 0] */
} rpa_cache_layout;

/*
 * Ragged batch description [RPA v2 page: ragged_paged_attention arguments;
 * MLA v1 page: kv_lens / page_indices / cu_q_lens]. All four arrays are
 * device int32. Only the first *num_seqs sequences are read.
 *   cu_q_lens    [max_num_seqs + 1]  packed query offsets; sequence i owns query
 *                                    tokens [cu_q_lens[i], cu_q_lens[i+1]).
 *   kv_lens      [max_num_seqs]      keys of sequence i, INCLUDING this step's
 *                                    new tokens; query r of sequence i sits at
 *                                    position kv_lens[i] - q_len_i + r.
 *   page_indices [max_num_seqs * pages_per_seq]  logical page lp of sequence i
 *                                    is physical page page_indices[i*pps + lp].
 *   num_seqs     [1]                 the dynamic sequence count.
 * max_num_seqs, pages_per_seq and max_num_tokens are host-known capacities
 * (max_num_tokens = rows of the packed query/output arrays).
 */
typedef struct {
  const int32_t* cu_q_lens;
  const int32_t* kv_lens;
  const int32_t* page_indices;
  const int32_t* num_seqs;
  int32_t max_num_seqs;
  int32_t pages_per_seq;
  int32_t max_num_tokens;
} rpa_ragged_meta;

/*
 * Attention options [RPA v2 page: ragged_paged_attention keyword arguments].
 *   sm_scale       multiplies q.k (default 1.0).
 *   sliding_window 0 = none; W > 0 masks keys at or before position - W.
 *   soft_cap       0 = none; otherwise scores become cap * tanh(score / cap)
 *                  after scaling and before masking.
 *   k_scale/v_scale multiply stored K and V (1.0 = none); used for fp8 and
 *                  int8 pools. mla_rpa_forward applies them as the MLA v1
 *                  page's kernel does: k_scale on the scores, v_scale on the
 *                  value sum.
 *   q_scale        multiplies the scores, i.e. dequantises stored queries
 *                  (1.0 = none) [MLA v1 page: flash_attention q_scale]; used
 *                  with fp8 queries.
 *   debug_validate 1 = copy the metadata to the host (synchronising the stream)
 *                  and run the value checks the pages run at runtime
 *                  (0 < q_len <= kv_len, page count <= pages_per_seq, page ids
 *                  in [0, P), total tokens <= max_num_tokens,
 *                  num_seqs <= max_num_seqs) before launching.
 *   split_keys     0 = tile sizes from the library's shape-keyed table (see
 *                  rpa_tile_config); otherwise a multiple of 64 in [64, 2^20]
 *                  fixing them, as the MLA v1 page's caller fixes its block
 *                  sizes: rpa_forward's target keys per decode split (at most
 *                  16 splits per sequence, larger chunks beyond that) and
 *                  mla_rpa_forward's smallest share of the key space per
 *                  workgroup. Results agree to rounding for every value.
 * Masked keys are excluded from the softmax exactly; on valid input this is
 * what the pages' finite mask value produces, since every query sees at least
 * its own position.
 */
typedef struct {
  float sm_scale;
  int32_t sliding_window;
  float soft_cap;
  float k_scale;
  float v_scale;
  int32_t debug_validate;
  int32_t split_keys;
  float q_scale;
} rpa_opts;

/* Fills *opts with the defaults above. */
void rpa_opts_init(rpa_opts* opts);

/*
 * Tile sizes a call will use [RPA v2 page: get_tuned_block_sizes; MLA v1
 * page: the block-size arguments of mla_ragged_paged_attention].
 *   path RPA_TILE_DECODE_SPLIT: rpa_forward's decode splits; kv_dtype, head
 *        counts and head_dim as rpa_forward gets them.
 *   path RPA_TILE_MLA_SHARE: mla_rpa_forward's smallest share; pass the
 *        latent dtype, num_q_heads = num_heads, num_kv_heads = 1 and
 *        head_dim = lkv_dim + r_dim.
 * The table is keyed by pool dtype, head_dim, num_kv_heads and the context
 * capacity meta->pages_per_seq * page_size (host values only; no device read).
 * out->keys: keys per split / per share; out->max_splits: split cap (decode
 * path; 0 otherwise); out->table_row: matching table row, -1 for the built-in
 * default, -2 when opts->split_keys fixed it.
 */
#define RPA_TILE_DECODE_SPLIT 0
#define RPA_TILE_MLA_SHARE 1
typedef struct {
  int32_t keys;
  int32_t max_splits;
  int32_t table_row;
} rpa_tile_params;
rpa_status rpa_tile_config(int32_t path, rpa_dtype kv_dtype, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                           const rpa_ragged_meta* meta, const rpa_opts* opts,
                           rpa_tile_params* out);

/* Thread-local description of the last error (empty string after success). */
const char* rpa_last_error(void);

/*
 * Thread-local name of the kernel path the last successful rpa_forward call on
 * this thread took (empty before the first call):
 *   "gqa_mfma"          work-list planner, MFMA tile kernel(s), split merge;
 *   "gqa_mfma_prefill"  as gqa_mfma, with prefill-class tiles on the
 *                       eight-wave prefill kernel;
 *   "gqa_generic"       one wave per (query token, q head) on plain vector
 *                       ALU, no MFMA: taken for fp32 queries, head_dim != 128,
 *                       page sizes that are not powers of two and pointers not
 *                       16-byte aligned. Correct, but far slower.
 */
const char* rpa_last_path(void);

/*
 * Profiling hook for benchmarks. `start` and `stop` are hipEvent_t handles
 * created by the caller (NULL, NULL turns the hook off). While set, each
 * rpa_forward / mla_rpa_forward / sparse_mla_forward call on this host thread
 * records `start` on its stream right before its main attention kernel (for
 * rpa_forward: the first of its prefill-tile and decode-tile kernels) and
 * `stop` right after it (the last of them), so hipEventElapsedTime(start,
 * stop) is the attention kernels' duration without the work-list planner and
 * the split merge. The library does not own or destroy the events.
 */
void rpa_set_profile_events(void* start, void* stop);

/*
 * Per-kernel profiling hook of rpa_forward. While set (both events of a pair
 * non-NULL), each rpa_forward call on this host thread records pre_start /
 * pre_stop around its prefill-tile kernel (launched only when that kernel
 * serves the call's shapes) and dec_start / dec_stop around its decode-tile
 * kernel. NULL pairs turn the respective hook off. The library does not own
 * or destroy the events.
 */
void rpa_set_profile_events_split(void* pre_start, void* pre_stop, void* dec_start,
                                  void* dec_stop);

/*
 * Workspace bytes rpa_forward needs for these capacities (host-only query;
 * depends only on meta's capacities max_num_seqs and max_num_tokens and on
 * the head counts and head_dim, never on device values or the page size).
 */
size_t rpa_workspace_size(const rpa_ragged_meta* meta, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim);

/*
 * GQA ragged paged attention [RPA v2 page: ragged_paged_attention].
 *   q         [max_num_tokens, num_q_heads, head_dim], q_dtype (F32, BF16, or
 *             FP8_E4M3 with opts->q_scale; fp8 queries need the MFMA path:
 *             head_dim 128, a BF16/FP8/INT8 pool, power-of-two page size,
 *             16-byte aligned q, kv_pages and out, else RPA_E_UNSUPPORTED).
 *   kv_pages  [total_num_pages, page_size, 2*num_kv_heads, head_dim], kv_dtype
 *             (F32, BF16, FP8_E4M3, or INT8 / INT4 with k_scale/v_scale
 *             dequantising the integers; INT4 needs an even head_dim and runs
 *             on the generic kernel); combined layout, K at 2h, V at 2h+1.
 *   new_kv    NULL, or the step's new tokens [max_num_tokens, 2*num_kv_heads,
 *             head_dim] in kv_dtype, laid out as a pool row (K of kv head h at
 *             2h, V at 2h+1): the call then equals kv_cache_update of these
 *             rows followed by attention, in one launch sequence. Keys at
 *             positions >= kv_len - q_len are read from new_kv, and each new
 *             row is copied to its pool slot (page_indices, kv_len - q_len + j)
 *             by a launch that reads nothing it writes; a slot past the table
 *             or on an invalid page is skipped. Two tokens mapping to one slot
 *             are an error (debug_validate). kv_pages is written only then.
 *   out       [max_num_tokens, num_q_heads, head_dim], q_dtype (BF16 for fp8
 *             queries). Rows of tokens at or past cu_q_lens[num_seqs] are not
 *             written.
 * Requires num_q_heads % num_kv_heads == 0. q head h reads kv head
 * h / (num_q_heads / num_kv_heads). The pool is read only at rows below each
 * sequence's kv_len - q_len (below kv_len without new_kv), so unused pages and
 * stale table entries are never read. Without new_kv the new tokens must
 * already be in the pool (call kv_cache_update first).
 */
rpa_status rpa_forward(const void* q, rpa_dtype q_dtype, int32_t num_q_heads, int32_t head_dim,
                       void* kv_pages, rpa_dtype kv_dtype, int32_t total_num_pages,
                       int32_t page_size, int32_t num_kv_heads, const void* new_kv,
                       const rpa_ragged_meta* meta, const rpa_opts* opts, void* out,
                       void* workspace, size_t workspace_bytes, rpa_stream_t stream);

/*
 * rpa_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory or create streams (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments and results are those of rpa_forward. The scratch space (work
 * list, counters, split partials) is a static array in the library, one per
 * device, of rpa_noalloc_scratch_bytes() bytes (96 MiB), held until the
 * process ends. Capacities whose rpa_workspace_size exceeds it are rejected
 * with RPA_E_WORKSPACE before any launch. All launches stay on `stream` (no
 * side stream). Every call on a device shares that device's array and leaves
 * its contents behind (the planner resets what must start at zero on each
 * call): calls that overlap in time on one device race, so serialise them.
 */
rpa_status rpa_forward_noalloc(const void* q, rpa_dtype q_dtype, int32_t num_q_heads,
                               int32_t head_dim, void* kv_pages, rpa_dtype kv_dtype,
                               int32_t total_num_pages, int32_t page_size, int32_t num_kv_heads,
                               const void* new_kv, const rpa_ragged_meta* meta,
                               const rpa_opts* opts, void* out, rpa_stream_t stream);

/* Bytes of the static per-device scratch array of rpa_forward_noalloc. */
size_t rpa_noalloc_scratch_bytes(void);

/*
 * Scatter new tokens into a paged cache, in place [MLA v1 page: update_kv_cache;
 * Sparse page: prefill_write_and_attend self-write].
 *   Page-table mode (slot_loc == NULL, meta required): new token j of
 *     sequence i (packed row cu_q_lens[i] + j) goes to position
 *     p = kv_lens[i] - q_len_i + j, i.e. page page_indices[i*pps + p/ps],
 *     row p % ps.
 *   Slot-list mode (slot_loc != NULL, device int32 [num_tokens]): token t goes
 *     to flat row slot_loc[t] of the [P*ps] rows; negative slots are skipped.
 *   layout COMBINED_GQA: new_a = K [T, heads, dim_a], new_b = V [T, heads, dim_a],
 *     cache_a [P, ps, 2*heads, dim_a]; cache_b unused (may be NULL).
 *   layout MLA_SPLIT: new_a = kv_c [T, dim_a], new_b = k_pe [T, dim_b];
 *     cache_a [P, ps, stride_a], cache_b [P, ps, stride_b]; the columns past
 *     the new data are written with zeros.
 *   layout MLA_FUSED: cache_a [P, ps, stride_a] receives [kv_c || k_pe || 0].
 * The copy is bitwise. Two tokens naming one slot is invalid input (rejected
 * under debug_validate via opts; otherwise which one lands is unspecified).
 * num_tokens = rows of new_a/new_b (for page-table mode, tokens at or past
 * cu_q_lens[num_seqs] are ignored).
 */
rpa_status kv_cache_update(rpa_cache_layout layout, const void* new_a, const void* new_b,
                           void* cache_a, void* cache_b, rpa_dtype dtype, int32_t total_num_pages,
                           int32_t page_size, int32_t heads, int32_t dim_a, int32_t dim_b,
                           int32_t stride_a, int32_t stride_b, int32_t num_tokens,
                           const rpa_ragged_meta* meta, const int32_t* slot_loc,
                           int32_t debug_validate, rpa_stream_t stream);

/* Workspace bytes mla_rpa_forward needs for these capacities (max_num_seqs,
 * max_num_tokens, num_heads, lkv_dim; host-only). */
size_t mla_rpa_workspace_size(const rpa_ragged_meta* meta, int32_t num_heads, int32_t lkv_dim);

/*
 * MLA ragged paged attention [MLA v1 page: mla_ragged_paged_attention].
 *   ql_nope [max_num_tokens, num_heads, lkv_dim], q_pe [.., num_heads, r_dim] (BF16)
 *   new_kv_c [max_num_tokens, lkv_dim], new_k_pe [max_num_tokens, r_dim]; when
 *     both are NULL the caches are used as they are (attention only).
 *   cache_kv_c [total_num_pages, page_size, kvc_stride] and
 *   cache_k_pe [total_num_pages, page_size, kpe_stride], updated in place
 *     (k_pe pad columns written as zeros).
 *   out [max_num_tokens, num_heads, lkv_dim] (BF16).
 * Every head attends the one latent per token: K_t = [kv_c_t || k_pe_t],
 * V_t = kv_c_t. The result equals scattering the new tokens into the caches
 * and then attending; one launch does both: keys at positions >= kv_len - q_len
 * are read from new_kv_c / new_k_pe, and each token's row is written to its
 * cache slot by the same work-group that finished attending for that token,
 * so no read of the caches in this call depends on those writes. Two tokens of
 * one call that map to the same cache slot are an error (debug_validate).
 * Scores are multiplied by sm_scale, k_scale and q_scale before the cap and the
 * value sum by v_scale, as the page's kernel applies its scales.
 * This build implements lkv_dim = 512, r_dim = 64, bf16.
 */
rpa_status mla_rpa_forward(const void* ql_nope, const void* q_pe, const void* new_kv_c,
                           const void* new_k_pe, void* cache_kv_c, void* cache_k_pe,
                           rpa_dtype dtype, int32_t num_heads, int32_t lkv_dim, int32_t r_dim,
                           int32_t kvc_stride, int32_t kpe_stride, int32_t total_num_pages,
                           int32_t page_size, const rpa_ragged_meta* meta, const rpa_opts* opts,
                           void* out, void* workspace, size_t workspace_bytes,
                           rpa_stream_t stream);

/*
 * Sparse MLA-latent attention, paged single-sequence mode [Sparse page:
 * sparse_mla_attention, _sparse_mla_kernel_chunked_hminor].
 *   q          [num_queries, num_heads, kv_lora_rank + rope_dim] (BF16)
 *   kv_cache   [total_num_pages, page_size, cache_dim] (BF16); token (page P,
 *              offset o) is row P*page_size + o; cache_dim >= kv_lora_rank+rope_dim.
 *   page_table [ptw]: logical page -> physical page.
 *   indices    [num_queries, top_k] unit ids (one unit = read_block consecutive
 *              logical tokens); -1 = padding.
 *   positions  [num_queries] query positions (causal bound).
 *   out        [num_queries, num_heads, kv_lora_rank] FP32.
 * Query s attends the multiset of keys u*RB + r (u = indices[s,k] >= 0, r < RB)
 * with u*RB + r <= positions[s] and < seq_len; a unit listed twice counts twice;
 * an empty set gives zeros. sm_scale is required (> 0, finite).
 * Requires read_block % 16 == 0 and page_size % read_block == 0; this build
 * handles top_k <= 256 units per query (RPA_E_UNSUPPORTED above).
 * Logical pages at or past ptw are clamped to ptw-1 for the address and masked.
 * Needs no workspace.
 */
rpa_status sparse_mla_forward(const void* q, const void* kv_cache, const int32_t* page_table,
                              const int32_t* indices, const int32_t* positions, int32_t seq_len,
                              int32_t num_queries, int32_t num_heads, int32_t top_k,
                              int32_t read_block, int32_t page_size, int32_t total_num_pages,
                              int32_t cache_dim, int32_t ptw, int32_t kv_lora_rank,
                              int32_t rope_dim, float sm_scale, float* out, rpa_stream_t stream);

/*
 * Sparse MLA-latent attention, packed-ragged mode: the tokens of num_seqs
 * requests packed along one axis, as the dense MLA path and the indexer lay
 * them out [Sparse page: prefill_write_and_attend_ragged, sparse_mla_attention
 * ragged branch]. One launch covers prefill chunks and decodes (a request
 * with one token is the S == 1 case).
 *   q          [num_tokens, num_heads, 576] (BF16), out [num_tokens, num_heads, 512] FP32.
 *   kv_cache   [total_num_pages, page_size, cache_dim] (BF16), as in sparse_mla_forward.
 *   page_indices [ptw]: the packed physical page list; request r's logical
 *              page lp is page_indices[cu_kv_lens[r] / page_size + lp].
 *   indices    [num_tokens, top_k] request-local unit ids (-1 = padding).
 *   positions  [num_tokens] absolute query positions (causal bound).
 *   cu_q_lens  [num_seqs + 1] non-decreasing token offsets; token t belongs to
 *              request min(#{j in 1..num_seqs : cu_q_lens[j] <= t}, num_seqs - 1),
 *              so tokens past cu_q_lens[num_seqs] count as the last request's.
 *   seq_lens   [num_seqs] per-request kv length (keys at or past it are masked).
 *   cu_kv_lens [num_seqs + 1] page-aligned kv offsets into page_indices.
 * All arrays are device memory owned by the caller; num_seqs is a host value.
 * Key set, duplicates and empty sets as in sparse_mla_forward; a logical page
 * outside page_indices (index < 0 or >= ptw) or a physical page outside the
 * pool is masked. No workspace. Same shape limits as sparse_mla_forward;
 * RPA_E_SHAPE if num_seqs <= 0.
 */
rpa_status sparse_mla_forward_ragged(const void* q, const void* kv_cache,
                                     const int32_t* page_indices, int32_t ptw,
                                     const int32_t* indices, const int32_t* positions,
                                     const int32_t* cu_q_lens, const int32_t* seq_lens,
                                     const int32_t* cu_kv_lens, int32_t num_seqs,
                                     int32_t num_tokens, int32_t num_heads, int32_t top_k,
                                     int32_t read_block, int32_t page_size,
                                     int32_t total_num_pages, int32_t cache_dim,
                                     int32_t kv_lora_rank, int32_t rope_dim, float sm_scale,
                                     float* out, rpa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H_ */
