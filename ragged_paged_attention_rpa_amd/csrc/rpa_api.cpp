// Host side of librpa.so: argument checks, workspace carving and launches.
//
// Static checks follow the pages' compile-time validators [RPA v2 page:
// static_validate_inputs; MLA v1 page: static_validate_inputs; Sparse page:
// sparse_mla_attention argument checks]; the value checks run only when the
// caller asks for them (debug_validate), as the pages' runtime validators do
// [RPA v2 page: dynamic_validate_inputs; MLA v1 page: dynamic_validate_inputs].
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <set>
#include <string>
#include <vector>

#include "../../include/rpa.h"
#include "rpa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local const char* g_last_path = "";
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;
thread_local hipEvent_t g_prof_k[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};

rpa_status fail(rpa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

// A roctx range around one call's launches, named after the operation and
// the sizes that shape its tiles, like the pages' profiler scope names [MLA
// v1 page: mla_ragged_paged_attention, named_scope]. rocprofv3
// --marker-trace records them; without a profiler attached a range costs one
// formatted string and two library calls.
class TraceRange {
 public:
  explicit TraceRange(const char* fmt, ...) {
    char buf[160];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    roctxRangePushA(buf);
  }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

rpa_status ok() {
  g_last_error.clear();
  return RPA_OK;
}

rpa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RPA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int dtype_bytes(rpa_dtype d) {
  switch (d) {
    case RPA_F32: return 4;
    case RPA_BF16: return 2;
    case RPA_FP8_E4M3: return 1;
    case RPA_INT8: return 1;
  }
  return 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

rpa_status check_meta(const rpa_ragged_meta* m, bool need_pages) {
  if (!m) return fail(RPA_E_INVALID, "meta is NULL");
  if (!m->cu_q_lens || !m->kv_lens || !m->num_seqs || (need_pages && !m->page_indices))
    return fail(RPA_E_INVALID, "meta has a NULL array");
  if (m->max_num_seqs <= 0) return fail(RPA_E_SHAPE, "max_num_seqs=%d must be > 0", m->max_num_seqs);
  if (need_pages && m->pages_per_seq <= 0)
    return fail(RPA_E_SHAPE, "pages_per_seq=%d must be > 0", m->pages_per_seq);
  if (m->max_num_tokens < 0) return fail(RPA_E_SHAPE, "max_num_tokens=%d must be >= 0", m->max_num_tokens);
  return RPA_OK;
}

rpa_status check_opts(const rpa_opts* o) {
  if (!o) return fail(RPA_E_INVALID, "opts is NULL");
  if (!std::isfinite(o->sm_scale)) return fail(RPA_E_INVALID, "sm_scale must be finite");
  if (o->sliding_window < 0)
    return fail(RPA_E_INVALID, "sliding_window=%d must be positive (0 = none)", o->sliding_window);
  if (!std::isfinite(o->soft_cap)) return fail(RPA_E_INVALID, "soft_cap must be finite (0 = none)");
  if (!std::isfinite(o->k_scale) || !std::isfinite(o->v_scale) || !std::isfinite(o->q_scale))
    return fail(RPA_E_INVALID, "k_scale, v_scale and q_scale must be finite");
  if (o->split_keys != 0 && (o->split_keys < 64 || o->split_keys > (1 << 20) || o->split_keys % 64))
    return fail(RPA_E_INVALID, "split_keys=%d must be 0 (tile table) or a multiple of 64 in [64, 2^20]",
                o->split_keys);
  return RPA_OK;
}

// Keys per decode split (path kTileGqaDecode) or smallest MLA share
// (kTileMlaShare): the caller's split_keys, else the tile table's row.
int resolve_tile_keys(int path, const rpa_opts* o, int kv_dtype, int head_dim, int num_kv_heads,
                      const rpa_ragged_meta* meta, int page_size, int* row) {
  if (o->split_keys > 0) {
    if (row) *row = -2;
    return o->split_keys;
  }
  const int64_t ctx = (int64_t)meta->pages_per_seq * page_size;
  return rpa::tile_keys(path, kv_dtype, head_dim, num_kv_heads, ctx, row);
}

struct HostMeta {
  std::vector<int32_t> cu, kv, pages;
  int32_t ns = 0;
};

rpa_status fetch_meta(const rpa_ragged_meta* m, bool need_pages, hipStream_t stream,
                      HostMeta* h) {
  h->cu.resize(m->max_num_seqs + 1);
  h->kv.resize(m->max_num_seqs);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "debug_validate sync");
  e = hipMemcpy(h->cu.data(), m->cu_q_lens, h->cu.size() * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(h->kv.data(), m->kv_lens, h->kv.size() * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(&h->ns, m->num_seqs, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && need_pages) {
    h->pages.resize((size_t)m->max_num_seqs * m->pages_per_seq);
    e = hipMemcpy(h->pages.data(), m->page_indices, h->pages.size() * 4, hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) return hip_status(e, "debug_validate copy");
  return RPA_OK;
}

// Runtime value checks [RPA v2 page: dynamic_validate_inputs; MLA v1 page:
// dynamic_validate_inputs].
rpa_status validate_values(const rpa_ragged_meta* m, const HostMeta& h, int page_size,
                           int total_num_pages) {
  if (h.ns < 0 || h.ns > m->max_num_seqs)
    return fail(RPA_E_INVALID, "num_seqs=%d must be in [0, max_num_seqs=%d]", h.ns, m->max_num_seqs);
  if (h.cu[h.ns] > m->max_num_tokens)
    return fail(RPA_E_INVALID, "total q tokens %d must be <= max_num_tokens=%d", h.cu[h.ns],
                m->max_num_tokens);
  for (int i = 0; i < h.ns; ++i) {
    const int q_len = h.cu[i + 1] - h.cu[i];
    const int kv_len = h.kv[i];
    if (q_len < 0 || q_len > kv_len)
      return fail(RPA_E_INVALID, "sequence %d: require 0 <= q_len=%d <= kv_len=%d", i, q_len, kv_len);
    const int cnt = (kv_len + page_size - 1) / page_size;
    if (cnt > m->pages_per_seq)
      return fail(RPA_E_INVALID, "sequence %d: %d pages needed for kv_len=%d > pages_per_seq=%d", i,
                  cnt, kv_len, m->pages_per_seq);
    for (int p = 0; p < cnt; ++p) {
      const int pg = h.pages[(size_t)i * m->pages_per_seq + p];
      if (pg < 0 || pg >= total_num_pages)
        return fail(RPA_E_INVALID, "sequence %d: page id %d at logical page %d not in [0, %d)", i,
                    pg, p, total_num_pages);
    }
  }
  return RPA_OK;
}

// No two new tokens of the batch may name one cache slot [MLA v1 page:
// update_kv_cache visits them in order, so the later one would win; here the
// scatter is parallel and such input is rejected].
rpa_status check_update_slots(const rpa_ragged_meta* meta, const HostMeta& h, int page_size) {
  std::set<int64_t> seen;
  for (int i = 0; i < h.ns; ++i) {
    const int q_len = h.cu[i + 1] - h.cu[i];
    for (int j = 0; j < q_len; ++j) {
      const int pos = h.kv[i] - q_len + j;
      const int64_t slot =
          (int64_t)h.pages[(size_t)i * meta->pages_per_seq + pos / page_size] * page_size +
          pos % page_size;
      if (!seen.insert(slot).second)
        return fail(RPA_E_INVALID, "sequence %d token %d: slot %lld written twice", i, j,
                    (long long)slot);
    }
  }
  return RPA_OK;
}

#define RPA_TRY(x)                 \
  do {                             \
    rpa_status _s = (x);           \
    if (_s != RPA_OK) return _s;   \
  } while (0)

}  // namespace

namespace rpa {
void prof_begin(hipStream_t stream) {
  if (g_prof_start) (void)hipEventRecord(g_prof_start, stream);
}
void prof_end(hipStream_t stream) {
  if (g_prof_stop) (void)hipEventRecord(g_prof_stop, stream);
}
void prof_kernel_begin(hipStream_t stream, int k) {
  if (g_prof_k[k][0]) (void)hipEventRecord(g_prof_k[k][0], stream);
}
void prof_kernel_end(hipStream_t stream, int k) {
  if (g_prof_k[k][1]) (void)hipEventRecord(g_prof_k[k][1], stream);
}
}  // namespace rpa

extern "C" {

void rpa_set_profile_events(void* start, void* stop) {
  if (start && stop) {
    g_prof_start = reinterpret_cast<hipEvent_t>(start);
    g_prof_stop = reinterpret_cast<hipEvent_t>(stop);
  } else {
    g_prof_start = nullptr;
    g_prof_stop = nullptr;
  }
}

void rpa_set_profile_events_split(void* pre_start, void* pre_stop, void* dec_start,
                                  void* dec_stop) {
  void* e[2][2] = {{pre_start, pre_stop}, {dec_start, dec_stop}};
  for (int k = 0; k < 2; ++k) {
    const bool on = e[k][0] && e[k][1];
    g_prof_k[k][0] = on ? reinterpret_cast<hipEvent_t>(e[k][0]) : nullptr;
    g_prof_k[k][1] = on ? reinterpret_cast<hipEvent_t>(e[k][1]) : nullptr;
  }
}

void rpa_opts_init(rpa_opts* o) {
  if (!o) return;
  o->sm_scale = 1.0f;
  o->sliding_window = 0;
  o->soft_cap = 0.0f;
  o->k_scale = 1.0f;
  o->v_scale = 1.0f;
  o->debug_validate = 0;
  o->split_keys = 0;
  o->q_scale = 1.0f;
}

rpa_status rpa_tile_config(int32_t path, rpa_dtype kv_dtype, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                           const rpa_ragged_meta* meta, const rpa_opts* opts,
                           rpa_tile_params* out) {
  if (!out || !meta || !opts) return fail(RPA_E_INVALID, "out, meta and opts must be non-NULL");
  RPA_TRY(check_opts(opts));
  if (path != RPA_TILE_DECODE_SPLIT && path != RPA_TILE_MLA_SHARE)
    return fail(RPA_E_INVALID, "path=%d must be RPA_TILE_DECODE_SPLIT or RPA_TILE_MLA_SHARE", path);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0 ||
      meta->pages_per_seq < 0)
    return fail(RPA_E_SHAPE, "head counts, head_dim, page_size must be positive");
  int row = -1;
  const int tp = path == RPA_TILE_DECODE_SPLIT ? rpa::kTileGqaDecode : rpa::kTileMlaShare;
  out->keys = resolve_tile_keys(tp, opts, (int)kv_dtype, head_dim, num_kv_heads, meta, page_size,
                                &row);
  out->max_splits = path == RPA_TILE_DECODE_SPLIT ? 16 : 0;
  out->table_row = row;
  return ok();
}

const char* rpa_last_error(void) { return g_last_error.c_str(); }

const char* rpa_last_path(void) { return g_last_path; }

size_t rpa_workspace_size(const rpa_ragged_meta* meta, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim) {
  if (!meta || num_kv_heads <= 0 || num_q_heads <= 0 || meta->max_num_seqs <= 0) return 0;
  return rpa::gqa_workspace_bytes(meta->max_num_seqs, meta->max_num_tokens, num_q_heads,
                                  num_kv_heads, head_dim, 0, nullptr);
}

}  // extern "C"

namespace {

// rpa_forward with its scratch either from the caller (workspace) or, for
// rpa_forward_noalloc, from the library's static per-device scratch array
// (noalloc: no stream is created, every launch stays on `stream`).
rpa_status gqa_forward(const void* q, rpa_dtype q_dtype, int32_t num_q_heads, int32_t head_dim,
                       void* kv_pages, rpa_dtype kv_dtype, int32_t total_num_pages,
                       int32_t page_size, int32_t num_kv_heads, const void* new_kv,
                       const rpa_ragged_meta* meta,
                       const rpa_opts* opts, void* out, void* workspace, size_t workspace_bytes,
                       bool noalloc, rpa_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  RPA_TRY(check_meta(meta, true));
  RPA_TRY(check_opts(opts));
  if (!q || !kv_pages || !out) return fail(RPA_E_INVALID, "q, kv_pages and out must be non-NULL");
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(RPA_E_SHAPE, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(RPA_E_SHAPE, "num_q_heads=%d must be divisible by num_kv_heads=%d", num_q_heads,
                num_kv_heads);
  if (head_dim <= 0 || head_dim > 512)
    return fail(RPA_E_SHAPE, "head_dim=%d must be in [1, 512]", head_dim);
  if (page_size <= 0 || total_num_pages <= 0)
    return fail(RPA_E_SHAPE, "page_size=%d and total_num_pages=%d must be positive", page_size,
                total_num_pages);
  if (q_dtype != RPA_F32 && q_dtype != RPA_BF16 && q_dtype != RPA_FP8_E4M3)
    return fail(RPA_E_DTYPE, "q dtype must be F32, BF16 or FP8_E4M3");
  if (dtype_bytes(kv_dtype) == 0 && kv_dtype != RPA_INT4)
    return fail(RPA_E_DTYPE, "kv dtype must be F32, BF16, FP8_E4M3, INT8 or INT4");
  if (kv_dtype == RPA_INT4 && (head_dim & 1))
    return fail(RPA_E_SHAPE, "an INT4 pool needs an even head_dim (got %d)", head_dim);

  rpa::GqaArgs a{};
  a.q = q;
  a.kv = kv_pages;
  a.new_kv = new_kv;
  a.kv_out = kv_pages;
  a.out = out;
  a.cu_q_lens = meta->cu_q_lens;
  a.kv_lens = meta->kv_lens;
  a.page_indices = meta->page_indices;
  a.num_seqs = meta->num_seqs;
  a.max_num_seqs = meta->max_num_seqs;
  a.pages_per_seq = meta->pages_per_seq;
  a.max_num_tokens = meta->max_num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.total_num_pages = total_num_pages;
  a.q_dtype = (int)q_dtype;
  a.kv_dtype = (int)kv_dtype;
  a.score_scale = opts->sm_scale * opts->k_scale * opts->q_scale;
  a.soft_cap = opts->soft_cap;
  a.v_scale = opts->v_scale;
  a.geo = rpa::gqa_geometry(num_q_heads, num_kv_heads, opts->sliding_window,
                            resolve_tile_keys(rpa::kTileGqaDecode, opts, a.kv_dtype, head_dim,
                                              num_kv_heads, meta, page_size, nullptr));

  const bool mfma = rpa::gqa_mfma_supported(a.q_dtype, a.kv_dtype, head_dim,
                                            num_q_heads / num_kv_heads) &&
                    is_pow2(page_size) && aligned16(q) && aligned16(kv_pages) && aligned16(out) &&
                    (new_kv == nullptr || aligned16(new_kv));
  if (q_dtype == RPA_FP8_E4M3 && !mfma)
    return fail(RPA_E_UNSUPPORTED,
                "fp8 queries run on the MFMA path only: head_dim 128, a BF16, FP8_E4M3 or INT8 "
                "pool, a power-of-two page size, 16-byte aligned q, kv_pages and out");
  if (mfma) {
    const size_t need = rpa_workspace_size(meta, num_q_heads, num_kv_heads, head_dim);
    if (noalloc) {
      if (need > rpa::noalloc_scratch_bytes())
        return fail(RPA_E_WORKSPACE,
                    "these capacities need %zu bytes of scratch; rpa_forward_noalloc holds at "
                    "most %zu (use rpa_forward with a workspace)",
                    need, rpa::noalloc_scratch_bytes());
      RPA_TRY(hip_status(rpa::noalloc_scratch(&workspace), "rpa_forward_noalloc scratch"));
      workspace_bytes = rpa::noalloc_scratch_bytes();
    }
    if (!workspace || workspace_bytes < need)
      return fail(RPA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(RPA_E_WORKSPACE, "workspace must be 16-byte aligned");
  }
  if (opts->debug_validate) {
    HostMeta h;
    RPA_TRY(fetch_meta(meta, true, stream, &h));
    RPA_TRY(validate_values(meta, h, page_size, total_num_pages));
    if (new_kv) RPA_TRY(check_update_slots(meta, h, page_size));
  }
  if (meta->max_num_tokens == 0) return ok();
  if (mfma) {
    rpa::gqa_bind_workspace(a, workspace);
    // The prefill kernel takes row maxima on raw scores, which needs an
    // increasing logit map: a positive score scale.
    a.single_stream = noalloc ? 1 : 0;
    // A bf16 batch whose token capacity leaves fewer than kPrefillMinTokens
    // tokens beyond one per sequence (a batch of decodes) keeps every tile on
    // the tile kernel: an empty prefill launch costs more than the rare short
    // chunk gains from it. One-byte pools keep the prefill kernel, whose
    // launch brings the one-byte decode kernel.
    constexpr int64_t kPrefillMinTokens = 256;
    const bool room_for_prefill =
        a.kv_dtype != (int)RPA_BF16 ||
        (int64_t)meta->max_num_tokens - meta->max_num_seqs >= kPrefillMinTokens;
    if (a.score_scale > 0.f && room_for_prefill &&
        rpa::gqa_prefill_supported(a.q_dtype, a.kv_dtype, head_dim, a.geo.group, page_size)) {
      // Prefill-class tiles of 256 rows for the eight-wave kernel (fewer tiles
      // than the workspace was sized for).
      a.pre_kernel = 1;
      a.geo.bq = rpa::gqa_prefill_rows() / a.geo.group;
    }
    TraceRange range("RPA-gqa-bq%d-kvs%d-p%d-g%d%s", a.geo.bq, a.geo.split_keys, page_size,
                     a.geo.group, a.pre_kernel ? "-prefill" : "");
    const rpa_status st = hip_status(rpa::launch_gqa(a, stream), "rpa_forward launch");
    if (st == RPA_OK) g_last_path = a.pre_kernel ? "gqa_mfma_prefill" : "gqa_mfma";
    return st;
  }
  TraceRange range("RPA-gqa-generic-d%d-p%d-g%d", head_dim, page_size, a.geo.group);
  const rpa_status st = hip_status(rpa::launch_gqa_generic(a, stream), "rpa_forward launch");
  if (st == RPA_OK) g_last_path = "gqa_generic";
  return st;
}

}  // namespace

extern "C" {

rpa_status rpa_forward(const void* q, rpa_dtype q_dtype, int32_t num_q_heads, int32_t head_dim,
                       void* kv_pages, rpa_dtype kv_dtype, int32_t total_num_pages,
                       int32_t page_size, int32_t num_kv_heads, const void* new_kv,
                       const rpa_ragged_meta* meta, const rpa_opts* opts, void* out,
                       void* workspace, size_t workspace_bytes, rpa_stream_t stream) {
  return gqa_forward(q, q_dtype, num_q_heads, head_dim, kv_pages, kv_dtype, total_num_pages,
                     page_size, num_kv_heads, new_kv, meta, opts, out, workspace, workspace_bytes,
                     false, stream);
}

rpa_status rpa_forward_noalloc(const void* q, rpa_dtype q_dtype, int32_t num_q_heads,
                               int32_t head_dim, void* kv_pages, rpa_dtype kv_dtype,
                               int32_t total_num_pages, int32_t page_size, int32_t num_kv_heads,
                               const void* new_kv, const rpa_ragged_meta* meta,
                               const rpa_opts* opts, void* out, rpa_stream_t stream) {
  return gqa_forward(q, q_dtype, num_q_heads, head_dim, kv_pages, kv_dtype, total_num_pages,
                     page_size, num_kv_heads, new_kv, meta, opts, out, nullptr, 0, true, stream);
}

size_t rpa_noalloc_scratch_bytes(void) { return rpa::noalloc_scratch_bytes(); }

rpa_status kv_cache_update(rpa_cache_layout layout, const void* new_a, const void* new_b,
                           void* cache_a, void* cache_b, rpa_dtype dtype, int32_t total_num_pages,
                           int32_t page_size, int32_t heads, int32_t dim_a, int32_t dim_b,
                           int32_t stride_a, int32_t stride_b, int32_t num_tokens,
                           const rpa_ragged_meta* meta, const int32_t* slot_loc,
                           int32_t debug_validate, rpa_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const int eb = dtype_bytes(dtype);
  if (eb == 0) return fail(RPA_E_DTYPE, "unknown dtype %d", (int)dtype);
  if (layout != RPA_LAYOUT_COMBINED_GQA && layout != RPA_LAYOUT_MLA_SPLIT &&
      layout != RPA_LAYOUT_MLA_FUSED)
    return fail(RPA_E_INVALID, "unknown layout %d", (int)layout);
  if (!new_a || !new_b || !cache_a) return fail(RPA_E_INVALID, "new_a, new_b and cache_a must be non-NULL");
  if (layout == RPA_LAYOUT_MLA_SPLIT && !cache_b)
    return fail(RPA_E_INVALID, "MLA split layout needs cache_b");
  if (total_num_pages <= 0 || page_size <= 0)
    return fail(RPA_E_SHAPE, "page_size=%d and total_num_pages=%d must be positive", page_size,
                total_num_pages);
  if (num_tokens < 0) return fail(RPA_E_SHAPE, "num_tokens=%d must be >= 0", num_tokens);
  if (dim_a <= 0) return fail(RPA_E_SHAPE, "dim_a=%d must be positive", dim_a);
  if (layout == RPA_LAYOUT_COMBINED_GQA) {
    if (heads <= 0) return fail(RPA_E_SHAPE, "heads=%d must be positive", heads);
  } else {
    if (dim_b <= 0) return fail(RPA_E_SHAPE, "dim_b=%d must be positive", dim_b);
    if (layout == RPA_LAYOUT_MLA_SPLIT && (stride_a < dim_a || stride_b < dim_b))
      return fail(RPA_E_SHAPE, "cache strides (%d, %d) must cover the new rows (%d, %d)", stride_a,
                  stride_b, dim_a, dim_b);
    if (layout == RPA_LAYOUT_MLA_FUSED && stride_a < dim_a + dim_b)
      return fail(RPA_E_SHAPE, "fused cache stride %d must cover %d + %d", stride_a, dim_a, dim_b);
  }
  if (!slot_loc) RPA_TRY(check_meta(meta, true));
  if (debug_validate) {
    std::set<int64_t> seen;
    if (slot_loc) {
      std::vector<int32_t> loc(num_tokens);
      hipError_t e = hipStreamSynchronize(stream);
      if (e == hipSuccess && num_tokens)
        e = hipMemcpy(loc.data(), slot_loc, (size_t)num_tokens * 4, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_status(e, "debug_validate copy");
      for (int t = 0; t < num_tokens; ++t) {
        if (loc[t] < 0) continue;
        if ((int64_t)loc[t] >= (int64_t)total_num_pages * page_size)
          return fail(RPA_E_INVALID, "token %d: slot %d out of range", t, loc[t]);
        if (!seen.insert(loc[t]).second)
          return fail(RPA_E_INVALID, "token %d: slot %d written twice", t, loc[t]);
      }
    } else {
      HostMeta h;
      RPA_TRY(fetch_meta(meta, true, stream, &h));
      RPA_TRY(validate_values(meta, h, page_size, total_num_pages));
      if (h.cu[h.ns] > num_tokens)
        return fail(RPA_E_INVALID, "total new tokens %d exceed num_tokens=%d", h.cu[h.ns], num_tokens);
      RPA_TRY(check_update_slots(meta, h, page_size));
    }
  }
  rpa::KvUpdateArgs a{};
  a.layout = (int)layout;
  a.new_a = new_a;
  a.new_b = new_b;
  a.cache_a = cache_a;
  a.cache_b = cache_b;
  a.elem_bytes = eb;
  a.total_num_pages = total_num_pages;
  a.page_size = page_size;
  a.heads = heads;
  a.dim_a = dim_a;
  a.dim_b = dim_b;
  a.stride_a = stride_a;
  a.stride_b = stride_b;
  a.slot_loc = slot_loc;
  if (meta) {
    a.cu_q_lens = meta->cu_q_lens;
    a.kv_lens = meta->kv_lens;
    a.page_indices = meta->page_indices;
    a.num_seqs = meta->num_seqs;
    a.max_num_seqs = meta->max_num_seqs;
    a.pages_per_seq = meta->pages_per_seq;
  }
  TraceRange range("RPA-kv_update-layout%d-t%d", (int)layout, num_tokens);
  return hip_status(rpa::launch_kv_update(a, num_tokens, stream), "kv_cache_update launch");
}

size_t mla_rpa_workspace_size(const rpa_ragged_meta* meta, int32_t num_heads, int32_t lkv_dim) {
  if (!meta || meta->max_num_seqs <= 0 || num_heads <= 0 || lkv_dim <= 0) return 0;
  return rpa::mla_workspace_bytes(meta->max_num_seqs, meta->max_num_tokens, num_heads, lkv_dim);
}

rpa_status mla_rpa_forward(const void* ql_nope, const void* q_pe, const void* new_kv_c,
                           const void* new_k_pe, void* cache_kv_c, void* cache_k_pe,
                           rpa_dtype dtype, int32_t num_heads, int32_t lkv_dim, int32_t r_dim,
                           int32_t kvc_stride, int32_t kpe_stride, int32_t total_num_pages,
                           int32_t page_size, const rpa_ragged_meta* meta, const rpa_opts* opts,
                           void* out, void* workspace, size_t workspace_bytes,
                           rpa_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  RPA_TRY(check_meta(meta, true));
  RPA_TRY(check_opts(opts));
  if (!ql_nope || !q_pe || !cache_kv_c || !cache_k_pe || !out)
    return fail(RPA_E_INVALID, "ql_nope, q_pe, caches and out must be non-NULL");
  if ((new_kv_c == nullptr) != (new_k_pe == nullptr))
    return fail(RPA_E_INVALID, "new_kv_c and new_k_pe must be both set or both NULL");
  if (dtype != RPA_BF16) return fail(RPA_E_UNSUPPORTED, "mla_rpa_forward implements BF16 only");
  if (num_heads <= 0) return fail(RPA_E_SHAPE, "num_heads=%d must be positive", num_heads);
  if (lkv_dim != 512 || r_dim != 64)
    return fail(RPA_E_UNSUPPORTED, "mla_rpa_forward implements lkv_dim=512, r_dim=64 (got %d, %d)",
                lkv_dim, r_dim);
  if (kvc_stride < lkv_dim || kpe_stride < r_dim)
    return fail(RPA_E_SHAPE, "cache strides (%d, %d) must cover (%d, %d)", kvc_stride, kpe_stride,
                lkv_dim, r_dim);
  // The page pads both latent parts to multiples of 128 columns.
  if (kvc_stride % 128 != 0 || kpe_stride % 128 != 0)
    return fail(RPA_E_SHAPE, "cache strides (%d, %d) must be multiples of 128", kvc_stride, kpe_stride);
  if (page_size <= 0 || total_num_pages <= 0 || !is_pow2(page_size))
    return fail(RPA_E_SHAPE, "page_size=%d must be a positive power of two; total_num_pages=%d > 0",
                page_size, total_num_pages);
  if (!aligned16(ql_nope) || !aligned16(q_pe) || !aligned16(cache_kv_c) || !aligned16(cache_k_pe) ||
      !aligned16(out))
    return fail(RPA_E_INVALID, "MLA tensors must be 16-byte aligned");
  const size_t need = mla_rpa_workspace_size(meta, num_heads, lkv_dim);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(RPA_E_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (opts->debug_validate) {
    HostMeta h;
    RPA_TRY(fetch_meta(meta, true, stream, &h));
    RPA_TRY(validate_values(meta, h, page_size, total_num_pages));
    if (new_kv_c) RPA_TRY(check_update_slots(meta, h, page_size));
  }
  if (meta->max_num_tokens == 0) return ok();
  // The step's new rows go to their cache slots inside the attention launch
  // (no separate scatter launch).
  rpa::MlaArgs a{};
  a.ql_nope = ql_nope;
  a.q_pe = q_pe;
  a.new_kv_c = new_kv_c;
  a.new_k_pe = new_k_pe;
  a.cache_kv_c = cache_kv_c;
  a.cache_k_pe = cache_k_pe;
  a.out = out;
  a.cu_q_lens = meta->cu_q_lens;
  a.kv_lens = meta->kv_lens;
  a.page_indices = meta->page_indices;
  a.num_seqs = meta->num_seqs;
  a.max_num_seqs = meta->max_num_seqs;
  a.pages_per_seq = meta->pages_per_seq;
  a.max_num_tokens = meta->max_num_tokens;
  a.num_heads = num_heads;
  a.lkv_dim = lkv_dim;
  a.r_dim = r_dim;
  a.kvc_stride = kvc_stride;
  a.kpe_stride = kpe_stride;
  a.page_size = page_size;
  a.total_num_pages = total_num_pages;
  // The MLA page's kernel scales the scores by k_scale and q_scale and the
  // value sum by v_scale.
  a.score_scale = opts->sm_scale * opts->k_scale * opts->q_scale;
  a.v_scale = opts->v_scale;
  a.soft_cap = opts->soft_cap;
  a.window = opts->sliding_window;
  a.min_share = resolve_tile_keys(rpa::kTileMlaShare, opts, (int)dtype, lkv_dim + r_dim, 1, meta,
                                  page_size, nullptr);
  rpa::mla_bind_workspace(a, workspace);
  TraceRange range("RPA-mla-h%d-share%d-p%d", num_heads, a.min_share, page_size);
  return hip_status(rpa::launch_mla(a, stream), "mla_rpa_forward launch");
}

}  // extern "C"

namespace {

// Checks shared by both sparse entry points; fills everything but the
// single-sequence / ragged fields.
rpa_status sparse_prepare(rpa::SparseArgs& a, const void* q, const void* kv_cache,
                          const int32_t* page_table, const int32_t* indices,
                          const int32_t* positions, int32_t num_queries, int32_t num_heads,
                          int32_t top_k, int32_t read_block, int32_t page_size,
                          int32_t total_num_pages, int32_t cache_dim, int32_t ptw,
                          int32_t kv_lora_rank, int32_t rope_dim, float sm_scale, float* out) {
  if (!q || !kv_cache || !page_table || !indices || !positions || !out)
    return fail(RPA_E_INVALID, "q, kv_cache, page table, indices, positions and out must be non-NULL");
  // sm_scale has no safe default [Sparse page: sparse_mla_attention].
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(RPA_E_INVALID, "sm_scale is required and must be finite and > 0");
  if (num_queries < 0 || num_heads <= 0 || top_k <= 0)
    return fail(RPA_E_SHAPE, "num_queries=%d >= 0, num_heads=%d > 0, top_k=%d > 0 required",
                num_queries, num_heads, top_k);
  if (read_block <= 0 || read_block % 16 != 0)
    return fail(RPA_E_INVALID, "read_block=%d must be a positive multiple of 16", read_block);
  if (top_k > 256)
    return fail(RPA_E_UNSUPPORTED, "top_k=%d selected units per query; this build handles up to 256",
                top_k);
  if (page_size <= 0 || page_size % read_block != 0)
    return fail(RPA_E_INVALID, "page_size=%d must be a multiple of read_block=%d", page_size, read_block);
  if (kv_lora_rank != 512 || rope_dim != 64)
    return fail(RPA_E_UNSUPPORTED, "sparse MLA implements kv_lora_rank=512, rope_dim=64");
  const int dk = kv_lora_rank + rope_dim;
  if (cache_dim < dk || cache_dim % 8 != 0)
    return fail(RPA_E_SHAPE, "cache_dim=%d must be >= %d and a multiple of 8", cache_dim, dk);
  if (total_num_pages <= 0 || ptw <= 0)
    return fail(RPA_E_SHAPE, "total_num_pages=%d and ptw=%d must be positive", total_num_pages, ptw);
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out))
    return fail(RPA_E_INVALID, "q, kv_cache and out must be 16-byte aligned");
  a = rpa::SparseArgs{};
  a.q = q;
  a.kv = kv_cache;
  a.page_table = page_table;
  a.indices = indices;
  a.positions = positions;
  a.out = out;
  a.num_queries = num_queries;
  a.num_heads = num_heads;
  a.top_k = top_k;
  a.read_block = read_block;
  a.page_size = page_size;
  a.total_num_pages = total_num_pages;
  a.cache_dim = cache_dim;
  a.ptw = ptw;
  a.dv = kv_lora_rank;
  a.dk = dk;
  a.score_scale = sm_scale;
  return RPA_OK;
}

}  // namespace

extern "C" {

rpa_status sparse_mla_forward(const void* q, const void* kv_cache, const int32_t* page_table,
                              const int32_t* indices, const int32_t* positions, int32_t seq_len,
                              int32_t num_queries, int32_t num_heads, int32_t top_k,
                              int32_t read_block, int32_t page_size, int32_t total_num_pages,
                              int32_t cache_dim, int32_t ptw, int32_t kv_lora_rank,
                              int32_t rope_dim, float sm_scale, float* out, rpa_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  rpa::SparseArgs a;
  const rpa_status st = sparse_prepare(a, q, kv_cache, page_table, indices, positions, num_queries,
                                       num_heads, top_k, read_block, page_size, total_num_pages,
                                       cache_dim, ptw, kv_lora_rank, rope_dim, sm_scale, out);
  if (st != RPA_OK) return st;
  if (seq_len < 0) return fail(RPA_E_INVALID, "seq_len=%d must be >= 0", seq_len);
  if (num_queries == 0) return ok();
  a.seq_len = seq_len;
  TraceRange range("RPA-sparse-k%d-rb%d-p%d", top_k, read_block, page_size);
  return hip_status(rpa::launch_sparse_mla(a, stream), "sparse_mla_forward launch");
}

rpa_status sparse_mla_forward_ragged(const void* q, const void* kv_cache,
                                     const int32_t* page_indices, int32_t ptw,
                                     const int32_t* indices, const int32_t* positions,
                                     const int32_t* cu_q_lens, const int32_t* seq_lens,
                                     const int32_t* cu_kv_lens, int32_t num_seqs,
                                     int32_t num_tokens, int32_t num_heads, int32_t top_k,
                                     int32_t read_block, int32_t page_size,
                                     int32_t total_num_pages, int32_t cache_dim,
                                     int32_t kv_lora_rank, int32_t rope_dim, float sm_scale,
                                     float* out, rpa_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  rpa::SparseArgs a;
  const rpa_status st = sparse_prepare(a, q, kv_cache, page_indices, indices, positions, num_tokens,
                                       num_heads, top_k, read_block, page_size, total_num_pages,
                                       cache_dim, ptw, kv_lora_rank, rope_dim, sm_scale, out);
  if (st != RPA_OK) return st;
  if (!cu_q_lens || !seq_lens || !cu_kv_lens)
    return fail(RPA_E_INVALID, "cu_q_lens, seq_lens and cu_kv_lens must be non-NULL");
  if (num_seqs <= 0) return fail(RPA_E_SHAPE, "num_seqs=%d must be positive", num_seqs);
  if (num_tokens == 0) return ok();
  a.cu_q_lens = cu_q_lens;
  a.seq_lens = seq_lens;
  a.cu_kv_lens = cu_kv_lens;
  a.num_seqs = num_seqs;
  TraceRange range("RPA-sparse-ragged-k%d-rb%d-p%d-s%d", top_k, read_block, page_size, num_seqs);
  return hip_status(rpa::launch_sparse_mla(a, stream), "sparse_mla_forward_ragged launch");
}

}  // extern "C"
