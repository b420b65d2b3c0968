// Internal interface between the host API (rpa_api.cpp) and the kernel
// launchers (*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rpa {

// Records the caller's profiling events (rpa_set_profile_events) around the
// main kernel of an entry point; no-ops when the hook is off.
void prof_begin(hipStream_t stream);
void prof_end(hipStream_t stream);
// Per-kernel events of rpa_forward (rpa_set_profile_events_split): kernel 0 is
// the prefill-tile kernel, kernel 1 the decode-tile kernel.
void prof_kernel_begin(hipStream_t stream, int k);
void prof_kernel_end(hipStream_t stream, int k);

// ---------------------------------------------------------------- update ----
struct KvUpdateArgs {
  int layout;  // 0 combined GQA, 1 MLA split, 2 MLA fused
  const void* new_a;
  const void* new_b;
  void* cache_a;
  void* cache_b;
  int elem_bytes;
  int total_num_pages, page_size, heads, dim_a, dim_b, stride_a, stride_b;
  const int32_t* cu_q_lens;
  const int32_t* kv_lens;
  const int32_t* page_indices;
  const int32_t* num_seqs;
  int max_num_seqs, pages_per_seq;
  const int32_t* slot_loc;
};
hipError_t launch_kv_update(const KvUpdateArgs& a, int num_tokens, hipStream_t stream);

// ------------------------------------------------------------------- GQA ----
// Work-list tile: one (sequence, kv head, query block, kv split) unit.
struct Tile {
  int32_t seq;
  int32_t qtok0;  // first query token of the block, relative to the sequence
  int32_t kvh;
  int32_t split;  // >= 0: split index of a decode-class tile; -1: whole key range
};

// Geometry shared by the planner, the attention kernel and the merge kernel.
struct GqaGeometry {
  int group;        // Hq / Hkv
  int qdec;         // sequences with q_len <= qdec are decode-class (q_len*group <= 16)
  int bq;           // query tokens per prefill-class tile (bq*group <= 64 on the four-wave
                    // kernel, <= 256 on the prefill kernel)
  int split_keys;   // target keys per decode split
  int max_splits;   // cap on splits per decode sequence
  int window;       // sliding window (0 = none)
};

struct GqaArgs {
  const void* q;
  const void* kv;
  // Step's new K/V rows [max_num_tokens, 2*num_kv_heads, head_dim] in the pool
  // dtype (K of kv head h at 2h, V at 2h+1), or NULL. Keys at positions
  // >= kv_len - q_len are read from here, and the merge launch copies these
  // rows to their pool slots.
  const void* new_kv;
  void* kv_out;  // the pool as a writable pointer (the slots of new_kv's rows)
  void* out;
  const int32_t* cu_q_lens;
  const int32_t* kv_lens;
  const int32_t* page_indices;
  const int32_t* num_seqs;
  int max_num_seqs, pages_per_seq, max_num_tokens;
  int num_q_heads, num_kv_heads, head_dim, page_size, total_num_pages;
  int q_dtype, kv_dtype;
  float score_scale;  // sm_scale * k_scale
  float soft_cap;     // 0 = none
  float v_scale;
  GqaGeometry geo;
  int pre_kernel;     // 1: prefill-class tiles go to gqa_prefill_kernel (geo.bq = its rows / group)
  int single_stream;  // 1: every launch on the caller's stream (no library side stream)
  // workspace
  Tile* tiles;
  int32_t* counters;  // [0] tile count, [1] decode-kernel cursor (starts past the prefill
                      // tiles when pre_kernel), [3] prefill tiles, [16 .. 23] prefill
                      // cursors (one per XCD)
  uint16_t* part_acc; // [max_num_seqs*Hkv*max_splits][16][D] acc / l of the split (fp16
                      // for fp8 pools, bf16 for bf16 pools)
  float* part_ml;     // [max_num_seqs*Hkv*max_splits][16][2]
  int tile_capacity;
};

constexpr int kXcdCursor0 = 16;  // first per-XCD prefill cursor in GqaArgs::counters
constexpr int kXcds = 8;         // XCDs of an MI355X (one prefill cursor each)

// Tile-size table (tile_table.cpp): keys per decode split (kTileGqaDecode)
// or smallest MLA share (kTileMlaShare) for a shape; *row receives the
// matching row (-1: built-in default).
enum TilePath { kTileGqaDecode = 0, kTileMlaShare = 1 };
int tile_keys(int path, int kv_dtype, int head_dim, int num_kv_heads, int64_t context, int* row);
GqaGeometry gqa_geometry(int num_q_heads, int num_kv_heads, int window, int split_keys);
size_t gqa_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_q_heads,
                           int num_kv_heads, int head_dim, int window, int* tile_capacity);
// Carves the workspace into tiles/counters/partials of GqaArgs.
void gqa_bind_workspace(GqaArgs& a, void* ws);
bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim, int group);
hipError_t launch_gqa(const GqaArgs& a, hipStream_t stream);
hipError_t launch_gqa_generic(const GqaArgs& a, hipStream_t stream);
// The static per-device scratch array of rpa_forward_noalloc: its size, and
// its device address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);
// Prefill-class tiles on eight waves (gqa_prefill.hip). Requires
// a.score_scale > 0 (the kernel takes row maxima on raw scores).
int gqa_prefill_rows();
bool gqa_prefill_supported(int q_dtype, int kv_dtype, int head_dim, int group, int page_size);
hipError_t launch_gqa_prefill(const GqaArgs& a, int ps_log2, int grid, hipStream_t stream);

// ------------------------------------------------------------------- MLA ----
constexpr int kMlaGrid = 256;  // workgroups of the MLA tile kernel (one share of keys each)

struct MlaArgs {
  const void* ql_nope;
  const void* q_pe;
  const void* new_kv_c;  // [max_num_tokens, lkv_dim] or NULL: the step's new rows, scattered
  const void* new_k_pe;  // [max_num_tokens, r_dim]    into the caches inside the attention launch
  void* cache_kv_c;
  void* cache_k_pe;
  void* out;
  const int32_t* cu_q_lens;
  const int32_t* kv_lens;
  const int32_t* page_indices;
  const int32_t* num_seqs;
  int max_num_seqs, pages_per_seq, max_num_tokens;
  int num_heads, lkv_dim, r_dim, kvc_stride, kpe_stride, page_size, total_num_pages;
  float score_scale;
  float soft_cap;
  int window;
  int min_share;      // smallest share of the key space per workgroup (multiple of 32)
  float v_scale;      // multiplies the normalised output (the page's scale on the value sum)
  // workspace
  int32_t* counters;  // [0] pieces, [1] partial slots used
  int32_t* wg_start;  // [kMlaGrid + 1] first piece of each workgroup's share
  long long* kpre;    // [max_num_tokens] inclusive prefix of visible keys per token
  int32_t* tok_slot;  // [head groups * max_num_tokens][2]: first partial slot (-1: whole), pieces
  int32_t* pieces;    // [piece_capacity][8]: {seq, token, lo, hi}, {head group, slot, writes, share}
  uint16_t* part_acc; // [slot_capacity][num_heads][lkv_dim] bf16: acc / l of the piece
  float* part_ml;     // [slot_capacity][num_heads][2]
  int piece_capacity, slot_capacity;
};
size_t mla_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_heads, int lkv_dim);
void mla_bind_workspace(MlaArgs& a, void* ws);
hipError_t launch_mla(const MlaArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- sparse ----
struct SparseArgs {
  const void* q;
  const void* kv;
  const int32_t* page_table;  // single sequence: [ptw]; ragged: the packed table [ptw]
  const int32_t* indices;
  const int32_t* positions;
  // Packed-ragged mode when cu_q_lens != nullptr: per-token request, bound
  // seq_lens[rid] and table base cu_kv_lens[rid] / page_size.
  const int32_t* cu_q_lens;
  const int32_t* seq_lens;
  const int32_t* cu_kv_lens;
  float* out;
  int seq_len, num_seqs, num_queries, num_heads, top_k, read_block, page_size, total_num_pages,
      cache_dim, ptw, dv, dk;
  float score_scale;
};
hipError_t launch_sparse_mla(const SparseArgs& a, hipStream_t stream);

}  // namespace rpa
