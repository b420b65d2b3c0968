// Tile sizes chosen per shape from a table of measured rows [RPA v2 page:
// ragged_paged_attention asks get_tuned_block_sizes for its KV-pages and
// query blocks, keyed by dtypes, head counts, head dim, page size and context
// length; MLA v1 page: mla_ragged_paged_attention takes the block sizes from
// the caller]. Here the sizes that vary with the shape are
//   - the decode split of rpa_forward: target keys per split of a decode-class
//     sequence (chunks stay multiples of 64 and at most 16 per sequence);
//   - the smallest share of mla_rpa_forward's key space per workgroup.
// A caller may fix either through rpa_opts.split_keys, as the MLA page's
// caller fixes its block sizes; rpa_tile_config reports what a call will use.
#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

struct TileRow {
  int path;          // kTileGqaDecode or kTileMlaShare
  int kv_dtype;      // DT_* of the pool, or -1 for any
  int head_dim;      // or -1 for any
  int kv_heads_max;  // the row applies when num_kv_heads <= kv_heads_max
  int ctx_min;       // ... and the context capacity (pages_per_seq * page_size) >= ctx_min
  int keys;          // split target (decode) or smallest share (MLA), in keys
};

// First matching row wins, so rows go from specific to general and each path
// ends with a catch-all. The values are measurements on MI355X with
// `python -m ragged_paged_attention_rpa_amd.tune` (candidates interleaved call
// by call, medians of 30 calls; run-to-run noise about 3%):
//   decode 128 x 512..8192 keys, 32/8 heads: bf16 pool 1024 keys per split
//     (0.406 ms; 512: 0.427, 2048: 0.409, 256: 0.464); fp8 pool 2048 (0.230 ms;
//     1024: 0.236, 512: 0.272);
//   decode 8 x 16k..32k, fp8: 2048 (0.106 ms; others 0.108..0.111);
//   decode 256 x 128..2048, bf16: 1024 (0.222 ms; 256: 0.268);
//   decode 32 x 2k..16k at 8/1 heads and 16 x 16k..64k at 16/2 heads (fp8):
//     every split from 256 to 2048 within noise of the row's value, 4096 up to
//     80% slower at one kv head;
//   MLA shares: 128 keys on 8 x 1..4k (0.110 ms; 64: 0.118, 512: 0.117),
//     2 x 2048 (0.063 ms; 64: 0.075, 1024: 0.104) and 4 x 512 with 4 query
//     tokens each (0.077 ms; 64: 0.079, 256: 0.080); no effect on
//     64 x 4k..32k (0.426..0.430 ms for every candidate), where the equal
//     shares are larger than any candidate.
constexpr TileRow kRows[] = {
    {kTileGqaDecode, DT_FP8, 128, 1 << 30, 0, 2048},
    {kTileGqaDecode, DT_BF16, 128, 1 << 30, 0, 1024},
    {kTileGqaDecode, -1, -1, 1 << 30, 0, 1024},
    {kTileMlaShare, -1, -1, 1 << 30, 0, 128},
};

}  // namespace

int tile_keys(int path, int kv_dtype, int head_dim, int num_kv_heads, int64_t context,
              int* row) {
  const int n = (int)(sizeof(kRows) / sizeof(kRows[0]));
  for (int i = 0; i < n; ++i) {
    const TileRow& r = kRows[i];
    if (r.path != path) continue;
    if (r.kv_dtype >= 0 && r.kv_dtype != kv_dtype) continue;
    if (r.head_dim >= 0 && r.head_dim != head_dim) continue;
    if (num_kv_heads > r.kv_heads_max) continue;
    if (context < r.ctx_min) continue;
    if (row) *row = i;
    return r.keys;
  }
  if (row) *row = -1;
  return path == kTileMlaShare ? 128 : 1024;
}

}  // namespace rpa
