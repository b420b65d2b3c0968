// Scatter of new tokens into paged caches [MLA v1 page: update_kv_cache;
// Sparse page: prefill_write_and_attend self-write].
//
// One workgroup per new token; its 64 lanes copy the token's rows in 16-byte
// pieces (bitwise copy, so bf16/fp8/fp32 are all the same to it). The slot of
// token j of sequence i is p = kv_len - q_len + j: page page_indices[i*pps +
// p/ps], row p % ps; in slot-list mode it is slot_loc[t] (negative = skip).
#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {

namespace {

// Copies `bytes` from src to dst with 16-byte pieces when both are 16-byte
// aligned and the size is a multiple of 16, else 2-byte/1-byte pieces.
__device__ __forceinline__ void lane_copy(char* dst, const char* src, int bytes, int lane) {
  if ((((uintptr_t)dst | (uintptr_t)src | (uintptr_t)bytes) & 15) == 0) {
    const int n = bytes >> 4;
    for (int i = lane; i < n; i += 64)
      reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
  } else if ((((uintptr_t)dst | (uintptr_t)src | (uintptr_t)bytes) & 1) == 0) {
    const int n = bytes >> 1;
    for (int i = lane; i < n; i += 64)
      reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[i];
  } else {
    for (int i = lane; i < bytes; i += 64) dst[i] = src[i];
  }
}

__device__ __forceinline__ void lane_zero(char* dst, int bytes, int lane) {
  if ((((uintptr_t)dst | (uintptr_t)bytes) & 15) == 0) {
    const int n = bytes >> 4;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = lane; i < n; i += 64) reinterpret_cast<u32x4*>(dst)[i] = z;
  } else {
    for (int i = lane; i < bytes; i += 64) dst[i] = 0;
  }
}

__global__ void __launch_bounds__(64) kv_update_kernel(KvUpdateArgs a) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  int64_t slot;
  if (a.slot_loc) {
    slot = a.slot_loc[t];
    if (slot < 0) return;
  } else {
    int ns = *a.num_seqs;
    ns = ns < 0 ? 0 : (ns > a.max_num_seqs ? a.max_num_seqs : ns);
    const int i = find_seq(a.cu_q_lens, ns, t);
    if (i < 0) return;
    const int q_len = a.cu_q_lens[i + 1] - a.cu_q_lens[i];
    const int pos = a.kv_lens[i] - q_len + (t - a.cu_q_lens[i]);
    if (pos < 0) return;
    const int lp = pos / a.page_size;
    if (lp >= a.pages_per_seq) return;
    const int page = a.page_indices[(int64_t)i * a.pages_per_seq + lp];
    if (page < 0 || page >= a.total_num_pages) return;
    slot = (int64_t)page * a.page_size + pos % a.page_size;
  }
  if (slot >= (int64_t)a.total_num_pages * a.page_size) return;
  const int eb = a.elem_bytes;
  if (a.layout == 0) {  // combined GQA
    const int row_bytes = a.dim_a * eb;
    char* base = (char*)a.cache_a + slot * (int64_t)(2 * a.heads) * row_bytes;
    for (int h = 0; h < a.heads; ++h) {
      lane_copy(base + (int64_t)(2 * h) * row_bytes,
                (const char*)a.new_a + ((int64_t)t * a.heads + h) * row_bytes, row_bytes, lane);
      lane_copy(base + (int64_t)(2 * h + 1) * row_bytes,
                (const char*)a.new_b + ((int64_t)t * a.heads + h) * row_bytes, row_bytes, lane);
    }
  } else if (a.layout == 1) {  // MLA split
    char* da = (char*)a.cache_a + slot * (int64_t)a.stride_a * eb;
    char* db = (char*)a.cache_b + slot * (int64_t)a.stride_b * eb;
    lane_copy(da, (const char*)a.new_a + (int64_t)t * a.dim_a * eb, a.dim_a * eb, lane);
    lane_zero(da + a.dim_a * eb, (a.stride_a - a.dim_a) * eb, lane);
    lane_copy(db, (const char*)a.new_b + (int64_t)t * a.dim_b * eb, a.dim_b * eb, lane);
    lane_zero(db + a.dim_b * eb, (a.stride_b - a.dim_b) * eb, lane);
  } else {  // MLA fused
    char* da = (char*)a.cache_a + slot * (int64_t)a.stride_a * eb;
    lane_copy(da, (const char*)a.new_a + (int64_t)t * a.dim_a * eb, a.dim_a * eb, lane);
    lane_copy(da + a.dim_a * eb, (const char*)a.new_b + (int64_t)t * a.dim_b * eb, a.dim_b * eb,
              lane);
    lane_zero(da + (a.dim_a + a.dim_b) * eb, (a.stride_a - a.dim_a - a.dim_b) * eb, lane);
  }
}

}  // namespace

hipError_t launch_kv_update(const KvUpdateArgs& a, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_update_kernel, dim3(num_tokens), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rpa
