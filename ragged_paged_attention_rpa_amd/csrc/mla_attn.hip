// MLA latent attention [MLA v1 page]. (Kernel lands in the next change.)
#include "rpa_device.h"
#include "rpa_internal.h"

namespace rpa {
size_t mla_workspace_bytes(int max_num_seqs, int max_num_tokens, int num_heads, int lkv_dim,
                           int* tile_capacity, int* max_splits) {
  if (tile_capacity) *tile_capacity = max_num_tokens + max_num_seqs;
  if (max_splits) *max_splits = 1;
  return 256;
}
void mla_bind_workspace(MlaArgs& a, void* ws) { a.counters = (int32_t*)ws; }
hipError_t launch_mla(const MlaArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sparse_mla(const SparseArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace rpa
