// pa_cache.hip - the cache write of one decode step (gfx950).
//
// Each new token's K and V rows ([num_kv_heads, head_dim] each) are copied,
// bit for bit, into the slot named for the token: block slot / block_size,
// offset slot % block_size, of the two pools ([INFRA] "【infra之路】10-
// PagedAttention 与 KV Cache 管理", §1.2 cache append and §3.3 next slot).
// One workgroup per token; each lane moves 16-byte chunks, so a head row is
// written with full, coalesced stores.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheParams p) {
  const int t = blockIdx.x;
  const int slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;  // negative: skip; too large: never write outside
  const int64_t blk = slot >> p.block_shift;
  const int64_t off = slot & ((1 << p.block_shift) - 1);
  const int per_head = p.row_chunks;
  const int total = p.num_kv_heads * per_head;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int h = i / per_head;
    const int ch = i - h * per_head;
    const int64_t src = ((int64_t)t * p.num_kv_heads + h) * per_head + ch;
    const int64_t dst = (((blk * p.num_kv_heads + h) << p.block_shift) + off) * per_head + ch;
    store_chunk(p.k_cache, dst * 16, load_chunk(p.key, src * 16));
    store_chunk(p.v_cache, dst * 16, load_chunk(p.value, src * 16));
  }
}

hipError_t launch_reshape_and_cache(const CacheParams &p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  const int total = p.num_kv_heads * p.row_chunks;
  const int threads = total >= 256 ? 256 : ((total + 63) / 64) * 64;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(p.num_tokens), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
