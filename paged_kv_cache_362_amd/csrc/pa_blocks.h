// pa_blocks.h - host-side declarations of the whole-block copy kernel
// (copy-on-write and swapping; pa_blocks.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v): pair i of
// block_mapping [num_pairs, 2] copies block block_mapping[2i] of the source
// pools to block block_mapping[2i + 1] of the destination pools. All pointers
// are device addresses (pinned host memory already translated).
struct BlockCopyParams {
  const void *src_k;
  const void *src_v;
  void *dst_k;
  void *dst_v;
  const int32_t *block_mapping;
  int num_pairs;
  int src_blocks;       // blocks in the source pools
  int dst_blocks;       // blocks in the destination pools
  int64_t block_bytes;  // num_kv_heads * block_size * head_dim * element bytes
};

hipError_t launch_copy_blocks(const BlockCopyParams &p, hipStream_t stream);

}  // namespace pa
