// pa_internal.h - kernel parameter blocks and launchers (internal to libpagedattn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Largest partition (tokens) a decode workgroup handles; bounds its LDS copy
// of the block-table entries.
constexpr int kMaxPartition = 2048;
constexpr int kDefaultPartition = 256;

struct DecodeParams {
  void *out;
  float *ws_acc;  // [S, Hq, max_partitions, D] float32 partial numerators
  float *ws_m;    // [S, Hq, max_partitions] running max (log2 domain)
  float *ws_l;    // [S, Hq, max_partitions] partial denominators
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float scale_log2;  // scale * log2(e)
  int num_seqs;
  int num_kv_heads;
  int group;  // query heads per KV head
  int head_dim;
  int block_shift;  // log2(block_size)
  int num_blocks;
  int max_blocks_per_seq;
  int max_context_len;
  int partition_size;
  int max_partitions;
  int dtype;
};

struct CacheParams {
  const void *key;
  const void *value;
  void *k_cache;
  void *v_cache;
  const int32_t *slot_mapping;
  int num_tokens;
  int num_kv_heads;
  int row_chunks;  // head_dim * element bytes / 16
  int block_shift;
  int64_t num_slots;  // num_blocks * block_size
};

enum DecodeStage { kStageBoth = 0, kStagePartitions = 1, kStageReduce = 2 };

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream, DecodeStage stage);
hipError_t launch_reshape_and_cache(const CacheParams &p, hipStream_t stream);

}  // namespace pa
