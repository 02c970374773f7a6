// pa_prefill.h - host-side declarations of the multi-token (chunked-prefill)
// paged attention kernel (pa_prefill.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// Queries of all sequences are packed along one token axis: sequence s owns
// tokens query_start_loc[s] .. query_start_loc[s+1]-1, a chunk of
// L_s = query_start_loc[s+1] - query_start_loc[s] tokens that ends its
// context_lens[s] cached tokens (position context_lens[s] - L_s + t for token
// t). Each query attends to its sequence's cached positions up to its own.
struct PrefillParams {
  void *out;                       // [num_tokens, Hq, D]
  const void *q;                   // [num_tokens, Hq, D]
  const void *k_cache;             // [num_blocks, Hkv, B, D]
  const void *v_cache;
  const int32_t *block_tables;     // [S, max_blocks_per_seq]
  const int32_t *context_lens;     // [S]
  const int32_t *query_start_loc;  // [S + 1]
  float scale_log2;                // scale * log2(e)
  int num_seqs;
  int num_tokens;                  // rows of q and out
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int block_shift;                 // log2(block_size)
  int max_blocks_per_seq;
  int num_blocks;                  // pool size: table entries are clamped into [0, num_blocks)
  int q_tiles;                     // query-row tiles per (sequence, KV head)
};

// dtype: PA_F16 or PA_BF16; head_dim 64 or 128; group Hq / Hkv in {1, 2, 4, 8}.
hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, int max_query_len,
                          hipStream_t stream);

// Query rows (token, head-of-group pairs) one workgroup covers.
constexpr int kPrefillRows = 128;

}  // namespace pa
