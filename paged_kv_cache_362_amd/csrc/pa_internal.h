// pa_internal.h - kernel parameter blocks and launchers (internal to libpagedattn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

// Largest partition (tokens) a decode workgroup of the fixed-partition form
// handles, and the default size of that form.
constexpr int kMaxPartition = 4096;
constexpr int kDefaultPartition = 256;

// Balanced (single-launch) form: at most this many sequences (its plan of
// per-sequence tile counts lives in LDS) and this many workgroups.
constexpr int kMaxPlanSeqs = 4096;
constexpr int kMaxFlatWorkgroups = 2048;
// Resident balanced-form workgroups per compute unit, at most. Measured on
// MI355X (fused decode step, two interleaved runs, 3 -> 2 per CU): LLaMA-7B
// layer 99.9 -> 98.7 us, GQA bf16 87.4 -> 86.2 us, LLaMA-13B layer with a
// shared prefix 107.4 -> 102.6 us, the 67 MB long context unchanged. Eight
// waves per CU still keep ~128 KB of loads in flight, the longer ranges cut
// split pieces, and fewer co-resident workgroups narrow the spread of the
// compute units' finishing times. One per CU is slower except on the shared
// prefix (101.5 us). 4 per CU was slower than 3.
constexpr int kMaxFlatWgsPerCu = 2;

struct DecodeParams {
  void *out;
  float *ws_acc;      // partial numerators (layout depends on the form)
  float *ws_m;        // partial maxima (log2 domain)
  float *ws_l;        // partial denominators
  int32_t *ws_count;  // balanced form: arrivals per (sequence, KV head); zero between calls
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
  // Balanced form: tiles of work charged for each (sequence, KV head) a
  // workgroup's range touches, on top of its tiles (see decode_flat_kernel).
  int seg_cost;
  int dtype;
  // Fused cache write (decode step form; null otherwise): token s of
  // new_key/new_value [S, Hkv, D] goes to slot_mapping[s] of the pools, and is
  // the last position (context_lens[s] - 1) of sequence s.
  const void *new_key;
  const void *new_value;
  const int32_t *slot_mapping;
  void *k_cache_w;
  void *v_cache_w;
  int64_t num_slots;
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

// kStageFlat: balanced single launch. kStageBoth: fixed partitions, then the
// reduce. kStagePartitions / kStageReduce: one of those two launches.
enum DecodeStage { kStageBoth = 0, kStagePartitions = 1, kStageReduce = 2, kStageFlat = 3 };

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream, DecodeStage stage);
hipError_t launch_reshape_and_cache(const CacheParams &p, hipStream_t stream);

// Dynamic LDS of the balanced form's plan: tile prefix sums [S + 1], clamped
// lengths [S] and this step's slots [S].
inline size_t flat_plan_lds_bytes(int num_seqs) { return size_t(3 * num_seqs + 1) * sizeof(int); }

// Workgroups of a balanced launch on the current device: as many as can be
// resident at once (capped at kMaxFlatWorkgroups), but no more than give each
// kMinFlatTiles of `max_tiles` (an upper bound of the call's 16-token tiles,
// from max_context_len), and at least one per compute unit or one per
// kMinFlatTilesFloor tiles, whichever is fewer. Defined in pa_api.cpp.
constexpr int kMinFlatTiles = 64;
// The "one per compute unit" floor above is itself capped at one workgroup per
// kMinFlatTilesFloor tiles of `max_tiles`: a tiny call (the 50-token, 4-head
// one: 16 tiles) then gets one workgroup per (sequence, KV head) instead of
// every head cut into one-tile pieces that pay the split-head combine.
constexpr int kMinFlatTilesFloor = 4;
// Overhead units charged per (sequence, KV head) by the balanced plan. Swept on
// MI355X over 0, 4, 8, 16, 32 tiles: 4 was best (GQA-4 bf16 decode 2% faster
// than 0; 16 and more lengthen every workload).
constexpr int kFlatSegmentCost = 4;
int flat_segment_cost();

// Static scratch of pa_decode_step_noalloc (pa_noalloc.hip): its bytes, this
// device's address of it (looked up once per device; nullptr on failure), and
// a kernel that zeroes its first n int32 words on `stream`.
constexpr size_t kNoallocScratchBytes = size_t(PA_NOALLOC_SCRATCH_BYTES);
void *noalloc_scratch();
hipError_t launch_clear_words(void *words, int n, hipStream_t stream);
int flat_grid_size(const void *kernel, int threads, size_t dynamic_lds, int64_t max_tiles);

}  // namespace pa
