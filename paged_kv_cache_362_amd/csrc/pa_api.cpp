// pa_api.cpp - the C ABI of libpagedattn.so: argument checks, the choice of
// decode form, workspace layout and sizing, the launch grid of the balanced
// form, and the optional (PA_DEBUG) device-side checks. Declarations and the
// contract of every entry point are in include/pagedattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <unordered_set>
#include <vector>

#include "pa_blocks.h"
#include "pa_internal.h"
#include "pa_prefill.h"
#include "pagedattn.h"

namespace {

constexpr int32_t kAbiVersion = 4;
constexpr size_t kAlign = 256;

bool debug_checks() {
  const char *e = std::getenv("PA_DEBUG");
  return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
  }
  return 0;
}

int exact_log2(int32_t x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) != x) ++s;
  return s;
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }
bool block_size_ok(int32_t b) { return b == 8 || b == 16 || b == 32 || b == 64; }
bool group_ok(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shape checks shared by pa_decode and pa_decode_workspace_size.
int32_t check_decode_shapes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_context_len, int32_t dtype) {
  if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
      num_q_heads <= 0 || max_context_len < 0)
    return PA_ERR_BAD_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (elem_bytes(dtype) == 0 || !head_dim_ok(head_dim) || !group_ok(num_q_heads / num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (head_dim * elem_bytes(dtype) > 512) return PA_ERR_UNSUPPORTED;  // f32 rows of 256
  return PA_OK;
}

// 0 = balanced form; otherwise a fixed partition size (multiple of 16).
bool partition_ok(int32_t requested) {
  return requested == 0 ||
         (requested >= 16 && requested <= pa::kMaxPartition && requested % 16 == 0);
}

int32_t num_partitions(int32_t max_context_len, int32_t partition) {
  const int32_t np = (max_context_len + partition - 1) / partition;
  return np < 1 ? 1 : np;
}

// Upper bound of the balanced form's work units (tiles plus the overhead
// charged per (sequence, KV head)); the kernel keeps unit positions in int32.
bool flat_units_fit(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  const int64_t per_item = (int64_t(max_context_len) + 15) / 16 + pa::flat_segment_cost();
  return int64_t(num_seqs) * num_kv_heads * per_item < (int64_t(1) << 31) - 1;
}

// The form a call takes: the balanced single launch, or fixed partitions of
// `*partition` tokens (the default size when the balanced form cannot plan
// this many sequences, or this much work).
bool use_balanced(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                  int32_t requested, int32_t *partition) {
  if (requested == 0 && num_seqs <= pa::kMaxPlanSeqs &&
      flat_units_fit(num_seqs, num_kv_heads, max_context_len)) {
    *partition = 0;
    return true;
  }
  *partition = requested == 0 ? pa::kDefaultPartition : requested;
  return false;
}

// Workspace layout: [arrival counters, int32 per (sequence, KV head)] then the
// partials of the form in use. The counters are only touched by the balanced
// form, which leaves them zero.
struct WsLayout {
  size_t counters = 0;  // bytes
  size_t slots = 0;     // partial rows of `width` floats
  size_t width = 0;     // floats per partial row of acc
  size_t stats = 0;     // floats of m (and of l)
  size_t total = 0;
};

WsLayout workspace_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_context_len, int32_t requested) {
  WsLayout w;
  int32_t partition = 0;
  w.counters = round_up(size_t(num_seqs) * size_t(num_kv_heads) * sizeof(int32_t));
  if (use_balanced(num_seqs, num_kv_heads, max_context_len, requested, &partition)) {
    const size_t group = size_t(num_q_heads / num_kv_heads);
    // one slot per (item, workgroup) piece: at most items + workgroups of them
    w.slots = size_t(num_seqs) * num_kv_heads + pa::kMaxFlatWorkgroups;
    w.width = group * head_dim;
    w.stats = w.slots * group;
  } else {
    const int32_t parts = num_partitions(max_context_len, partition);
    if (parts > 1) {
      w.slots = size_t(num_seqs) * num_q_heads * parts;
      w.width = size_t(head_dim);
      w.stats = w.slots;
    }
  }
  w.total = w.counters + round_up((w.slots * w.width + 2 * w.stats) * sizeof(float));
  return w;
}

// The address a kernel uses for p: p itself for device (or managed) memory,
// the mapped device address for pinned host memory. Pageable host memory and
// unknown pointers are refused: a kernel touching them would fault.
int32_t device_address(const void *p, const void **dev) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next call
    return PA_ERR_BAD_POINTER;
  }
  if (a.type == hipMemoryTypeDevice || a.isManaged) {
    *dev = p;
    return PA_OK;
  }
  if (a.type == hipMemoryTypeHost) {
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void *>(p), 0) != hipSuccess || d == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_BAD_POINTER;
    }
    *dev = d;
    return PA_OK;
  }
  return PA_ERR_BAD_POINTER;
}

int32_t sync_copy_to_host(void *dst, const void *src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return PA_OK;
  if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

namespace pa {

int flat_grid_size(const void *kernel, int threads, size_t dynamic_lds, int64_t max_tiles) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void *, size_t>, std::pair<int, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const auto key = std::make_tuple(dev, kernel, dynamic_lds);
  int cus = 0, resident = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      cus = it->second.first;
      resident = it->second.second;
    } else {
      int per_cu = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dynamic_lds) !=
          hipSuccess)
        return -1;
      if (per_cu > kMaxFlatWgsPerCu) per_cu = kMaxFlatWgsPerCu;
      if (const char *e = std::getenv("PA_FLAT_WGS_PER_CU")) {  // tuning knob
        const int v = std::atoi(e);
        if (v > 0) per_cu = v;
      }
      resident = cus * (per_cu > 0 ? per_cu : 1);
      if (resident > kMaxFlatWorkgroups) resident = kMaxFlatWorkgroups;
      cache[key] = std::make_pair(cus, resident);
    }
  }
  // Small calls: fewer, longer ranges (each workgroup has a fixed start-up cost
  // and a split (sequence, KV head) costs a combine), but every compute unit
  // streams unless the call is tiny.
  int64_t want = (max_tiles + kMinFlatTiles - 1) / kMinFlatTiles;
  int64_t floor_wgs = (max_tiles + kMinFlatTilesFloor - 1) / kMinFlatTilesFloor;
  if (floor_wgs > cus) floor_wgs = cus;
  if (want < floor_wgs) want = floor_wgs;
  if (want < 1) want = 1;
  return want < resident ? int(want) : resident;
}

// Tiles of work a segment's start and epilogue cost in the balanced plan;
// PA_FLAT_SEG_COST overrides it (a tuning knob).
int flat_segment_cost() {
  static const int cost = [] {
    int c = kFlatSegmentCost;
    if (const char *e = std::getenv("PA_FLAT_SEG_COST")) c = std::atoi(e);
    return c < 0 ? 0 : c > 1024 ? 1024 : c;
  }();
  return cost;
}

}  // namespace pa

extern "C" {

int32_t pa_abi_version(void) { return kAbiVersion; }

const char *pa_status_str(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "null pointer argument";
    case PA_ERR_BAD_SHAPE: return "bad or inconsistent shape argument";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype, group or alignment";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_BAD_INDEX: return "device-side index precondition violated (PA_DEBUG)";
    case PA_ERR_BAD_POINTER: return "memory is neither GPU memory nor pinned host memory";
    case PA_ERR_SCRATCH_TOO_SMALL: return "the call needs more scratch than the static array holds";
  }
  return "unknown status";
}

int32_t pa_reshape_and_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int32_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, void *stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PA_ERR_BAD_SHAPE;
  if (elem_bytes(dtype) == 0 || !head_dim_ok(head_dim) || !block_size_ok(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t num_slots = int64_t(num_blocks) * block_size;

  if (debug_checks()) {
    std::vector<int32_t> slots(num_tokens);
    int32_t st = sync_copy_to_host(slots.data(), slot_mapping, sizeof(int32_t) * num_tokens, s);
    if (st != PA_OK) return st;
    std::unordered_set<int32_t> seen;
    for (int32_t v : slots) {
      if (v < 0) continue;
      if (v >= num_slots || !seen.insert(v).second) return PA_ERR_BAD_INDEX;
    }
  }

  pa::CacheParams p{};
  p.key = key;
  p.value = value;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.row_chunks = head_dim * elem_bytes(dtype) / 16;
  p.block_shift = exact_log2(block_size);
  p.num_slots = num_slots;
  return pa::launch_reshape_and_cache(p, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_mapping,
                       int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t dtype, void *stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks < 0) return PA_ERR_BAD_SHAPE;
  if (elem_bytes(dtype) == 0 || !head_dim_ok(head_dim) || !block_size_ok(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int32_t> map(size_t(num_pairs) * 2);
    int32_t st = sync_copy_to_host(map.data(), block_mapping, sizeof(int32_t) * map.size(), s);
    if (st != PA_OK) return st;
    std::unordered_set<int32_t> dsts, srcs;
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int32_t a = map[2 * i], b = map[2 * i + 1];
      if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks) return PA_ERR_BAD_INDEX;
      if (!dsts.insert(b).second) return PA_ERR_BAD_INDEX;
      srcs.insert(a);
    }
    for (int32_t b : dsts)
      if (srcs.count(b)) return PA_ERR_BAD_INDEX;  // a destination that is also a source
  }
  pa::BlockCopyParams p{};
  p.src_k = k_cache;
  p.src_v = v_cache;
  p.dst_k = k_cache;
  p.dst_v = v_cache;
  p.block_mapping = block_mapping;
  p.num_pairs = num_pairs;
  p.src_blocks = num_blocks;
  p.dst_blocks = num_blocks;
  p.block_bytes = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  return pa::launch_copy_blocks(p, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                       const int32_t *block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t src_num_blocks,
                       int32_t dst_num_blocks, int32_t dtype, void *stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || src_num_blocks < 0 || dst_num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  if (elem_bytes(dtype) == 0 || !head_dim_ok(head_dim) || !block_size_ok(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return PA_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const void *dev[4];
  const void *host[4] = {src_k, src_v, dst_k, dst_v};
  for (int i = 0; i < 4; ++i) {
    const int32_t st = device_address(host[i], &dev[i]);
    if (st != PA_OK) return st;
  }
  const void *map_dev = nullptr;
  if (const int32_t st = device_address(block_mapping, &map_dev); st != PA_OK) return st;
  if (debug_checks()) {
    std::vector<int32_t> map(size_t(num_pairs) * 2);
    int32_t st = sync_copy_to_host(map.data(), block_mapping, sizeof(int32_t) * map.size(), s);
    if (st != PA_OK) return st;
    std::unordered_set<int32_t> dsts;
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int32_t a = map[2 * i], b = map[2 * i + 1];
      if (a < 0 || a >= src_num_blocks || b < 0 || b >= dst_num_blocks) return PA_ERR_BAD_INDEX;
      if (!dsts.insert(b).second) return PA_ERR_BAD_INDEX;
    }
  }
  pa::BlockCopyParams p{};
  p.src_k = dev[0];
  p.src_v = dev[1];
  p.dst_k = const_cast<void *>(dev[2]);
  p.dst_v = const_cast<void *>(dev[3]);
  p.block_mapping = static_cast<const int32_t *>(map_dev);
  p.num_pairs = num_pairs;
  p.src_blocks = src_num_blocks;
  p.dst_blocks = dst_num_blocks;
  p.block_bytes = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  return pa::launch_copy_blocks(p, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start_loc, float scale, int32_t num_seqs,
                   int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t max_blocks_per_seq, int32_t max_query_len, int32_t dtype,
                   void *stream) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_query_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return PA_ERR_BAD_SHAPE;
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || scale == INFINITY) return PA_ERR_UNSUPPORTED;
  if (!block_size_ok(block_size) || !group_ok(num_q_heads / num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (max_query_len > num_tokens) return PA_ERR_BAD_SHAPE;
  if (int64_t(max_blocks_per_seq) * block_size > (int64_t(1) << 31) - 1) return PA_ERR_BAD_SHAPE;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PA_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const int64_t group = num_q_heads / num_kv_heads;
  const int64_t q_tiles = (int64_t(max_query_len) * group + pa::kPrefillRows - 1) / pa::kPrefillRows;
  if (int64_t(num_seqs) * num_kv_heads * q_tiles > (int64_t(1) << 31) - 8) return PA_ERR_BAD_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int32_t> qsl(size_t(num_seqs) + 1), lens(num_seqs),
        tab(size_t(num_seqs) * max_blocks_per_seq);
    int32_t st = sync_copy_to_host(qsl.data(), query_start_loc, sizeof(int32_t) * qsl.size(), s);
    if (st == PA_OK) st = sync_copy_to_host(lens.data(), context_lens, sizeof(int32_t) * lens.size(), s);
    if (st == PA_OK) st = sync_copy_to_host(tab.data(), block_tables, sizeof(int32_t) * tab.size(), s);
    if (st != PA_OK) return st;
    if (qsl[0] != 0 || qsl[num_seqs] != num_tokens) return PA_ERR_BAD_INDEX;
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t chunk = qsl[i + 1] - qsl[i], n = lens[i];
      if (chunk < 0 || chunk > max_query_len || n < chunk ||
          int64_t(n) > int64_t(max_blocks_per_seq) * block_size)
        return PA_ERR_BAD_INDEX;
      if (chunk > 0 && n < 1) return PA_ERR_BAD_INDEX;
      for (int32_t b = 0; b < (n + block_size - 1) / block_size; ++b) {
        const int32_t id = tab[size_t(i) * max_blocks_per_seq + b];
        if (id < 0 || id >= num_blocks) return PA_ERR_BAD_INDEX;
      }
    }
  }
  pa::PrefillParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start_loc = query_start_loc;
  p.scale_log2 = float(double(scale) * 1.4426950408889634074);
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.block_shift = __builtin_ctz(unsigned(block_size));
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.q_tiles = int(q_tiles);
  return pa::launch_prefill(p, dtype, head_dim, max_query_len, s) == hipSuccess ? PA_OK
                                                                               : PA_ERR_HIP;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len,
                                int32_t partition_size, int32_t dtype) {
  if (check_decode_shapes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          dtype) != PA_OK)
    return size_t(-1);
  if (!partition_ok(partition_size)) return size_t(-1);
  return workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_size)
      .total;
}

}  // extern "C"

namespace {

// This step's new tokens (decode step form), or all null.
struct StepArgs {
  const void *key = nullptr;
  const void *value = nullptr;
  void *k_cache = nullptr;
  void *v_cache = nullptr;
  const int32_t *slot_mapping = nullptr;
  // The scratch is the library's static array (pa_decode_step_noalloc), not
  // the workspace arguments; its counters are cleared on the stream first.
  bool static_scratch = false;
};

int32_t decode_impl(void *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                    int32_t dtype, void *workspace, size_t workspace_bytes, void *stream,
                    const StepArgs &step) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t st = check_decode_shapes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   max_context_len, dtype);
  if (st != PA_OK) return st;
  if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return PA_ERR_BAD_SHAPE;
  if (int64_t(max_context_len) > int64_t(max_blocks_per_seq) * block_size) return PA_ERR_BAD_SHAPE;
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return PA_ERR_BAD_SHAPE;
  if (!partition_ok(partition_size)) return PA_ERR_BAD_SHAPE;
  int32_t part = 0;
  const bool balanced = use_balanced(num_seqs, num_kv_heads, max_context_len, partition_size,
                                     &part);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  const bool fused = step.slot_mapping != nullptr;
  if (fused) {
    if (!step.key || !step.value) return PA_ERR_NULL_POINTER;
    if (!aligned16(step.key) || !aligned16(step.value)) return PA_ERR_UNSUPPORTED;
  }
  const WsLayout lay = workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len, partition_size);
  const int32_t max_parts = balanced ? 1 : num_partitions(max_context_len, part);
  const bool needs_ws = balanced || max_parts > 1;
  if (step.static_scratch) {
    if (lay.total > pa::kNoallocScratchBytes) return PA_ERR_SCRATCH_TOO_SMALL;
    workspace = pa::noalloc_scratch();
    if (workspace == nullptr) return PA_ERR_HIP;
    workspace_bytes = pa::kNoallocScratchBytes;
  }
  if (needs_ws) {
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (workspace_bytes < lay.total) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return PA_ERR_UNSUPPORTED;
  }
  const int64_t num_slots = int64_t(num_blocks) * block_size;

  if (debug_checks()) {
    std::vector<int32_t> lens(num_seqs);
    std::vector<int32_t> tab(size_t(num_seqs) * max_blocks_per_seq);
    st = sync_copy_to_host(lens.data(), context_lens, sizeof(int32_t) * lens.size(), s);
    if (st != PA_OK) return st;
    st = sync_copy_to_host(tab.data(), block_tables, sizeof(int32_t) * tab.size(), s);
    if (st != PA_OK) return st;
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t n = lens[i];
      if (n < 0 || n > max_context_len) return PA_ERR_BAD_INDEX;
      const int32_t used = (n + block_size - 1) / block_size;
      for (int32_t j = 0; j < used; ++j) {
        const int32_t b = tab[size_t(i) * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks) return PA_ERR_BAD_INDEX;
      }
    }
    if (fused) {
      // Each written slot is either its own sequence's last attended position
      // or a slot no sequence attends: the launch reads no other slot it writes.
      std::vector<int32_t> slots(num_seqs);
      st = sync_copy_to_host(slots.data(), step.slot_mapping, sizeof(int32_t) * slots.size(), s);
      if (st != PA_OK) return st;
      std::unordered_set<int32_t> seen;
      bool any_elsewhere = false;
      for (int32_t i = 0; i < num_seqs; ++i) {
        const int32_t v = slots[i];
        if (v < 0) continue;
        if (v >= num_slots || !seen.insert(v).second) return PA_ERR_BAD_INDEX;
        const int32_t n = lens[i];
        bool last_pos = false;
        if (n >= 1) {
          const int32_t last = n - 1;
          last_pos = v == tab[size_t(i) * max_blocks_per_seq + last / block_size] * block_size +
                              last % block_size;
        }
        any_elsewhere |= !last_pos;
      }
      if (any_elsewhere) {
        for (int32_t i = 0; i < num_seqs; ++i)
          for (int32_t t = 0; t < lens[i]; ++t) {
            const int32_t slot =
                tab[size_t(i) * max_blocks_per_seq + t / block_size] * block_size + t % block_size;
            const bool own_last = t == lens[i] - 1 && slots[i] == slot;
            if (!own_last && seen.count(slot)) return PA_ERR_BAD_INDEX;
          }
      }
    }
    if (balanced && !step.static_scratch) {  // the arrival counters must be zero
      std::vector<int32_t> cnt(size_t(num_seqs) * num_kv_heads);
      st = sync_copy_to_host(cnt.data(), workspace, sizeof(int32_t) * cnt.size(), s);
      if (st != PA_OK) return st;
      for (int32_t c : cnt)
        if (c != 0) return PA_ERR_BAD_INDEX;
    }
  }

  if (step.static_scratch && balanced) {
    // The static scratch keeps the last call's contents: zero the arrival
    // counters (lay.counters bytes, within the scratch by the check above).
    if (pa::launch_clear_words(workspace, int(lay.counters / sizeof(int32_t)), s) != hipSuccess)
      return PA_ERR_HIP;
  }

  if (fused && !balanced) {
    // Fixed partitions cannot take the new rows from LDS: write them first.
    st = pa_reshape_and_cache(step.key, step.value, step.k_cache, step.v_cache,
                              step.slot_mapping, num_seqs, num_kv_heads, head_dim, block_size,
                              num_blocks, dtype, stream);
    if (st != PA_OK) return st;
  }

  pa::DecodeParams p{};
  p.out = out;
  if (needs_ws) {
    char *ws = static_cast<char *>(workspace);
    p.ws_count = reinterpret_cast<int32_t *>(ws);
    p.ws_acc = reinterpret_cast<float *>(ws + lay.counters);
    p.ws_m = p.ws_acc + lay.slots * lay.width;
    p.ws_l = p.ws_m + lay.stats;
  }
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.scale_log2 = float(double(scale) * 1.4426950408889634074);
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.head_dim = head_dim;
  p.block_shift = exact_log2(block_size);
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.partition_size = balanced ? 0 : part;
  p.max_partitions = max_parts;
  p.seg_cost = pa::flat_segment_cost();
  p.dtype = dtype;
  if (fused && balanced) {
    p.new_key = step.key;
    p.new_value = step.value;
    p.slot_mapping = step.slot_mapping;
    p.k_cache_w = step.k_cache;
    p.v_cache_w = step.v_cache;
    p.num_slots = num_slots;
  }
  const pa::DecodeStage stage = balanced ? pa::kStageFlat : pa::kStageBoth;
  return pa::launch_decode(p, s, stage) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, float scale,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                  int32_t dtype, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, partition_size, dtype, workspace,
                     workspace_bytes, stream, StepArgs{});
}

int32_t pa_decode_step(void *out, const void *q, const void *key, const void *value,
                       void *k_cache, void *v_cache, const int32_t *slot_mapping,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype,
                       void *workspace, size_t workspace_bytes, void *stream) {
  if (num_seqs > 0 && !slot_mapping) return PA_ERR_NULL_POINTER;
  StepArgs step;
  step.key = key;
  step.value = value;
  step.k_cache = k_cache;
  step.v_cache = v_cache;
  step.slot_mapping = slot_mapping;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, 0, dtype, workspace, workspace_bytes,
                     stream, step);
}

int32_t pa_decode_step_noalloc(void *out, const void *q, const void *key, const void *value,
                               void *k_cache, void *v_cache, const int32_t *slot_mapping,
                               const int32_t *block_tables, const int32_t *context_lens,
                               float scale, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int32_t dtype, void *stream) {
  if (num_seqs > 0 && !slot_mapping) return PA_ERR_NULL_POINTER;
  StepArgs step;
  step.key = key;
  step.value = value;
  step.k_cache = k_cache;
  step.v_cache = v_cache;
  step.slot_mapping = slot_mapping;
  step.static_scratch = true;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, 0, dtype, nullptr, 0, stream, step);
}

}  // extern "C"
