// pa_blocks.hip - whole-block copies between KV pools (gfx950).
//
// Two uses, both from [INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理",
// §4.3 (the block table allows flexible scheduling):
//  * copy-on-write: requests (or beams) share physical blocks through their
//    tables; before a shared block is written, the writer gets a private copy
//    of it in the same pool;
//  * swapping: the blocks of a preempted request move to host memory and come
//    back later, between a device pool and a pool in pinned host memory.
//
// Each (src, dst) pair copies one whole block of K and of V: every KV head and
// every slot, num_kv_heads * block_size * head_dim elements, bit for bit. One
// workgroup per (pair, slice of kCopySlice bytes); every thread moves 16-byte
// chunks, kCopyUnroll of K and of V in flight. Stores are non-temporal (the
// copy is not read back soon); loads are plain: measured on gfx950 with 128 KiB
// blocks, non-temporal loads as well were 25% slower, plain stores 6% slower.
#include "pa_common.h"
#include "pa_blocks.h"

namespace pa {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopySlice = int64_t(kCopyThreads) * 16 * kCopyUnroll;  // 16 KiB

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(BlockCopyParams p) {
  const int pair = blockIdx.x;
  const int src = p.block_mapping[2 * pair];
  const int dst = p.block_mapping[2 * pair + 1];
  // Pairs naming a block outside either pool copy nothing.
  if (src < 0 || src >= p.src_blocks || dst < 0 || dst >= p.dst_blocks) return;
  const int64_t chunks = p.block_bytes / 16;
  const int64_t first = blockIdx.y * (kCopySlice / 16);
  const int64_t last = min(first + kCopySlice / 16, chunks);
  const int64_t soff = (int64_t)src * chunks;
  const int64_t doff = (int64_t)dst * chunks;
  const u32x4 *sk = reinterpret_cast<const u32x4 *>(p.src_k) + soff;
  const u32x4 *sv = reinterpret_cast<const u32x4 *>(p.src_v) + soff;
  u32x4 *dk = reinterpret_cast<u32x4 *>(p.dst_k) + doff;
  u32x4 *dv = reinterpret_cast<u32x4 *>(p.dst_v) + doff;
  for (int64_t c0 = first + threadIdx.x; c0 < last; c0 += kCopyThreads * kCopyUnroll) {
    u32x4 k[kCopyUnroll], v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t c = c0 + u * kCopyThreads;
      if (c < last) {
        k[u] = sk[c];
        v[u] = sv[c];
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t c = c0 + u * kCopyThreads;
      if (c < last) {
        __builtin_nontemporal_store(k[u], dk + c);
        __builtin_nontemporal_store(v[u], dv + c);
      }
    }
  }
}

hipError_t launch_copy_blocks(const BlockCopyParams &p, hipStream_t stream) {
  if (p.num_pairs <= 0) return hipSuccess;
  const int64_t slices = (p.block_bytes + kCopySlice - 1) / kCopySlice;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(p.num_pairs, (unsigned)slices), dim3(kCopyThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
