// pa_prefill.hip - multi-token (chunked-prefill) paged attention for gfx950.
//
// Every query token of a chunk attends, head by head, to the cached keys of
// its sequence up to and including its own position: the per-step attention
// of [INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" §1.1 applied to
// each token of the chunk, with the cache read through the block table as in
// §3.3-§3.4. [OPS] (the ops-transformer PagedAttention article, its Python
// example) calls the operator with a whole sequence of queries, [1, 32, 8192,
// 64]; this is that call with the KV cache paged and the mask causal.
//
// Work: one workgroup (4 waves) per (sequence, KV head, tile of kPrefillRows
// query rows); a query row is a (token, query head of the group) pair, so the
// G heads that share a KV head share every K/V byte. Each wave owns 2 blocks
// of 16 rows. The keys are walked in tiles of 32 (any block size divides or is
// a multiple of... the tile is assembled key by key through the table, so
// block sizes 8-64 all work), double-buffered in LDS:
//
//   * K tile [32 keys][D] row-major (rows padded by 16 bytes).
//   * V tile transposed, [D][32 keys], so that a lane's MFMA operand (8
//     consecutive keys of one dim) is one 16-byte LDS read. The keys are
//     stored permuted (see v_slot) so that those 8 keys are exactly the 8
//     score values the same lane holds after the score product.
//
// Products, all on v_mfma_f32_16x16x32_{f16,bf16} with fp32 accumulation:
//   S^T [16 keys x 16 rows] = K [keys x D] . Q^T [D x rows]     (2 key blocks)
//   O^T [16 dims x 16 rows] += V^T [dims x 32 keys] . P^T [32 keys x rows]
// Computing the transposed scores puts each query row in one lane column, so
// the softmax weights P^T feed the second product from the registers they are
// in. The online softmax runs in the log2 domain with a running maximum per
// row; the row sum is kept per lane and reduced once at the end.
//
// Precision of P: fp16 weights carry 2^-11 relative error (the largest weight
// is exactly 1), bf16 weights 2^-8, too much for a 2e-3 output bound, so the
// bf16 path splits P into a bf16 high part and a bf16 remainder and issues
// both products (error about 2^-16).
#include "pa_common.h"
#include "pa_prefill.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kTileKeys = 32;

template <int D, int QB> struct PfShape {
  static constexpr int KS = D / 32;                      // k-steps of the score product
  static constexpr int DB = D / 16;                      // 16-dim blocks of the output
  static constexpr int ROWS = kPfWaves * QB * 16;        // query rows per workgroup
  static constexpr int KPITCH = D * 2 + 16;              // bytes per K row in LDS
  static constexpr int VPITCH = kTileKeys * 2;           // bytes per V^T row in LDS
  static constexpr int KBYTES = kTileKeys * KPITCH;
  static constexpr int BUF = KBYTES + D * VPITCH;        // one stage
  static constexpr int DCH = D / 8;                      // 16-byte chunks per row
  static constexpr int KCH_T = kTileKeys * DCH / kPfThreads;        // K chunks per thread
  static constexpr int VITEMS = (kTileKeys / 2) * DCH;              // (key pair, chunk) items
  static constexpr int VIT_T = (VITEMS + kPfThreads - 1) / kPfThreads;
  static_assert(kTileKeys * DCH % kPfThreads == 0, "K chunks must divide over the threads");
  static_assert(ROWS == kPrefillRows, "tile rows and host constant disagree");
};

// LDS position (0..31) of key k of a tile in the transposed V tile. Key
// 16*blk + 4*g + i (blk < 2, g < 4, i < 4) goes to 8*g + 4*blk + i: lane group
// g of a wave then reads keys {4g..4g+3, 16+4g..16+4g+3}, the keys whose
// scores it holds (result rows 4g+j of both 16-key score blocks).
__device__ __forceinline__ int v_slot(int k) {
  return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3);
}

template <int DT> __device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma16<PA_F16>(const u32x4 &a, const u32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16<PA_BF16>(const u32x4 &a, const u32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> one dword of two storage elements (round to nearest even).
template <int DT> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  using T = typename Store<DT>::T;
  const T a = Store<DT>::cvt(lo), b = Store<DT>::cvt(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Storage element -> float (exact).
template <int DT> __device__ __forceinline__ float unpack_lo(uint32_t w);
template <> __device__ __forceinline__ float unpack_lo<PA_F16>(uint32_t w) {
  return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xffffu)));
}
template <> __device__ __forceinline__ float unpack_lo<PA_BF16>(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
template <int DT> __device__ __forceinline__ float unpack_hi(uint32_t w);
template <> __device__ __forceinline__ float unpack_hi<PA_F16>(uint32_t w) {
  return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
}
template <> __device__ __forceinline__ float unpack_hi<PA_BF16>(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Global -> register staging of one key tile, and the table entries it needs.
template <int D, int QB> struct Stager {
  using S = PfShape<D, QB>;
  const char *kbase;     // k_cache + kh * B * D elements, in bytes
  const char *vbase;
  const int32_t *table;  // this sequence's table row
  int64_t blk_bytes;     // Hkv * B * D * 2: one physical block of all KV heads
  int row_bytes;         // D * 2
  int bshift, bmask;
  int n;                 // context length
  int kkey[S::KCH_T], kdc[S::KCH_T];   // K chunks of this thread
  int vkey[S::VIT_T], vdc[S::VIT_T];   // V (even key, chunk) items of this thread
  int kphys[S::KCH_T], vphys[S::VIT_T];
  u32x4 k[S::KCH_T], v0[S::VIT_T], v1[S::VIT_T];

  __device__ void init(int tid) {
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u) {
      const int c = tid + u * kPfThreads;
      kkey[u] = c / S::DCH;
      kdc[u] = c % S::DCH;
    }
#pragma unroll
    for (int u = 0; u < S::VIT_T; ++u) {
      // D = 64 has fewer items than threads: the upper threads repeat the
      // lower ones' items (identical loads and LDS writes), so no branch.
      const int it = (tid + u * kPfThreads) % S::VITEMS;
      vkey[u] = 2 * (it % (kTileKeys / 2));
      vdc[u] = it / (kTileKeys / 2);
    }
  }
  // Position of key `key` of tile j, clamped to the last cached position: keys
  // past the context read real data that the softmax then gives weight 0.
  __device__ __forceinline__ int pos_of(int j, int key) const { return min(j * kTileKeys + key, n - 1); }

  __device__ void load_table(int j) {
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u) kphys[u] = table[pos_of(j, kkey[u]) >> bshift];
#pragma unroll
    for (int u = 0; u < S::VIT_T; ++u) vphys[u] = table[pos_of(j, vkey[u]) >> bshift];
  }
  __device__ void load_kv(int j) {
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u) {
      const int pos = pos_of(j, kkey[u]);
      const int64_t off = int64_t(kphys[u]) * blk_bytes + (pos & bmask) * row_bytes + kdc[u] * 16;
      k[u] = *reinterpret_cast<const u32x4 *>(kbase + off);
    }
#pragma unroll
    for (int u = 0; u < S::VIT_T; ++u) {
      // The two keys of a pair are in one block (even key, block size >= 8).
      const int p0 = pos_of(j, vkey[u]), p1 = pos_of(j, vkey[u] + 1);
      const int64_t b = int64_t(vphys[u]) * blk_bytes + vdc[u] * 16;
      v0[u] = *reinterpret_cast<const u32x4 *>(vbase + b + (p0 & bmask) * row_bytes);
      v1[u] = *reinterpret_cast<const u32x4 *>(vbase + b + (p1 & bmask) * row_bytes);
    }
  }
  __device__ void store_lds(char *buf) const {
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u)
      *reinterpret_cast<u32x4 *>(buf + kkey[u] * S::KPITCH + kdc[u] * 16) = k[u];
#pragma unroll
    for (int u = 0; u < S::VIT_T; ++u) {
      char *col = buf + S::KBYTES + v_slot(vkey[u]) * 2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = v0[u][w], b = v1[u][w];
        // dims 8*dc + 2w and 8*dc + 2w + 1: (key, key + 1) pairs of each
        const uint32_t even = __builtin_amdgcn_perm(b, a, 0x05040100u);
        const uint32_t odd = __builtin_amdgcn_perm(b, a, 0x07060302u);
        *reinterpret_cast<uint32_t *>(col + (8 * vdc[u] + 2 * w) * S::VPITCH) = even;
        *reinterpret_cast<uint32_t *>(col + (8 * vdc[u] + 2 * w + 1) * S::VPITCH) = odd;
      }
    }
  }
};

template <int DT, int D, int G, int QB>
__global__ __launch_bounds__(kPfThreads) void prefill_kernel(PrefillParams p) {
  using S = PfShape<D, QB>;
  extern __shared__ __align__(16) char lds[];

  // Item of this workgroup. Workgroups are dispatched round-robin over the 8
  // XCDs; consecutive items (the query tiles of one (sequence, KV head), which
  // read the same K/V) are given to workgroups of one XCD so they share its L2.
  const int items = p.num_seqs * p.num_kv_heads * p.q_tiles;
  const int per_xcd = (items + 7) / 8;
  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (item >= items) return;
  const int qt = p.q_tiles - 1 - item % p.q_tiles;  // the longest tiles first
  const int kh = (item / p.q_tiles) % p.num_kv_heads;
  const int seq = item / (p.q_tiles * p.num_kv_heads);
  const int q0 = p.query_start_loc[seq];
  const int L = p.query_start_loc[seq + 1] - q0;
  const int rows = L * G;
  if (qt * S::ROWS >= rows) return;
  const int n = p.context_lens[seq];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int hq = p.num_q_heads;

  // Query rows of this lane (one per 16-row block) and their positions.
  u32x4 qreg[QB][S::KS];
  int qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = qt * S::ROWS + (wave * QB + qb) * 16 + lr;
    const int t = r / G;
    const bool valid = t < L;
    const int tc = valid ? t : L - 1;
    const int h = kh * G + r % G;
    qpos[qb] = n - L + t;
    const char *qrow = reinterpret_cast<const char *>(p.q) + (int64_t(q0 + tc) * hq + h) * D * 2;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + (32 * ks + 8 * lg) * 2);
      qreg[qb][ks] = valid ? v : u32x4{0, 0, 0, 0};
    }
  }
  const int r_last = min(rows, (qt + 1) * S::ROWS) - 1;
  const int last_pos = n - L + r_last / G;
  const int ntiles = last_pos / kTileKeys + 1;

  Stager<D, QB> st;
  st.kbase = reinterpret_cast<const char *>(p.k_cache) + int64_t(kh) * p.block_size * D * 2;
  st.vbase = reinterpret_cast<const char *>(p.v_cache) + int64_t(kh) * p.block_size * D * 2;
  st.table = p.block_tables + int64_t(seq) * p.max_blocks_per_seq;
  st.blk_bytes = int64_t(p.num_kv_heads) * p.block_size * D * 2;
  st.row_bytes = D * 2;
  st.bshift = p.block_shift;
  st.bmask = p.block_size - 1;
  st.n = n;
  st.init(tid);

  f32x4 acc[QB][S::DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int last = ntiles - 1;
  st.load_table(0);
  st.load_kv(0);
  st.load_table(min(1, last));
  st.store_lds(lds);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    // Next tile's loads are in flight while this one is computed. The last
    // iteration reloads tile `last` into the idle buffer (never read).
    st.load_kv(min(j + 1, last));
    st.load_table(min(j + 2, last));
    const char *kb_lds = lds + (j & 1) * S::BUF;
    const char *vt_lds = kb_lds + S::KBYTES;

    // S^T = K . Q^T for 2 blocks of 16 keys.
    f32x4 s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb][0] = s[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(kb_lds + (16 * kb + lr) * S::KPITCH +
                                                           (32 * ks + 8 * lg) * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma16<DT>(a, qreg[qb][ks], s[qb][kb]);
      }
    }

    // Online softmax per query row (lane column), and P^T in storage form.
    u32x4 ph[QB], pl[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = j * kTileKeys + 16 * kb + 4 * lg + jj;
          const float v = s[qb][kb][jj] * p.scale_log2;
          x[4 * kb + jj] = key <= qpos[qb] ? v : -INFINITY;
        }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = xor_max(mx);
      const float m_new = fmaxf(m[qb], mx);
      const float alpha = fast_exp2(m[qb] - m_new);
      m[qb] = m_new;
      float e[8], sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = fast_exp2(x[i] - m_new);
        sum += e[i];
      }
      l[qb] = l[qb] * alpha + sum;
#pragma unroll
      for (int db = 0; db < S::DB; ++db) acc[qb][db] *= alpha;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t hw = pack2<DT>(e[2 * w], e[2 * w + 1]);
        ph[qb][w] = hw;
        if (DT == PA_BF16)
          pl[qb][w] = pack2<DT>(e[2 * w] - unpack_lo<DT>(hw), e[2 * w + 1] - unpack_hi<DT>(hw));
      }
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      const u32x4 a = *reinterpret_cast<const u32x4 *>(vt_lds + (16 * db + lr) * S::VPITCH + 16 * lg);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        acc[qb][db] = mfma16<DT>(a, ph[qb], acc[qb][db]);
        if (DT == PA_BF16) acc[qb][db] = mfma16<DT>(a, pl[qb], acc[qb][db]);
      }
    }

    st.store_lds(lds + ((j + 1) & 1) * S::BUF);
    __syncthreads();
  }

  // out = acc / l for the valid rows.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.f / xor_sum(l[qb]);
    const int r = qt * S::ROWS + (wave * QB + qb) * 16 + lr;
    const int t = r / G;
    if (t >= L) continue;
    const int h = kh * G + r % G;
    char *orow = reinterpret_cast<char *>(p.out) + (int64_t(q0 + t) * hq + h) * D * 2;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      const f32x4 o = acc[qb][db] * inv;
      uint2 w;
      w.x = pack2<DT>(o[0], o[1]);
      w.y = pack2<DT>(o[2], o[3]);
      *reinterpret_cast<uint2 *>(orow + (16 * db + 4 * lg) * 2) = w;
    }
  }
}

template <int DT, int D, int G>
hipError_t launch_g(const PrefillParams &p, hipStream_t stream) {
  constexpr int QB = 2;
  using S = PfShape<D, QB>;
  const int64_t items = int64_t(p.num_seqs) * p.num_kv_heads * p.q_tiles;
  if (items == 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_kernel<DT, D, G, QB>), dim3(unsigned(grid)), dim3(kPfThreads),
                     2 * S::BUF, stream, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_d(const PrefillParams &p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<DT, D, 1>(p, stream);
    case 2: return launch_g<DT, D, 2>(p, stream);
    case 4: return launch_g<DT, D, 4>(p, stream);
    case 8: return launch_g<DT, D, 8>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const PrefillParams &p, int head_dim, int group, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<DT, 64>(p, group, stream);
    case 128: return launch_d<DT, 128>(p, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, int max_query_len,
                          hipStream_t stream) {
  (void)max_query_len;
  const int group = p.num_q_heads / p.num_kv_heads;
  switch (dtype) {
    case PA_F16: return launch_dt<PA_F16>(p, head_dim, group, stream);
    case PA_BF16: return launch_dt<PA_BF16>(p, head_dim, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
