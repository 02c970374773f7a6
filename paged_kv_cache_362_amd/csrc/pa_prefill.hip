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
// of 16 rows. The keys are walked in tiles of 32, assembled through the table
// (so block sizes 8-64 all work) by gfx950's direct global -> LDS loads into
// three LDS buffers (two tiles in flight while one is read), each a K tile
// and a V tile, both [32 keys][D] row-major with the 16-byte chunks of each
// row permuted (swz). The V operand of the second product (8 keys of one dim
// per lane, the keys whose scores that lane holds) is read from the row-major
// V tile by gfx950's transposing LDS read, so V is staged exactly as K is.
//
// Products, all on v_mfma_f32_16x16x32_{f16,bf16} with fp32 accumulation:
//   S^T [16 keys x 16 rows] = K [keys x D] . Q^T [D x rows]     (2 key blocks)
//   O^T [16 dims x 16 rows] += V^T [dims x 32 keys] . P^T [32 keys x rows]
// Computing the transposed scores puts each query row in one lane column, so
// the softmax weights P^T feed the second product from the registers they are
// in. The online softmax runs in the log2 domain with a running maximum per
// row that is raised lazily (see kRescaleSlack); the row sums come from one
// more MFMA per row block against an all-ones V^T block. Scores are masked
// only in the tiles that cross a row's position. The scale must be positive
// (the tile maximum is taken on unscaled scores).
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
constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay below 256

template <int D, int QB> struct PfShape {
  static constexpr int KS = D / 32;                      // k-steps of the score product
  static constexpr int DB = D / 16;                      // 16-dim blocks of the output
  static constexpr int ROWS = kPfWaves * QB * 16;        // query rows per workgroup
  static constexpr int KPITCH = D * 2;                   // bytes per K or V row in LDS
  static constexpr int KBYTES = kTileKeys * KPITCH;
  static constexpr int BUF = 2 * KBYTES;                 // one stage: K tile, V tile
  static constexpr int DCH = D / 8;                      // 16-byte chunks per row
  static constexpr int KCH_T = kTileKeys * DCH / kPfThreads;        // (key, column) items per thread
  static constexpr int RPB = 256 / KPITCH;               // rows per 256 bytes (64 LDS banks)
  static_assert(kTileKeys * DCH % kPfThreads == 0, "K chunks must divide over the threads");
  static_assert(ROWS == kPrefillRows, "tile rows and host constant disagree");
};

// 16-byte chunk c of key k's row sits at chunk c ^ swz(k) of that row in
// LDS. With m = (k / RPB) % DCH, swz moves m's low bits up by one and its top
// bit down to bit 0, so that the 16 keys a K read takes at one column, and
// the 8 consecutive keys of a transposing V read at one column pair, fall in
// distinct 16-byte bank groups.
template <int D> __device__ __forceinline__ uint32_t swz(uint32_t k) {
  using S = PfShape<D, 2>;
  const uint32_t m = (k / S::RPB) % S::DCH;
  return ((m & (S::DCH / 2 - 1)) << 1) | (m / (S::DCH / 2));
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

// Two floats -> two storage elements in one dword, round to nearest even, by
// gfx950's packed conversions (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int DT> __device__ __forceinline__ uint32_t cvt2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t cvt2<PA_F16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
template <> __device__ __forceinline__ uint32_t cvt2<PA_BF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
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

// Maximum over the 4 lanes l, l^16, l^32, l^48 (the lane groups that
// hold one query row's keys). permlane16_swap hands each lane the values of
// its row pair (rows 2r, 2r+1), permlane32_swap those of lanes l%32 and
// 32 + l%32: two VALU exchanges, no LDS traffic. The pair's elements are
// copied to scalars before any bit cast (a bit cast of a vector element
// lvalue reads element 0 with this compiler).
__device__ __forceinline__ void swap16(float v, float &a, float &b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap32(float v, float &a, float &b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float group_max(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

// Transposing LDS read of 4 16-bit elements (ds_read_b64_tr_b16): within each
// group of 16 lanes, lane c receives as its element r the element c % 4 of the
// 8 bytes addressed by lane 4 r + c / 4 of the group.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const char *p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((address_space(3))) char lds_char;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)((lds_char *)p));
  return __builtin_bit_cast(uint2, r);
}

// Table entries of one key tile: a wave's 64 slots of one load are 64 / DCH
// consecutive keys, aligned to that count, which divides every block size
// (8 to 64), so they lie in one block and the entry is uniform across the
// wave (scalar registers and a scalar load). Positions past the context are
// clamped to its last one, which then lies in the wave's aligned group or
// before it (all of the wave's keys clamped): the block is still the one the
// wave's first key gives.
template <int D> struct KVStage {
  using S = PfShape<D, 2>;
  int32_t phys[S::KCH_T];
};

// What each thread stages of a key tile, and how. The tile's K (and V) rows
// are staged by direct global -> LDS loads of 16 bytes per lane (lane i's
// bytes land at the wave's LDS address plus 16 i), so a wave's load fills 64
// consecutive 16-byte LDS slots, slot 64 (wave + 4 u) + lane.
// Slot q holds key q / DCH, column chunk (q % DCH) ^ swz(key): so the 8 (or
// 16) lanes of one key read its row's 128 (or 256) bytes from global memory.
template <int D> struct Stager {
  using S = PfShape<D, 2>;
  const char *kbase;     // k_cache + kh * B * D elements, in bytes
  const char *vbase;
  const int32_t *table;  // this sequence's table row
  uint32_t blk_bytes;    // Hkv * B * D * 2: one physical block of all KV heads
  uint32_t max_block;    // num_blocks - 1: table entries are clamped to it
  uint32_t bshift, bmask;
  uint32_t last_pos;     // context length - 1
  uint32_t key[S::KCH_T], col[S::KCH_T];  // item's key in the tile and byte column
  uint32_t slot0[S::KCH_T];               // LDS byte offset of the wave's 64 slots
  uint32_t key0[S::KCH_T];                // the wave's first key of each load (uniform)

  __device__ void init(int tid) {
    const int wave = tid / kWave, lane = tid % kWave;
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u) {
      const int q = (wave + kPfWaves * u) * kWave + lane;
      key[u] = q / S::DCH;
      col[u] = ((q % S::DCH) ^ swz<D>(key[u])) * 16;
      slot0[u] = __builtin_amdgcn_readfirstlane((wave + kPfWaves * u) * kWave * 16);
      key0[u] = __builtin_amdgcn_readfirstlane((wave + kPfWaves * u) * kWave / S::DCH);
    }
  }
  // Position of key `k` of tile j, clamped to the last cached position: keys
  // past the context read real data that the softmax then gives weight 0.
  __device__ __forceinline__ uint32_t pos_of(int j, uint32_t k) const {
    return min(uint32_t(j) * kTileKeys + k, last_pos);
  }

  __device__ void load_table(KVStage<D> &r, int j) const {
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u) {
      // Read through the constant address space: the table is not written
      // during the call, and the uniform load then goes through the scalar
      // cache, apart from the vector-memory count the K/V loads are waited on.
      typedef const __attribute__((address_space(4))) int32_t const_i32;
      r.phys[u] = ((const_i32 *)table)[pos_of(j, key0[u]) >> bshift];
    }
  }
  // 2 * KCH_T loads (K, V per item), in that order.
  __device__ void load_kv(const KVStage<D> &r, int j, char *buf) const {
    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(1))) void glb_void;
#pragma unroll
    for (int u = 0; u < S::KCH_T; ++u) {
      // Never address outside the pool, whatever the table holds. The entry
      // is clamped here, at its use one tile after its load.
      // The block's address is uniform (scalar registers); each lane adds its
      // row and column as a 32-bit offset.
      const uint32_t phys = min(uint32_t(max(int(r.phys[u]), 0)), max_block);
      const uint64_t blk = uint64_t(phys) * blk_bytes;
      const uint32_t off = ((pos_of(j, key[u]) & bmask) * (D * 2)) | col[u];
      __builtin_amdgcn_global_load_lds((glb_void *)(kbase + blk + off), (lds_void *)(buf + slot0[u]),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void *)(vbase + blk + off),
                                       (lds_void *)(buf + S::KBYTES + slot0[u]), 16, 0, 0);
    }
  }
};

// Workgroup barrier that waits for nothing: the LDS loads' completion is
// waited for explicitly (wait_vm), and the compiler fences keep memory
// accesses on their side of it.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt for at most N vector-memory operations and no LDS operation
// outstanding (gfx9 encoding): before a barrier, this wave's reads of the
// buffer that the next loads overwrite have completed.
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// head_dim 64 fits 128 VGPRs with no scratch when bounded: 4 waves per SIMD,
// which lets the softmax of one wave overlap the products of more others.
// head_dim 128 is left unbounded and fits 168 (3 waves).
template <int DT, int D, int G, int QB, int NSET>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 1)))
void prefill_kernel(PrefillParams p) {
  using S = PfShape<D, QB>;
  static_assert(NSET == 3, "three LDS buffers");
  // NSET = 3 K/V tile buffers: tile j is read from buffer j % 3 while the
  // loads of tiles j + 1 and j + 2 land in the other two. Separate arrays, so
  // the compiler sees that reading one does not wait for loads into another.
  __shared__ __align__(16) char lds0[S::BUF];
  __shared__ __align__(16) char lds1[S::BUF];
  __shared__ __align__(16) char lds2[S::BUF];

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
  // A chunk outside the packed tokens, a chunk longer than its context, or a
  // context longer than its table row breaks the call's preconditions
  // (checked on the host only under PA_DEBUG): such a sequence gets no output
  // rather than accesses outside q, out or its table row. Positions below are
  // then in [0, n), so the uint32 ones are safe.
  if (q0 < 0 || q0 > p.num_tokens - L || L > n || n > (p.max_blocks_per_seq << p.block_shift))
    return;

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
  const int wave_min_qpos =
      __builtin_amdgcn_readfirstlane(n - L + (qt * S::ROWS + wave * QB * 16) / G);
  const int r_last = min(rows, (qt + 1) * S::ROWS) - 1;
  const int last_pos = n - L + r_last / G;
  const int ntiles = last_pos / kTileKeys + 1;

  Stager<D> st;
  st.kbase = reinterpret_cast<const char *>(p.k_cache) + int64_t(kh) * p.block_size * D * 2;
  st.vbase = reinterpret_cast<const char *>(p.v_cache) + int64_t(kh) * p.block_size * D * 2;
  st.table = p.block_tables + int64_t(seq) * p.max_blocks_per_seq;
  st.blk_bytes = uint32_t(p.num_kv_heads) * p.block_size * D * 2;
  st.max_block = uint32_t(p.num_blocks - 1);
  st.bshift = p.block_shift;
  st.bmask = p.block_size - 1;
  st.last_pos = n - 1;
  st.init(tid);

  // acc: O^T blocks; lsum: the row sums of P, as one more O^T block whose
  // V^T rows are all ones (the MFMA sums the weights it is given, so the
  // denominator uses exactly the rounded weights the numerator does).
  f32x4 acc[QB][S::DB], lsum[QB];
  float nm[QB];  // minus the running maximum (log2 domain), as the exponent FMA takes it
  // head_dim 64: raw score above which a row's weight would exceed
  // 2^kRescaleSlack, (kRescaleSlack + m) / scale_log2 (the scale is
  // positive), so the test below needs no FMA. At 128 the two extra live
  // VGPRs would cost the kernel its third wave per SIMD, and the test takes
  // the FMA instead.
  float thr[QB];
  const float inv_scale_log2 = 1.f / p.scale_log2;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    nm[qb] = INFINITY;
    thr[qb] = -INFINITY;
    lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < S::DB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = DT == PA_F16 ? 0x3C003C00u : 0x3F803F80u;  // two 1.0 elements
  const u32x4 ones = {one2, one2, one2, one2};

  // Per-lane LDS offsets of the operand reads (the chunk swizzle is a XOR
  // with a per-lane value, so the per-step offsets are formed once here).
  uint32_t koff[S::KS];
  {
    const uint32_t x = uint32_t(lg) ^ swz<D>(uint32_t(lr));
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) koff[ks] = lr * S::KPITCH + ((x ^ (4 * ks)) * 16);
  }
  const uint32_t vkey = 4 * lg + (lr >> 2);
  const uint32_t vx = uint32_t((lr & 3) >> 1) ^ swz<D>(vkey);
  const uint32_t vrow = vkey * S::KPITCH + (lr & 1) * 8;
  // At head_dim 64 the per-block offsets are formed once (4 VGPRs). At 128
  // they are formed per tile: written as 8 values formed once, the kernel
  // took 186-198 VGPRs instead of 166 and lost its third wave per SIMD.
  uint32_t voff[D == 64 ? S::DB : 1];
#pragma unroll
  for (int db = 0; db < (D == 64 ? S::DB : 1); ++db) voff[db] = vrow + (vx ^ (2 * db)) * 16;

  // Pipeline: at the top of iteration j, buffer j % 3 holds tile j (every
  // wave's loads of it complete, then a barrier), the loads of tile j + 1 are
  // in flight into buffer (j + 1) % 3, and T[j % 3] holds the table entries of
  // tile j + 2. Iteration j requests the entries of tile j + 3, then loads
  // tile j + 2 into buffer (j + 2) % 3, which every wave finished reading in
  // iteration j - 1. Tiles past the last are clamped to it (the loads are
  // redundant but keep the count of loads per iteration fixed, which the wait
  // before the barrier relies on), and iterations past it compute with every
  // key masked (no effect), so the loop runs a multiple of 3 iterations with
  // compile-time buffer indices.
  const int last = ntiles - 1;
  char *const bufs[NSET] = {lds0, lds1, lds2};
  KVStage<D> T[NSET];  // T[(t + 1) % NSET] holds the entries of tile t
#pragma unroll
  for (int t = 0; t < NSET - 1; ++t) {
    st.load_table(T[(t + 1) % NSET], min(t, last));
    st.load_kv(T[(t + 1) % NSET], min(t, last), bufs[t]);
  }
  st.load_table(T[0], min(NSET - 1, last));
  wait_vm<S::KCH_T * 2 * (NSET - 2)>();  // tile 0 complete
  wg_barrier();

  for (int j0 = 0; j0 < ntiles; j0 += NSET) {
#pragma unroll
    for (int u = 0; u < NSET; ++u) {
      const int j = j0 + u;
      KVStage<D> &cur = T[u];                  // entries of tile j + NSET - 1
      KVStage<D> &nxt = T[(u + 1) % NSET];     // gets the entries of tile j + NSET
      st.load_table(nxt, min(j + NSET, last));
      st.load_kv(cur, min(j + NSET - 1, last), bufs[(u + NSET - 1) % NSET]);
      const bool live = j < ntiles;
      const char *kb_lds = bufs[u];
      const char *vt_lds = kb_lds + S::KBYTES;

      // S^T = K . Q^T for 2 blocks of 16 keys.
      f32x4 s[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][0] = s[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a =
              *reinterpret_cast<const u32x4 *>(kb_lds + 16 * kb * S::KPITCH + koff[ks]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma16<DT>(a, qreg[qb][ks], s[qb][kb]);
        }
      }

      // Mask keys past each row's position (and every key of the iterations
      // past the last tile). Only tiles that reach past the wave's first row
      // need it; the branch is uniform across the wave.
      if (!live || j * kTileKeys + kTileKeys - 1 > wave_min_qpos) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int key = j * kTileKeys + 16 * kb + 4 * lg + jj;
              if (!(live && key <= qpos[qb])) s[qb][kb][jj] = -INFINITY;
            }
      }

      // Online softmax per query row (lane column). The running maximum m is
      // only raised when a row's tile maximum exceeds it by more than
      // kRescaleSlack (log2 units): weights then stay below 2^kRescaleSlack,
      // well inside fp16/bf16 range, and the rescale of the accumulators (a
      // branch uniform across the wave) is rare after the first tile. Each
      // lane tests its own 8 scores; only the branch takes the row maxima
      // across lanes.
      bool raise = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (D == 64) {
          // a chain of three-input maxima, against the raw-score threshold
          float mx = fmaxf(fmaxf(s[qb][0][0], s[qb][0][1]), s[qb][0][2]);
          mx = fmaxf(fmaxf(mx, s[qb][0][3]), s[qb][1][0]);
          mx = fmaxf(fmaxf(mx, s[qb][1][1]), s[qb][1][2]);
          raise |= fmaxf(mx, s[qb][1][3]) > thr[qb];
        } else {
          float mx = fmaxf(fmaxf(s[qb][0][0], s[qb][0][1]), fmaxf(s[qb][0][2], s[qb][0][3]));
          mx = fmaxf(mx, fmaxf(fmaxf(s[qb][1][0], s[qb][1][1]), fmaxf(s[qb][1][2], s[qb][1][3])));
          raise |= fmaf(mx, p.scale_log2, nm[qb]) > kRescaleSlack;
        }
      }
      if (__any(raise)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // the lane's maximum again, in another order (nothing held across the test)
          float mx = fmaxf(fmaxf(s[qb][0][0], s[qb][1][0]), fmaxf(s[qb][0][1], s[qb][1][1]));
          mx = fmaxf(mx, fmaxf(fmaxf(s[qb][0][2], s[qb][1][2]), fmaxf(s[qb][0][3], s[qb][1][3])));
          const float m_new = fmaxf(-nm[qb], group_max(mx) * p.scale_log2);
          const float alpha = fast_exp2(-nm[qb] - m_new);
          nm[qb] = -m_new;
          if (D == 64) thr[qb] = (kRescaleSlack + m_new) * inv_scale_log2;
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < S::DB; ++db) acc[qb][db] *= alpha;
        }
      }
      u32x4 ph[QB], pl[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float e[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            e[4 * kb + jj] = fast_exp2(fmaf(s[qb][kb][jj], p.scale_log2, nm[qb]));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t hw = cvt2<DT>(e[2 * w], e[2 * w + 1]);
          ph[qb][w] = hw;
          if (DT == PA_BF16)
            pl[qb][w] = cvt2<DT>(e[2 * w] - unpack_lo<DT>(hw), e[2 * w + 1] - unpack_hi<DT>(hw));
        }
      }

      // O^T += V^T . P^T, and the row sums. A lane's V^T operand is dim
      // 16 db + lr of the 8 keys whose weights it holds (keys 4 lg .. 4 lg + 3
      // and 16 + 4 lg .. 16 + 4 lg + 3 of the tile, in that order), built from
      // the row-major V tile by two transposing reads: lane (lr, lg) addresses
      // key 4 lg + lr / 4 (then that key + 16), dims 16 db + 4 (lr % 4) .. + 3.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        lsum[qb] = mfma16<DT>(ones, ph[qb], lsum[qb]);
        if (DT == PA_BF16) lsum[qb] = mfma16<DT>(ones, pl[qb], lsum[qb]);
      }
#pragma unroll
      for (int db = 0; db < S::DB; ++db) {
        const uint32_t vo = D == 64 ? voff[D == 64 ? db : 0] : vrow + (vx ^ (2 * db)) * 16;
        const uint2 lo = lds_read_tr16(vt_lds + vo);
        const uint2 hi = lds_read_tr16(vt_lds + vo + 16 * S::KPITCH);
        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          acc[qb][db] = mfma16<DT>(a, ph[qb], acc[qb][db]);
          if (DT == PA_BF16) acc[qb][db] = mfma16<DT>(a, pl[qb], acc[qb][db]);
        }
      }

      // Tile j + 1 complete for this wave: only tile j + 2's loads were
      // issued after its loads (the table entries take the scalar path).
      // Then for every wave.
      wait_vm<S::KCH_T * 2 * (NSET - 2)>();
      wg_barrier();
    }
  }
  wait_vm<0>();  // no load into this workgroup's LDS outlives its waves

  // out = acc / l for the valid rows. The row index is rebuilt from an
  // opaque copy of the lane so that no address of this store is computed
  // before the loop and held in registers across it.
  int lr_out = lr;
  asm volatile("" : "+v"(lr_out));
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.f / lsum[qb][0];
    const int r = qt * S::ROWS + (wave * QB + qb) * 16 + lr_out;
    const int t = r / G;
    if (t >= L) continue;
    const int h = kh * G + r % G;
    char *orow = reinterpret_cast<char *>(p.out) + (int64_t(q0 + t) * hq + h) * D * 2;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      const f32x4 o = acc[qb][db] * inv;
      uint2 w;
      w.x = cvt2<DT>(o[0], o[1]);
      w.y = cvt2<DT>(o[2], o[3]);
      *reinterpret_cast<uint2 *>(orow + (16 * db + 4 * lg) * 2) = w;
    }
  }
}

template <int DT, int D, int G>
hipError_t launch_g(const PrefillParams &p, hipStream_t stream) {
  constexpr int QB = 2;
  constexpr int NSET = 3;
  const int64_t items = int64_t(p.num_seqs) * p.num_kv_heads * p.q_tiles;
  if (items == 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_kernel<DT, D, G, QB, NSET>), dim3(unsigned(grid)), dim3(kPfThreads),
                     0, stream, p);
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
