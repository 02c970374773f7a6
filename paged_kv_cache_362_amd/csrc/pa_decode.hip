// pa_decode.hip - decode-phase paged attention kernels for gfx950 (MI355X).
//
// What is computed ([INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理",
// §1.1 and §3.4): for sequence s and query head h, the scores of the new query
// against the first n = context_lens[s] cached keys of KV head h / G, scaled,
// softmax-normalised, and used to average the cached values. The cached rows
// are found through the sequence's block table (§3.3).
//
// How. Split-K in the manner of flash decoding ([INFRA] Q2 of §8): the
// context of each (sequence, KV head) is cut into pieces, each piece is reduced
// to (running max, sum of weights, weighted sum of values), and the pieces are
// combined by a log-sum-exp reduction. Two ways of cutting:
//   decode_flat_kernel       balanced form: the whole (sequence, KV head, tile)
//                            space is divided evenly among the resident
//                            workgroups, one launch, split heads combined by
//                            the last workgroup to finish;
//   decode_partition_kernel  fixed partitions of P tokens, one workgroup each,
//                            then decode_reduce_kernel.
// Four waves per workgroup. All G query heads of a KV head share every K/V
// byte read ([INFRA] §2.1, GQA).
//
// * Work of a workgroup: a segment (a token range of one sequence and KV
//   head) is cut into windows; each of the four waves takes a contiguous chunk
//   of a window that touches at most 64 blocks. The wave loads the chunk's
//   table entries once, one per lane (clamped into the pool), so a 16-token
//   tile's physical block is a v_readlane away and tile base addresses live in
//   scalar registers.
// * Rounds: a wave takes NT 16-token tiles per round. The next round's K and V
//   loads are issued before the current round is consumed (two register
//   buffers, with a scheduling barrier so the compiler cannot sink the loads to
//   their uses; the loop holds no other memory operation), which keeps 16-32
//   KB per wave in flight: the path is bound by HBM reads, not arithmetic.
// * QK^T on the matrix cores (v_mfma 16x16x32 f16/bf16, 16x16x4 f32). Operand
//   A is the K tile (row m = a token, loaded as 16 rows x 64 bytes per load),
//   operand B the group's queries (column n = query head n % G), staged in LDS
//   once per segment rather than held in registers (fewer VGPRs: GQA-4 runs
//   three waves per SIMD instead of two). The tile's
//   tokens are assigned to A rows through a fixed permutation chosen so that
//   result slot i of lane l is the score of exactly the token whose V row
//   segment lane l loads in V load i: scores never cross lanes for MHA.
// * V is loaded as whole contiguous rows (64 lanes x 16 bytes = 1 KB per load;
//   a "token group" of 8 or 16 lanes holds one token's row) and accumulated in
//   float32 on the vector ALUs. With G > 1 a lane computes the softmax weight
//   of its own head (n % G) and the other heads' weights arrive by DPP/swizzle
//   from the lanes of the same token group.
// * Online softmax in the log2 domain, per (token group, head): each token
//   group keeps its own reference maximum, so the loop has no cross-lane max,
//   and raises it (rescaling the accumulators) only when a round exceeds it by
//   2^8, so the per-round rescale is a rarely taken branch.
// * Masking by select: scores of tokens at or past the context end are -inf and
//   their V values are replaced by 0, so NaN in unused slots cannot leak. Table
//   entries are clamped into [0, num_blocks), so no load leaves the pool.
// * Epilogue: token groups merge across lanes (shuffles), waves through LDS. A
//   piece that is a whole (sequence, KV head) writes its output rows;
//   otherwise its (max, sum, weighted values) go to the workspace.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

template <int DT, int D, int G, int NT> struct DecodeShape {
  static constexpr int E = Elem<DT>::kBytes;
  static constexpr int EPC = Elem<DT>::kPerChunk;    // elements per 16-byte chunk
  static constexpr int ROWB = D * E;                 // bytes of one token's row
  static constexpr int SEGB = ROWB < 256 ? ROWB : 256;  // row segment one token group loads
  static constexpr int NSEG = ROWB / SEGB;           // segments per row (1 or 2)
  static constexpr int LPT = SEGB / 16;              // lanes per token group (8 or 16)
  static constexpr int TPI = kWave / LPT;            // tokens per V load (8 or 4)
  static constexpr int VI = 16 / TPI;                // V loads per tile and segment
  static constexpr int NV = VI * NSEG;               // V loads per tile
  static constexpr int KS = ROWB / 64;               // K loads per tile (MFMA k-steps of 64 B)
  static constexpr int ROUND = 16 * NT;              // tokens per round
  static_assert(ROWB == 128 || ROWB == 256 || ROWB == 512, "row must be 128, 256 or 512 bytes");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(G <= LPT, "a token group must hold every head of the group");
};

// acc += A(16 x k) * B(k x 16) over one 16-byte chunk of the contraction.
template <int DT> __device__ __forceinline__ f32x4 mfma_chunk(const u32x4 &a, const u32x4 &b, f32x4 acc);

template <> __device__ __forceinline__ f32x4 mfma_chunk<PA_F16>(const u32x4 &a, const u32x4 &b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma_chunk<PA_BF16>(const u32x4 &a, const u32x4 &b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma_chunk<PA_F32>(const u32x4 &a, const u32x4 &b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, chunk_word(a, e)),
                                               __builtin_bit_cast(float, chunk_word(b, e)), acc,
                                               0, 0, 0);
  return acc;
}

// Token (0..15, within a 16-token tile) that MFMA row m stands for. Result slot
// j of lane l is row 4*(l/16) + j; the permutation makes that the token lane l
// holds in V load j (LPT 16) or 2*(j/2)... (LPT 8), see the header comment.
template <int LPT> __device__ __forceinline__ int tile_token_of_row(int m) {
  const int g = m >> 2, j = m & 3;
  if (LPT == 16) return 4 * j + g;
  return 8 * (j >> 1) + 2 * g + (j & 1);
}

// Value of v in the lane of this lane's token group whose own head is h.
template <int G> __device__ __forceinline__ float from_head(float v, int h) {
  if (G == 1) return v;
  const int iv = __builtin_bit_cast(int, v);
  if (G <= 4) {
    // quad_perm [h, h, h, h]: lane (l & ~3) | h
    switch (h) {
      case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x00, 0xF, 0xF, false));
      case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x55, 0xF, 0xF, false));
      case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0xAA, 0xF, 0xF, false));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0xFF, 0xF, 0xF, false));
    }
  }
  // bitmask swizzle inside 32-lane halves: lane (l & 0x18) | h
  switch (h) {
    case 0: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (0 << 5)));
    case 1: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (1 << 5)));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (2 << 5)));
    case 3: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (3 << 5)));
    case 4: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (4 << 5)));
    case 5: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (5 << 5)));
    case 6: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (6 << 5)));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x18 | (7 << 5)));
  }
}

template <int DT, int D, int G, int NT> struct RoundBuf {
  using S = DecodeShape<DT, D, G, NT>;
  u32x4 k[NT][S::KS];
  u32x4 v[NT][S::NV];
};

// Per-wave constants of the loop over one chunk of a segment (a token range
// of one sequence and KV head). The chunk's table entries (at most 64) are
// held one per lane: lane i has the entry of block first_blk + i.
struct WaveCtx {
  const char *k_cache;
  const char *v_cache;
  int64_t head_off;   // kv head offset inside a block, bytes
  int64_t blk_bytes;  // bytes of one physical block (all kv heads)
  int tabv;           // clamped table entry of block first_blk + lane
  int first_blk;      // first block of the chunk
  int bshift;
  uint32_t koff;      // K lane offset in its tile (16-token blocks and larger)
  uint32_t koff8;     // K lane offset in its block (8-token blocks)
  uint32_t voff;      // V lane offset inside a V load
  bool khi;           // 8-token blocks: this lane's K row is in the tile's second block
};

// 16-byte K/V load at a wave-uniform address `base + imm` plus a per-lane
// 32-bit offset (one address register per tile, immediates for the rest). The
// pools are streamed once per call, so the loads are non-temporal: they do not
// displace other lines from the caches (measured 12% faster on the
// LLaMA-7B-layer decode than ordinary loads).
__device__ __forceinline__ u32x4 load_at(const char *base, uint32_t off, int imm = 0) {
  const char *b = base + imm;
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b + (size_t)off));
}

// Issue the K and V loads of the round starting at token rtok (wave-uniform).
template <bool BS8, int DT, int D, int G, int NT>
__device__ __forceinline__ void load_round(RoundBuf<DT, D, G, NT> &R, const WaveCtx &c, int rtok) {
  using S = DecodeShape<DT, D, G, NT>;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tt = rtok + 16 * t;
    const int local0 = min((tt >> c.bshift) - c.first_blk, 63);
    const int phys0 = __builtin_amdgcn_readlane(c.tabv, local0);
    if (!BS8) {
      // The whole tile lies in one block: scalar base, per-lane constant offsets.
      const int64_t base = (int64_t)phys0 * c.blk_bytes + c.head_off +
                           (int64_t)(tt & ((1 << c.bshift) - 1)) * S::ROWB;
      const char *kb = c.k_cache + base;
      const char *vb = c.v_cache + base;
#pragma unroll
      for (int s = 0; s < S::KS; ++s) R.k[t][s] = load_at(kb, c.koff, s * 64);
#pragma unroll
      for (int i = 0; i < S::VI; ++i)
#pragma unroll
        for (int sg = 0; sg < S::NSEG; ++sg)
          R.v[t][i * S::NSEG + sg] = load_at(vb, c.voff, i * S::TPI * S::ROWB + sg * S::SEGB);
    } else {
      // 8-token blocks: the tile spans two blocks.
      const int phys1 = __builtin_amdgcn_readlane(c.tabv, min(local0 + 1, 63));
      const int64_t base0 = (int64_t)phys0 * c.blk_bytes + c.head_off;
      const int64_t base1 = (int64_t)phys1 * c.blk_bytes + c.head_off;
      const char *kb = c.k_cache + (c.khi ? base1 : base0);
#pragma unroll
      for (int s = 0; s < S::KS; ++s) R.k[t][s] = load_at(kb, c.koff8, s * 64);
#pragma unroll
      for (int i = 0; i < S::VI; ++i) {
        const int first = i * S::TPI;  // tile token of this load's first row
        const char *vb = c.v_cache + (first < 8 ? base0 : base1);
#pragma unroll
        for (int sg = 0; sg < S::NSEG; ++sg)
          R.v[t][i * S::NSEG + sg] = load_at(vb, c.voff, (first & 7) * S::ROWB + sg * S::SEGB);
      }
    }
  }
}

// Online-softmax state of one lane: its own head's running max and sum for its
// token group, and the weighted V sums of every head for its row chunk(s).
template <int DT, int D, int G, int NT> struct SoftState {
  using S = DecodeShape<DT, D, G, NT>;
  float m;
  float l;
  float acc[G][S::NSEG][S::EPC];
};

// The row of the token written in this decode step, staged in LDS.
struct NewRow {
  int pos;            // its position in the sequence, or -1 when the chunk holds none
  const u32x4 *k;     // 16-byte chunks of its K row (this KV head)
  const u32x4 *v;
};

// Decode step: the position written this step takes its K/V from the staged
// copy of the new row instead of the pool (another workgroup may be writing
// that pool row right now). Only a chunk's last round can hold it.
template <int DT, int D, int G, int NT>
__device__ __forceinline__ void apply_new_row(RoundBuf<DT, D, G, NT> &R, const NewRow &nr,
                                              int rtok) {
  using S = DecodeShape<DT, D, G, NT>;
  if (nr.pos < rtok || nr.pos >= rtok + S::ROUND) return;
  const int lane = __lane_id();
  const int ktok = tile_token_of_row<S::LPT>(lane & 15);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (rtok + 16 * t + ktok == nr.pos) {
#pragma unroll
      for (int s = 0; s < S::KS; ++s) R.k[t][s] = nr.k[(lane >> 4) + 4 * s];
    }
#pragma unroll
    for (int i = 0; i < S::VI; ++i) {
      if (rtok + 16 * t + i * S::TPI + lane / S::LPT == nr.pos) {
#pragma unroll
        for (int sg = 0; sg < S::NSEG; ++sg)
          R.v[t][i * S::NSEG + sg] = nr.v[sg * (S::SEGB / 16) + lane % S::LPT];
      }
    }
  }
}

template <bool MASK, int DT, int D, int G, int NT>
__device__ __forceinline__ void consume_round(const RoundBuf<DT, D, G, NT> &R,
                                              SoftState<DT, D, G, NT> &st, const u32x4 (*qb)[D * 4 / 16],
                                              float scale_log2, int rtok, int p_end) {
  using S = DecodeShape<DT, D, G, NT>;
  const int lane = __lane_id();
  const bool odd8 = (lane & 15) >= 8;          // LPT 8: second token group of the row
  const int vtok = lane / S::LPT;              // token of this lane inside a V load

  // Scores of this lane's own head for the tokens of its V loads.
  float x[NT][S::VI];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s) a = mfma_chunk<DT>(R.k[t][s], qb[(lane & 15) % G][(lane >> 4) + 4 * s], a);
#pragma unroll
    for (int i = 0; i < S::VI; ++i) {
      float v;
      if (S::LPT == 16) v = a[i];
      else v = odd8 ? a[2 * i + 1] : a[2 * i];
      v *= scale_log2;
      if (MASK) {
        const int tok = rtok + 16 * t + i * S::TPI + vtok;
        v = tok < p_end ? v : -INFINITY;
      }
      x[t][i] = v;
    }
  }

  // Lazy rescale: the reference maximum st.m is raised only when some lane's
  // round maximum exceeds it by more than 2^8 (log2 domain), a wave-uniform
  // branch that is rarely taken after the first round. Weights are then at
  // most 2^8, and the sums and accumulators stay relative to one reference,
  // so the result is the same softmax; the usual every-round rescale of the
  // accumulators is skipped.
  float mx = x[0][0];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < S::VI; ++i) mx = fmaxf(mx, x[t][i]);
  if (__builtin_amdgcn_ballot_w64(mx > st.m + 8.0f) != 0) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = st.m == -INFINITY ? 0.0f : fast_exp2(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = from_head<G>(alpha, h);
#pragma unroll
      for (int sg = 0; sg < S::NSEG; ++sg)
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) st.acc[h][sg][e] *= ah;
    }
  }
  const float m_ref = st.m == -INFINITY ? 0.0f : st.m;
  float psum = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < S::VI; ++i) {
      x[t][i] = fast_exp2(x[t][i] - m_ref);
      psum += x[t][i];
    }
  st.l += psum;

#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < S::VI; ++i) {
      bool valid = true;
      if (MASK) valid = rtok + 16 * t + i * S::TPI + vtok < p_end;
      float vf[S::NSEG][S::EPC];
#pragma unroll
      for (int sg = 0; sg < S::NSEG; ++sg)
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) {
          const float f = chunk_elem<DT>(R.v[t][i * S::NSEG + sg], e);
          vf[sg][e] = (MASK && !valid) ? 0.0f : f;
        }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = from_head<G>(x[t][i], h);
#pragma unroll
        for (int sg = 0; sg < S::NSEG; ++sg)
#pragma unroll
          for (int e = 0; e < S::EPC; ++e) st.acc[h][sg][e] = fmaf(ph, vf[sg][e], st.acc[h][sg][e]);
      }
    }
  }
}

// WG-shared buffers of the epilogue (the waves' merged partial results).
template <int G, int D> struct MergeLds {
  float acc[kWaves][G][D];
  float m[kWaves][G];
  float l[kWaves][G];
  u32x4 q[G][D * 4 / 16];  // the group's query rows in 16-byte chunks (room for f32 rows)
  u32x4 newk[D * 4 / 16];  // decode step: this KV head's row of the token written this step
  u32x4 newv[D * 4 / 16];
  int new_slot;            // decode step: the slot that row is written to
};

// Tiles of a wave's chunk inside one window: at most 64 blocks of table.
template <bool BS8> constexpr int chunk_tiles() { return BS8 ? 32 : 63; }

// Per-lane K/V addressing constants of one KV head.
template <int DT, int D, int G, int NT>
__device__ __forceinline__ WaveCtx make_wave_ctx(const DecodeParams &p, int kh) {
  using S = DecodeShape<DT, D, G, NT>;
  const int lane = __lane_id();
  WaveCtx c;
  c.k_cache = reinterpret_cast<const char *>(p.k_cache);
  c.v_cache = reinterpret_cast<const char *>(p.v_cache);
  c.bshift = p.block_shift;
  c.blk_bytes = (int64_t)p.num_kv_heads * (S::ROWB << c.bshift);
  c.head_off = (int64_t)kh * (S::ROWB << c.bshift);
  const int ktok = tile_token_of_row<S::LPT>(lane & 15);
  c.koff = ktok * S::ROWB + (lane >> 4) * 16;
  c.koff8 = (ktok & 7) * S::ROWB + (lane >> 4) * 16;
  c.khi = ktok >= 8;
  c.voff = (lane / S::LPT) * S::ROWB + (lane % S::LPT) * 16;
  return c;
}

// The nr rounds of one chunk [tok0, tok_end) of a wave (its table entries are
// in c.tabv), through two register buffers: at the top of the loop only A
// (round r) is in flight.
// With PRELOADED, round 0 is already in flight in A (issued before the
// segment's query staging).
template <bool BS8, bool PRELOADED, int DT, int D, int G, int NT>
__device__ __forceinline__ void stream_rounds(const WaveCtx &c, SoftState<DT, D, G, NT> &st,
                                              const u32x4 (*qb)[D * 4 / 16], const NewRow &new_row,
                                              float sl2, int tok0, int tok_end, int nr,
                                              RoundBuf<DT, D, G, NT> &A) {
  using S = DecodeShape<DT, D, G, NT>;
  auto rtok_of = [&](int r) { return tok0 + r * S::ROUND; };
  RoundBuf<DT, D, G, NT> B;
  if (!PRELOADED) load_round<BS8>(A, c, rtok_of(0));
  int r = 0;
  while (r + 2 < nr) {
    load_round<BS8>(B, c, rtok_of(r + 1));
    __builtin_amdgcn_sched_barrier(0);
    consume_round<false>(A, st, qb, sl2, rtok_of(r), tok_end);
    load_round<BS8>(A, c, rtok_of(r + 2));
    __builtin_amdgcn_sched_barrier(0);
    consume_round<false>(B, st, qb, sl2, rtok_of(r + 1), tok_end);
    r += 2;
  }
  // Rounds r and (if it exists) r + 1 remain; only the chunk's last round can be partial.
  if (r + 1 < nr) {
    load_round<BS8>(B, c, rtok_of(r + 1));
    __builtin_amdgcn_sched_barrier(0);
    consume_round<false>(A, st, qb, sl2, rtok_of(r), tok_end);
    if (new_row.pos >= 0) apply_new_row(B, new_row, rtok_of(r + 1));
    consume_round<true>(B, st, qb, sl2, rtok_of(r + 1), tok_end);
  } else {
    if (new_row.pos >= 0) apply_new_row(A, new_row, rtok_of(r));
    consume_round<true>(A, st, qb, sl2, rtok_of(r), tok_end);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave: within each 16-lane row
// by DPP row shifts (row_shr 1, 2, 4, 8; lanes with no source lane in the row
// add 0), then each row adds the totals of the rows before it (lanes 15, 31,
// 47, read as scalars). No LDS crossbar round trips.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int lane = __lane_id();
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Sum / maximum of v over lanes l and l ^ mask (mask 8, 16 or 32), in every
// lane. 16 and 32 go through gfx950's row-swap permutes (v_permlane16_swap:
// odd 16-lane rows of one operand with even rows of the other; v_permlane32_swap:
// the upper 32 lanes of one with the lower 32 of the other), so each step is
// two VALU operations instead of an LDS crossbar round trip; the two operands
// then hold the pair's two values in every lane. Addition is commutative, so
// every lane gets the same bits, and the pairs are those of a butterfly.
template <bool MAX>
__device__ __forceinline__ float xor_reduce(float v, int mask) {
  if (mask == 16 || mask == 32) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = mask == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                              : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    const float a = __builtin_bit_cast(float, r0), b = __builtin_bit_cast(float, r1);
    return MAX ? fmaxf(a, b) : a + b;
  }
  const float o = __shfl_xor(v, mask);
  return MAX ? fmaxf(v, o) : v + o;
}

// Merge the token groups of the wave (lanes l, l ^ LPT, l ^ 2 LPT, ... hold the
// same row chunk for different tokens). Afterwards every lane holds each
// head's wave maximum mw and sum lw, and lanes l < LPT the head's merged
// weighted sums of row chunk l (relative to mw) in st.acc.
template <int DT, int D, int G, int NT>
__device__ __forceinline__ void merge_token_groups(SoftState<DT, D, G, NT> &st, float (&mw)[G],
                                                   float (&lw)[G]) {
  using S = DecodeShape<DT, D, G, NT>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mg = from_head<G>(st.m, h);
    float m = mg;
#pragma unroll
    for (int mask = S::LPT; mask < kWave; mask <<= 1) m = xor_reduce<true>(m, mask);
    const float f = m == -INFINITY ? 0.0f : fast_exp2(mg - m);
    float l = from_head<G>(st.l, h) * f;
#pragma unroll
    for (int mask = S::LPT; mask < kWave; mask <<= 1) l = xor_reduce<false>(l, mask);
#pragma unroll
    for (int sg = 0; sg < S::NSEG; ++sg)
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) {
        float a = st.acc[h][sg][e] * f;
#pragma unroll
        for (int mask = S::LPT; mask < kWave; mask <<= 1) a = xor_reduce<false>(a, mask);
        st.acc[h][sg][e] = a;
      }
    mw[h] = m;
    lw[h] = l;
  }
}

// Partials shared between workgroups are written and read at agent scope:
// written through to the device-coherent level and read from it, never from a
// stale per-XCD L2 line.
__device__ __forceinline__ void publish(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A split piece of a workgroup's range whose partials are published and whose
// arrival is not yet counted (item -1: none).
struct PendingPiece {
  int item, first, last;
};

// The last piece of a split (sequence, KV head) to arrive combines the
// partials of pieces first..last (slots item + j) in one pass with a running
// maximum, a batch of pieces at a time. Every output element a thread owns
// (G * D / 256 of them, or one) is handled in the same batch, so all of its
// requests are in flight together: the partials are read at agent scope, and
// each round trip from there costs microseconds while the memory system is
// busy.
template <int DT, int G, int D>
__device__ __forceinline__ void combine_pieces(const DecodeParams &p, typename Store<DT>::T *out,
                                               int item, int first, int last) {
  constexpr int E = (G * D + kThreads - 1) / kThreads;  // elements per thread
  constexpr int PB = E >= 4 ? 2 : E == 2 ? 4 : 8;        // pieces per batch: 24 requests a thread
  int tid = threadIdx.x;
  // Opaque to the optimiser, so these addresses are formed here rather than
  // hoisted out of the segment loop and kept (or spilled) across it.
  asm volatile("" : "+v"(tid));
  float mrun[E], num[E], den[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    mrun[e] = -INFINITY;
    num[e] = 0.0f;
    den[e] = 0.0f;
  }
  for (int j0 = first; j0 <= last; j0 += PB) {
    float mj[E][PB], lj[E][PB], aj[E][PB];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = min(tid + e * kThreads, G * D - 1);
      const int h = idx / D, d = idx % D;
#pragma unroll
      for (int u = 0; u < PB; ++u) {  // `last` is uniform: no request past the last piece
        const int64_t sl = (int64_t)item + j0 + u;
        const bool have = j0 + u <= last;
        mj[e][u] = have ? fetch(p.ws_m + sl * G + h) : -INFINITY;
        lj[e][u] = have ? fetch(p.ws_l + sl * G + h) : 0.0f;
        aj[e][u] = have ? fetch(p.ws_acc + (sl * G + h) * D + d) : 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float mnew = mrun[e];
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (j0 + u <= last) mnew = fmaxf(mnew, mj[e][u]);
      const float sc = mrun[e] == -INFINITY ? 0.0f : fast_exp2(mrun[e] - mnew);
      num[e] *= sc;
      den[e] *= sc;
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        if (j0 + u > last) continue;
        const float f = fast_exp2(mj[e][u] - mnew);
        num[e] = fmaf(f, aj[e][u], num[e]);
        den[e] = fmaf(f, lj[e][u], den[e]);
      }
      mrun[e] = mnew;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = tid + e * kThreads;
    if (idx < G * D) {
      const int h = idx / D, d = idx % D;
      out[((int64_t)item * G + h) * D + d] = Store<DT>::cvt(num[e] / den[e]);
    }
  }
}

// A segment [p_start, p_end) of sequence `seq`, KV head `kh`, processed by the
// four waves. The segment is cut into windows of up to 4 * chunk_tiles tiles;
// each wave takes a contiguous quarter of a window (a chunk that touches at
// most 64 table entries), and runs its rounds of NT tiles through the
// double-buffered loop. Leaves each wave's merged (max, sum, weighted values)
// per head in LDS; the caller synchronises the workgroup before reading them.
template <int DT, int D, int G, int NT, bool BS8>
__device__ __forceinline__ void run_segment(const DecodeParams &p, int seq, int kh, int p_start,
                                            int p_end, int wave, MergeLds<G, D> &lds,
                                            int new_pos, int new_slot, PendingPiece &pend,
                                            int *s_pend_last) {
  using S = DecodeShape<DT, D, G, NT>;
  const int lane = __lane_id();
  const int num_q_heads = p.num_kv_heads * G;
  const int32_t *table_row = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;

  WaveCtx c = make_wave_ctx<DT, D, G, NT>(p, kh);

  const int seg_tiles = (p_end - p_start + 15) >> 4;
  constexpr int kWin = kWaves * chunk_tiles<BS8>();

  // Start-up of a segment: the group's query rows (MFMA operand B, lane l:
  // query head (l % 16) % G, chunk (l / 16) + 4 s, read from LDS), for the
  // decode step this KV head's new row, and the table entries of this wave's
  // part of the first window are requested together. The rows go to LDS as
  // they arrive; once the table entries are in, the first round of K/V loads
  // is issued, and only then does the workgroup synchronise, so the first K/V
  // bytes are on their way during the barrier. (The rows are written before
  // the round is issued so that their registers are free by then.)
  int w_t0, w_t1, tok0, tok_end;
  {
    const int win = min(kWin, seg_tiles);
    w_t0 = wave * win / kWaves;
    w_t1 = (wave + 1) * win / kWaves;
    tok0 = p_start + 16 * w_t0;
    tok_end = min(p_start + 16 * w_t1, p_end);
  }
  const int tid = threadIdx.x;
  constexpr int kQChunks = G * (S::ROWB / 16);  // <= 256: one per thread
  static_assert(kQChunks <= kThreads, "one query chunk per thread");
  {
    u32x4 qv = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
    const char *qrow0 = reinterpret_cast<const char *>(p.q) + ((int64_t)seq * num_q_heads + kh * G) * S::ROWB;
    if (tid < kQChunks) qv = load_chunk(qrow0, (int64_t)(tid / (S::ROWB / 16)) * S::ROWB + (tid % (S::ROWB / 16)) * 16);
    const bool new_thread = new_pos >= 0 && tid < 2 * (S::ROWB / 16);
    const int ch = tid % (S::ROWB / 16);
    if (new_thread) {  // decode step: the new row
      const int64_t src = ((int64_t)seq * p.num_kv_heads + kh) * S::ROWB + ch * 16;
      nv = load_chunk(tid < S::ROWB / 16 ? p.new_key : p.new_value, src);
    }
    c.first_blk = tok0 >> c.bshift;
    c.tabv = table_row[min(c.first_blk + lane, p.max_blocks_per_seq - 1)];
    if (tid < kQChunks) lds.q[tid / (S::ROWB / 16)][tid % (S::ROWB / 16)] = qv;
    if (new_thread) {
      if (tid < S::ROWB / 16) lds.newk[ch] = nv;
      else lds.newv[ch] = nv;
      if (tid == 0) lds.new_slot = new_slot;
    }
  }
  // The previous split piece of this range, published but not yet counted:
  // its partials were stored before this segment's first loads, so once those
  // have returned (and every thread has waited for its own) the piece is
  // counted in, while this segment's first K/V round is requested; the count's
  // round trip and the stores' completion overlap this segment's start.
  const bool counting = pend.item >= 0;
  if (counting) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  c.tabv = min(max(c.tabv, 0), p.num_blocks - 1);  // never address outside the pool
  int arrived = 0;
  if (counting && tid == 0)
    arrived = __hip_atomic_fetch_add(p.ws_count + pend.item, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  RoundBuf<DT, D, G, NT> A;
  const bool first_issued = w_t0 < w_t1;
  if (first_issued) load_round<BS8>(A, c, tok0);
  if (counting && tid == 0) *s_pend_last = arrived == pend.last - pend.first;
  __syncthreads();
  if (counting) {
    if (*s_pend_last) {
      combine_pieces<DT, G, D>(p, reinterpret_cast<typename Store<DT>::T *>(p.out), pend.item,
                               pend.first, pend.last);
      if (tid == 0)  // leave the counter zero for the next call
        __hip_atomic_store(p.ws_count + pend.item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    pend.item = -1;
  }
  // Decode step: the sequence's last attended position takes the staged row
  // only if this step writes that position's slot (the row may go to a fresh
  // block outside the context instead, where nothing in this launch reads it).
  // The check is made per chunk, from its table entries, with scalar values.
  auto new_pos_in = [&](int t_begin, int t_end) -> int {
    if (new_pos < t_begin || new_pos >= t_end) return -1;
    const int phys = __builtin_amdgcn_readlane(c.tabv, (new_pos >> c.bshift) - c.first_blk);
    const int slot = (phys << c.bshift) + (new_pos & ((1 << c.bshift) - 1));
    return slot == __builtin_amdgcn_readfirstlane(lds.new_slot) ? new_pos : -1;
  };
  NewRow new_row{new_pos_in(tok0, tok_end), lds.newk, lds.newv};
  const u32x4 (*qb)[D * 4 / 16] = lds.q;

  SoftState<DT, D, G, NT> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int sg = 0; sg < S::NSEG; ++sg)
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) st.acc[h][sg][e] = 0.0f;

  const float sl2 = p.scale_log2;
  if (first_issued)
    stream_rounds<BS8, true>(c, st, qb, new_row, sl2, tok0, tok_end,
                             (w_t1 - w_t0 + NT - 1) / NT, A);
  for (int w0 = kWin; w0 < seg_tiles; w0 += kWin) {
    const int win = min(kWin, seg_tiles - w0);
    const int t0 = w0 + wave * win / kWaves;
    const int t1 = w0 + (wave + 1) * win / kWaves;
    if (t0 >= t1) continue;
    const int wtok0 = p_start + 16 * t0;
    const int wtok_end = min(p_start + 16 * t1, p_end);
    c.first_blk = wtok0 >> c.bshift;
    c.tabv = min(max(table_row[min(c.first_blk + lane, p.max_blocks_per_seq - 1)], 0),
                 p.num_blocks - 1);
    new_row.pos = new_pos_in(wtok0, wtok_end);
    stream_rounds<BS8, false>(c, st, qb, new_row, sl2, wtok0, wtok_end, (t1 - t0 + NT - 1) / NT, A);
  }

  float mw[G], lw[G];
  merge_token_groups(st, mw, lw);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane < S::LPT) {
#pragma unroll
      for (int sg = 0; sg < S::NSEG; ++sg)
#pragma unroll
        for (int e = 0; e < S::EPC; ++e)
          lds.acc[wave][h][sg * (S::SEGB / S::E) + lane * S::EPC + e] = st.acc[h][sg][e];
    }
    if (lane == 0) {
      lds.m[wave][h] = mw[h];
      lds.l[wave][h] = lw[h];
    }
  }
}

// The workgroup's combined (max, numerator, denominator) of element (h, d).
template <int G, int D>
__device__ __forceinline__ void wg_combine(const MergeLds<G, D> &lds, int h, int d, float &mmax,
                                           float &num, float &den) {
  mmax = lds.m[0][h];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mmax = fmaxf(mmax, lds.m[w][h]);
  num = 0.0f;
  den = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = lds.m[w][h] == -INFINITY ? 0.0f : fast_exp2(lds.m[w][h] - mmax);
    num = fmaf(f, lds.acc[w][h][d], num);
    den = fmaf(f, lds.l[w][h], den);
  }
}

// ---------------------------------------------------------------------------
// Fixed partitions: one workgroup per (partition, KV head, sequence).
// ---------------------------------------------------------------------------

template <int DT, int D, int G, int NT, bool BS8>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeParams p) {
  using OutT = typename Store<DT>::T;
  __shared__ MergeLds<G, D> lds;

  const int part = blockIdx.x;
  const int kh = blockIdx.y;
  const int seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int num_q_heads = p.num_kv_heads * G;
  const int p_start = part * p.partition_size;
  OutT *out = reinterpret_cast<OutT *>(p.out);
  const int n = min(p.context_lens[seq], p.max_context_len);

  if (n <= 0) {  // empty context: zero output rows
    if (part == 0)
      for (int i = tid; i < G * D; i += kThreads)
        out[((int64_t)seq * num_q_heads + kh * G) * D + i] = Store<DT>::cvt(0.0f);
    return;
  }
  if (p_start >= n) return;
  const int p_end = min(p_start + p.partition_size, n);
  PendingPiece none{-1, 0, 0};
  run_segment<DT, D, G, NT, BS8>(p, seq, kh, p_start, p_end, wave, lds, -1, -1, none, nullptr);
  __syncthreads();

  const bool single = n <= p.partition_size;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float mmax, num, den;
    wg_combine(lds, h, d, mmax, num, den);
    const int64_t row = (int64_t)seq * num_q_heads + kh * G + h;
    if (single) {
      out[row * D + d] = Store<DT>::cvt(num / den);
    } else {
      const int64_t slot = row * p.max_partitions + part;
      p.ws_acc[slot * D + d] = num;
      if (d == 0) {
        p.ws_m[slot] = mmax;
        p.ws_l[slot] = den;
      }
    }
  }
}

// Log-sum-exp combine of a sequence's partitions: one workgroup per
// (query head, sequence), one thread per dim.
template <int DT, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeParams p) {
  using OutT = typename Store<DT>::T;
  const int hq = blockIdx.x;
  const int seq = blockIdx.y;
  const int d = threadIdx.x;
  const int n = min(p.context_lens[seq], p.max_context_len);
  if (n <= p.partition_size) return;
  const int np = (n + p.partition_size - 1) / p.partition_size;
  const int num_q_heads = p.num_kv_heads * p.group;
  const int64_t base = ((int64_t)seq * num_q_heads + hq) * p.max_partitions;
  float mmax = -INFINITY;
  for (int i = 0; i < np; ++i) mmax = fmaxf(mmax, p.ws_m[base + i]);
  float num = 0.0f, den = 0.0f;
  for (int i = 0; i < np; ++i) {
    const float f = fast_exp2(p.ws_m[base + i] - mmax);
    num = fmaf(f, p.ws_acc[(base + i) * D + d], num);
    den = fmaf(f, p.ws_l[base + i], den);
  }
  reinterpret_cast<OutT *>(p.out)[((int64_t)seq * num_q_heads + hq) * D + d] = Store<DT>::cvt(num / den);
}

// ---------------------------------------------------------------------------
// Balanced schedule: the (sequence, KV head, 16-token tile) space, flattened in
// that order with a fixed overhead charge in front of each (sequence, KV head),
// is cut into equal ranges of `sz` units, one per workgroup. A workgroup walks
// its range as segments (the part of one (sequence, KV head) inside the range).
// A segment that is a whole (sequence, KV head) writes its output rows; the
// pieces of a split one leave partials in the workspace and the last
// workgroup to finish a piece combines them (log-sum-exp), so one launch does
// the whole decode and every workgroup gets the same work (tiles plus segment
// overheads) whatever the mix of context lengths. Unit positions fit in int32:
// the host takes this form only when an upper bound of the units does.
// ---------------------------------------------------------------------------


__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The equal cut of `total` units over `nwg` ranges with 32-bit arithmetic (a
// 64-bit division is a long instruction sequence here, on every workgroup's
// start-up path): with total = q nwg + r, floor(w total / nwg) = w q +
// floor(w r / nwg), and w r < nwg^2 fits.
__device__ __forceinline__ int cut_lo(int w, int total, int nwg) {
  const int q = total / nwg;
  const int r = total - q * nwg;
  return w * q + (w * r) / nwg;
}

// Coordinates of the segment of a range [.., end) that starts at unit pos,
// inside sequence seq: KV head kh, its tiles [a, b) (b <= a: the range ends in
// the item's overhead units), the item's tile count and first tile unit. All
// wave-uniform; read from the plan in LDS, so the caller can re-derive them
// after the streaming loop instead of keeping them in registers across it.
struct SegCoords {
  int kh, a, b, tiles, tile_base;
};

__device__ __forceinline__ SegCoords seg_coords(const int *s_tc, int seq, int hkv, int cost,
                                                int pos, int end) {
  SegCoords c;
  const int tc0 = uniform_i32(s_tc[seq]);
  const int units = uniform_i32(s_tc[seq + 1]) - tc0;
  c.tiles = units - cost;
  const int seq_base = hkv * tc0;
  c.kh = (pos - seq_base) / units;
  c.tile_base = seq_base + c.kh * units + cost;  // the item's overhead units, then its tiles
  c.a = max(pos - c.tile_base, 0);
  c.b = min(end - c.tile_base, c.tiles);
  return c;
}

// Decode step: this step's K/V rows go into the pools one (sequence, KV head)
// pair per workgroup in turn (pair i by workgroup i mod grid). Nothing in the
// launch reads them back from the pools: the attention takes them from LDS
// (see consume_round). A workgroup loads its first pair at the start, next to
// the plan's loads, and stores it once the plan is done; further pairs (more
// pairs than workgroups) are copied after its attention work. The slot is
// range-checked at the store, so both loads are in flight together.
template <int DT, int D, int G> struct NewRowCopy {
  static constexpr int kChunks = DecodeShape<DT, D, G, 1>::ROWB / 16;
  u32x4 data;
  int slot = -1;

  __device__ __forceinline__ void load(const DecodeParams &p, int pair) {
    const int tid = threadIdx.x;
    if (pair < p.num_seqs * p.num_kv_heads && tid < 2 * kChunks) {
      slot = p.slot_mapping[pair / p.num_kv_heads];
      const int64_t src = ((int64_t)pair * kChunks + tid % kChunks) * 16;
      data = load_chunk(tid < kChunks ? p.new_key : p.new_value, src);
    }
  }
  __device__ __forceinline__ void store(const DecodeParams &p, int pair) const {
    const int tid = threadIdx.x;
    if (slot < 0 || slot >= p.num_slots) return;  // negative: skip; too large: never write outside
    const int kh = pair % p.num_kv_heads;
    const int bshift = p.block_shift;
    const int64_t row = (((int64_t)(slot >> bshift) * p.num_kv_heads + kh) << bshift) +
                        (slot & ((1 << bshift) - 1));
    const int64_t dst = (row * kChunks + tid % kChunks) * 16;
    store_chunk(tid < kChunks ? p.k_cache_w : p.v_cache_w, dst, data);
  }
};

// Pairs first, first + grid, ... (the ones past a workgroup's first).
template <int DT, int D, int G>
__device__ __forceinline__ void copy_new_rows(const DecodeParams &p, int first) {
  for (int pair = first; pair < p.num_seqs * p.num_kv_heads; pair += gridDim.x) {
    NewRowCopy<DT, D, G> row;
    row.load(p, pair);
    row.store(p, pair);
  }
}

// MIN_WAVES: the minimum waves per SIMD the register allocation must allow
// (1: no constraint).
template <int DT, int D, int G, int NT, bool BS8, bool STEP, int MIN_WAVES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MIN_WAVES)))
void decode_flat_kernel(DecodeParams p) {
  using OutT = typename Store<DT>::T;
  extern __shared__ int s_plan[];  // tiles prefix [S + 1], clamped lengths [S], slots [S]
  __shared__ MergeLds<G, D> lds;
  __shared__ int s_wsum[kWaves];
  __shared__ int s_last;
  __shared__ int s_pend_last;
  __shared__ int s_found;

  const int S = p.num_seqs;
  const int hkv = p.num_kv_heads;
  const int num_q_heads = hkv * G;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  int *s_tc = s_plan;
  int *s_n = s_plan + S + 1;
  int *s_slot = s_n + S;  // decode step: this step's slot per sequence (-1: none)
  OutT *out = reinterpret_cast<OutT *>(p.out);

  NewRowCopy<DT, D, G> first_row;
  if (STEP) first_row.load(p, w);

  // Plan: work units per sequence and their prefix sums (every workgroup
  // computes the same plan from context_lens). A (sequence, KV head) of t tiles
  // is `cost` units of overhead followed by its t tiles, so cutting the units
  // evenly gives a workgroup whose range touches more (sequence, KV head)
  // pairs fewer tiles: each segment costs a start-up and an epilogue.
  const int cost = p.seg_cost;
  if (tid == 0) s_tc[0] = 0;
  int carry = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    int n = s < S ? min(p.context_lens[s], p.max_context_len) : 0;
    // requested with the length, not after the scan's barrier (which would add
    // a memory round trip to every workgroup's start)
    const int slot = STEP && s < S ? p.slot_mapping[s] : -1;
    n = max(n, 0);
    int x = (n + 15) >> 4;
    if (x > 0) x += cost;  // each (sequence, KV head) is charged `cost` tiles more
    x = wave_inclusive_scan(x);
    if (lane == kWave - 1) s_wsum[wave] = x;
    __syncthreads();
    int off = carry, total = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      off += v < wave ? s_wsum[v] : 0;
      total += s_wsum[v];
    }
    if (s < S) {
      s_tc[s + 1] = off + x;
      s_n[s] = n;
      s_slot[s] = slot >= 0 && slot < p.num_slots ? slot : -1;
    }
    carry += total;
    __syncthreads();
  }
  const int total = hkv * carry;  // < 2^31 (checked on the host)

  if (STEP) first_row.store(p, w);

  // Empty contexts: zero output rows, spread over the workgroups.
  for (int s = w; s < S; s += gridDim.x)
    if (s_n[s] == 0)
      for (int i = tid; i < num_q_heads * D; i += kThreads)
        out[(int64_t)s * num_q_heads * D + i] = Store<DT>::cvt(0.0f);

  // Workgroup w takes units [floor(w T / nwg), floor((w + 1) T / nwg)); with
  // fewer units than workgroups only the first `total` take part, so every
  // range is non-empty (the piece count of the combine counts on that). The
  // range holding unit x is floor(((x + 1) nwg - 1) / T).
  const int nwg = min((int)gridDim.x, total);
  if (w >= nwg) {
    if (STEP) copy_new_rows<DT, D, G>(p, w + gridDim.x);
    return;
  }
  const int start = cut_lo(w, total, nwg);
  const int end = cut_lo(w + 1, total, nwg);
  for (int s = tid; s < S; s += kThreads)
    if (hkv * s_tc[s] <= start && start < hkv * s_tc[s + 1]) s_found = s;
  __syncthreads();
  int seq = uniform_i32(s_found);

  PendingPiece pend{-1, 0, 0};
  int pos = start;
  while (pos < end) {
    while (pos >= hkv * s_tc[seq + 1]) ++seq;  // skips empty sequences
    {
      const SegCoords c = seg_coords(s_tc, seq, hkv, cost, pos, end);
      if (c.b <= c.a) break;  // the range ends inside this pair's overhead units
      const int n = s_n[seq];
      // decode step: the last attended position, when this segment ends the
      // item (its staged row replaces the pool's if the step writes that slot)
      int new_pos = -1;
      if (STEP && c.b == c.tiles && s_slot[seq] >= 0) new_pos = n - 1;
      run_segment<DT, D, G, NT, BS8>(p, seq, c.kh, 16 * c.a, min(16 * c.b, n), wave, lds,
                                     new_pos, s_slot[seq], pend, &s_pend_last);
    }
    __syncthreads();
    const SegCoords c = seg_coords(s_tc, seq, hkv, cost, pos, end);
    const int kh = c.kh, a = c.a, b = c.b, tiles = c.tiles, tile_base = c.tile_base;

    const bool whole = a == 0 && b == tiles;
    const int item = seq * hkv + kh;
    const int first_w = (int)(((int64_t)(tile_base + 1) * nwg - 1) / total);
    const int64_t slot = (int64_t)item + w;  // distinct for every (item, workgroup) pair
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int h = idx / D;
      const int d = idx % D;
      float mmax, num, den;
      wg_combine(lds, h, d, mmax, num, den);
      if (whole) {
        out[((int64_t)item * G + h) * D + d] = Store<DT>::cvt(num / den);
      } else {
        publish(p.ws_acc + (slot * G + h) * D + d, num);
        if (d == 0) {
          publish(p.ws_m + slot * G + h, mmax);
          publish(p.ws_l + slot * G + h, den);
        }
      }
    }
    if (!whole) {
      // Counted in at the start of the range's next segment (see run_segment),
      // or below when no segment follows. The item's last workgroup to arrive
      // combines. The partials were written through to the device-coherent
      // level (agent scope) and every thread waits for its writes to complete
      // before the arrival is counted, so the last arriver, reading them back
      // at agent scope, sees all of them. No L2 write-back or invalidate is
      // needed.
      pend = PendingPiece{item, first_w,
                          (int)(((int64_t)(tile_base + tiles) * nwg - 1) / total)};
    }
    __syncthreads();  // lds and s_last are reused by the next segment
    pos = tile_base + b;
  }
  if (pend.item >= 0) {  // the range's last piece: no segment follows to overlap its count
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(p.ws_count + pend.item, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == pend.last - pend.first;
    __syncthreads();
    if (s_last) {
      combine_pieces<DT, G, D>(p, out, pend.item, pend.first, pend.last);
      if (tid == 0)  // leave the counter zero for the next call
        __hip_atomic_store(p.ws_count + pend.item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (STEP) copy_new_rows<DT, D, G>(p, w + gridDim.x);
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

template <int DT, int D, int G> constexpr int rounds_tiles() {
  return (D * Elem<DT>::kBytes) >= 256 ? 1 : 2;
}

// Register bound of the balanced-form instances (waves per SIMD the
// allocation must allow). Where set, the instance fits with no scratch, while
// unbounded the compiler takes a few registers more and loses a wave per SIMD:
// 16-bit head_dim 128 with one query head per KV head fits 128 VGPRs (4 waves),
// with two or four 168 (3 waves); fp16 head_dim 64 with one fits 128, 16-bit
// head_dim 64 with two fits 168. Other instances would spill and stay unbounded.
template <int DT, int D, int G> constexpr int flat_min_waves() {
  if (DT == PA_F32) return 1;
  if (D == 128) return G == 1 ? 4 : G <= 4 ? 3 : 1;
  if (D == 64) return (G == 1 && DT == PA_F16) ? 4 : G == 2 ? 3 : 1;
  return 1;
}

template <int DT, int D, int G, bool BS8, bool STEP>
static hipError_t launch_flat(const DecodeParams &p, hipStream_t stream) {
  constexpr int NT = rounds_tiles<DT, D, G>();
  constexpr int kMinWaves = flat_min_waves<DT, D, G>();
  auto kern = decode_flat_kernel<DT, D, G, NT, BS8, STEP, kMinWaves>;
  const size_t shmem = flat_plan_lds_bytes(p.num_seqs);
  const int64_t max_tiles =
      (int64_t)p.num_seqs * p.num_kv_heads * ((p.max_context_len + 15) / 16);
  const int grid = flat_grid_size(reinterpret_cast<const void *>(kern), kThreads, shmem, max_tiles);
  if (grid <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), shmem, stream, p);
  return hipGetLastError();
}

template <int DT, int D, int G>
static hipError_t launch_dtg(const DecodeParams &p, hipStream_t stream, DecodeStage stage) {
  constexpr int NT = rounds_tiles<DT, D, G>();
  const bool bs8 = p.block_shift == 3;
  if (stage == kStageFlat) {
    if (p.slot_mapping != nullptr)
      return bs8 ? launch_flat<DT, D, G, true, true>(p, stream)
                 : launch_flat<DT, D, G, false, true>(p, stream);
    return bs8 ? launch_flat<DT, D, G, true, false>(p, stream)
               : launch_flat<DT, D, G, false, false>(p, stream);
  }
  if (stage != kStageReduce) {
    dim3 grid(p.max_partitions, p.num_kv_heads, p.num_seqs);
    if (bs8)
      hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, NT, true>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, NT, false>), grid, dim3(kThreads), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stage != kStagePartitions && p.max_partitions > 1) {
    dim3 rgrid(p.num_kv_heads * G, p.num_seqs);
    hipLaunchKernelGGL((decode_reduce_kernel<DT, D>), rgrid, dim3(D), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int DT, int D>
static hipError_t launch_dt(const DecodeParams &p, hipStream_t stream, DecodeStage stage) {
  switch (p.group) {
    case 1: return launch_dtg<DT, D, 1>(p, stream, stage);
    case 2: return launch_dtg<DT, D, 2>(p, stream, stage);
    case 4: return launch_dtg<DT, D, 4>(p, stream, stage);
    case 8: return launch_dtg<DT, D, 8>(p, stream, stage);
  }
  return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_d(const DecodeParams &p, hipStream_t stream, DecodeStage stage) {
  switch (p.head_dim) {
    case 64: return launch_dt<DT, 64>(p, stream, stage);
    case 128: return launch_dt<DT, 128>(p, stream, stage);
    case 256:
      if constexpr (DT != PA_F32) return launch_dt<DT, 256>(p, stream, stage);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream, DecodeStage stage) {
  switch (p.dtype) {
    case PA_F32: return launch_d<PA_F32>(p, stream, stage);
    case PA_F16: return launch_d<PA_F16>(p, stream, stage);
    case PA_BF16: return launch_d<PA_BF16>(p, stream, stage);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
