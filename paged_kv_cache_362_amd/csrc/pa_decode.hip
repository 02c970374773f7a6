// pa_decode.hip - decode-phase paged attention kernels for gfx950 (MI355X).
//
// What is computed ([INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理",
// §1.1 and §3.4): for sequence s and query head h, the scores of the new query
// against the first n = context_lens[s] cached keys of KV head h / G, scaled,
// softmax-normalised, and used to average the cached values. The cached rows
// are found through the sequence's block table (§3.3).
//
// How (one workgroup per (context partition, KV head, sequence); split-K and a
// log-sum-exp combine in the manner of flash decoding, [INFRA] Q2 of §8):
//
// * A partition is `partition_size` consecutive tokens of one sequence. Its
//   four waves take rounds of 16*TR tokens in turn. The partition's table
//   entries are staged in LDS once, so every lane finds its token's physical
//   block with one LDS read.
// * Keys: QK^T runs on the matrix cores. For each 16-token tile, MFMA operand B
//   is K^T (column = token, lane l holds 16 contiguous bytes of token l%16),
//   operand A is the group's queries (row = query head, replicated over the
//   four row groups when the group has fewer than four heads). The 16x16
//   result leaves each token's score for every head of the group in the lane
//   that loaded that token, so no cross-lane sum is needed. All G query heads
//   of a KV head share each K tile read ([INFRA] §2.1 GQA).
// * Values: loaded as whole contiguous rows (16 bytes per lane, 64 lanes
//   covering 1 KB), so each lane owns 16 bytes of dims of a few tokens. The
//   softmax weight of each token is fetched from the lane holding its score
//   (ds_bpermute) and accumulated in float32 on the vector ALUs.
// * Softmax is online per round in the log2 domain: the wave keeps the running
//   maximum per head (wave-uniform) and rescales its partial sums when it grows.
// * Tokens past the partition's end or the context are never read from
//   unused slots: their addresses are clamped to the last valid token and
//   their scores set to -inf, so their weights are exactly 0 and poisoned
//   (NaN) pad slots cannot leak into the output.
// * The four waves merge through LDS. A sequence with one partition writes the
//   output directly; otherwise (m, l, acc) of the partition go to the
//   workspace and decode_reduce_kernel combines them.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kTabCache = kMaxPartition / 8 + 8;  // table entries one partition spans

template <int DT, int D, int G> struct DecodeShape {
  static constexpr int E = Elem<DT>::kBytes;
  static constexpr int EPC = Elem<DT>::kPerChunk;  // elements per 16-byte chunk
  static constexpr int CPR = D * E / 16;           // chunks per token row
  static constexpr int CPL = CPR / 4;              // K chunks per lane per tile
  static constexpr int LPT = CPR;                  // V: lanes per token
  static constexpr int TPI = kWave / LPT;          // V: tokens per load instruction
  static constexpr int NVI = 16 / TPI;             // V: load instructions per tile
  static constexpr int GH = G < 4 ? G : 4;         // query heads per MFMA head group
  static constexpr int NHG = (G + 3) / 4;          // MFMA head groups
  static constexpr int TR = CPL >= 8 ? 1 : 8 / CPL;  // tiles per round
  static constexpr int ROUND = 16 * TR;            // tokens per round
  static_assert(CPR >= 4 && CPR <= 64 && (CPR & (CPR - 1)) == 0, "row must be 4..64 chunks");
  static_assert(NVI == CPL, "V instructions per tile equal K chunks per lane");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
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

template <int DT, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeParams p) {
  using S = DecodeShape<DT, D, G>;
  using OutT = typename Store<DT>::T;
  constexpr int E = S::E;

  const int part = blockIdx.x;
  const int kh = blockIdx.y;
  const int seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int num_q_heads = p.num_kv_heads * G;
  const int n = min(p.context_lens[seq], p.max_context_len);
  const int p_start = part * p.partition_size;
  OutT *out = reinterpret_cast<OutT *>(p.out);

  if (n <= 0) {  // empty context: zero output rows
    if (part == 0)
      for (int i = tid; i < G * D; i += kThreads)
        out[((int64_t)seq * num_q_heads + kh * G) * D + i] = Store<DT>::cvt(0.0f);
    return;
  }
  if (p_start >= n) return;
  const int p_end = min(p_start + p.partition_size, n);
  const int bshift = p.block_shift;
  const int bmask = (1 << bshift) - 1;

  // Table entries of this partition -> LDS.
  __shared__ int s_tab[kTabCache];
  const int first_blk = p_start >> bshift;
  const int nblk = ((p_end - 1) >> bshift) - first_blk + 1;
  const int32_t *tab = p.block_tables + (int64_t)seq * p.max_blocks_per_seq + first_blk;
  for (int i = tid; i < nblk; i += kThreads) {
    const int b = tab[i];
    s_tab[i] = min(max(b, 0), p.num_blocks - 1);  // never address outside the pool
  }

  // MFMA operand A: queries of the group, one 16-byte chunk per k-step.
  const int r = lane & 15;  // token column of this lane in K tiles
  const int c = lane >> 4;  // row group (selects the K chunk)
  u32x4 qop[S::NHG][S::CPL];
#pragma unroll
  for (int hg = 0; hg < S::NHG; ++hg) {
    const int head = hg * 4 + ((lane & 3) % S::GH);
    const int64_t qbase = ((int64_t)seq * num_q_heads + kh * G + head) * D * E;
#pragma unroll
    for (int s = 0; s < S::CPL; ++s) qop[hg][s] = load_chunk(p.q, qbase + (c + 4 * s) * 16);
  }

  float m_run[G], l_run[G], acc[G][S::EPC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < S::EPC; ++e) acc[h][e] = 0.0f;
  }

  const int64_t head_stride = (int64_t)1 << bshift;  // rows per (block, head)
  const int vtok = lane / S::LPT;                     // V: token within an instruction
  const int vchunk = lane % S::LPT;                   // V: chunk within the row
  __syncthreads();

  for (int rs = p_start + wave * S::ROUND; rs < p_end; rs += kWaves * S::ROUND) {
    u32x4 kb[S::TR][S::CPL];
    u32x4 vb[S::TR][S::NVI];
#pragma unroll
    for (int j = 0; j < S::TR; ++j) {
      const int tb = rs + 16 * j;
      const int tk = min(tb + r, p_end - 1);
      const int64_t krow =
          ((int64_t)s_tab[(tk >> bshift) - first_blk] * p.num_kv_heads + kh) * head_stride + (tk & bmask);
#pragma unroll
      for (int s = 0; s < S::CPL; ++s) kb[j][s] = load_chunk(p.k_cache, krow * (D * E) + (c + 4 * s) * 16);
#pragma unroll
      for (int i = 0; i < S::NVI; ++i) {
        const int tv = min(tb + i * S::TPI + vtok, p_end - 1);
        const int64_t vrow =
            ((int64_t)s_tab[(tv >> bshift) - first_blk] * p.num_kv_heads + kh) * head_stride + (tv & bmask);
        vb[j][i] = load_chunk(p.v_cache, vrow * (D * E) + vchunk * 16);
      }
    }

    // Scores (log2 domain), masked past the partition end.
    float x[S::TR][G];
#pragma unroll
    for (int j = 0; j < S::TR; ++j) {
      const bool valid = rs + 16 * j + r < p_end;
#pragma unroll
      for (int hg = 0; hg < S::NHG; ++hg) {
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < S::CPL; ++s) a = mfma_chunk<DT>(qop[hg][s], kb[j][s], a);
#pragma unroll
        for (int i = 0; i < S::GH; ++i) {
          const int h = hg * 4 + i;
          if (h < G) x[j][h] = valid ? a[i] * p.scale_log2 : -INFINITY;
        }
      }
    }

    // Online softmax update per head.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = x[0][h];
#pragma unroll
      for (int j = 1; j < S::TR; ++j) mx = fmaxf(mx, x[j][h]);
      mx = uniform_f32(row16_max(mx));
      const float m_new = fmaxf(m_run[h], mx);
      const float alpha = fast_exp2(m_run[h] - m_new);
      m_run[h] = m_new;
      l_run[h] *= alpha;
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int j = 0; j < S::TR; ++j) x[j][h] = fast_exp2(x[j][h] - m_new);
    }

    // P V on the vector ALUs, float32 accumulation.
#pragma unroll
    for (int j = 0; j < S::TR; ++j) {
#pragma unroll
      for (int i = 0; i < S::NVI; ++i) {
        const int src = i * S::TPI + vtok;  // lane (row group 0) holding this token's scores
        float vf[S::EPC];
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) vf[e] = chunk_elem<DT>(vb[j][i], e);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pv = lane_read(x[j][h], src);
          l_run[h] += pv;
#pragma unroll
          for (int e = 0; e < S::EPC; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
        }
      }
    }
  }

  // Sum over the lanes that hold the same dims (different tokens).
#pragma unroll
  for (int mask = S::LPT; mask < kWave; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l_run[h] += lane_xor(l_run[h], mask);
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) acc[h][e] += lane_xor(acc[h][e], mask);
    }
  }

  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  if (lane < S::LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) s_acc[wave][h][lane * S::EPC + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m_run[h];
      s_l[wave][h] = l_run[h];
    }
  }
  __syncthreads();

  const bool single = n <= p.partition_size;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float mmax = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mmax = fmaxf(mmax, s_m[w][h]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][h] - mmax);
      num = fmaf(f, s_acc[w][h][d], num);
      den = fmaf(f, s_l[w][h], den);
    }
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

template <int DT, int D, int G>
static hipError_t launch_dtg(const DecodeParams &p, hipStream_t stream, DecodeStage stage) {
  if (stage != kStageReduce) {
    dim3 grid(p.max_partitions, p.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G>), grid, dim3(kThreads), 0, stream, p);
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
    case 256: return launch_dt<DT, 256>(p, stream, stage);
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
