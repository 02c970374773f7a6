// pa_common.h - device helpers shared by the paged-attention kernels (gfx950).
//
// Internal to libpagedattn.so. Element types, 16-byte chunk access, wave-level
// cross-lane moves (DPP within rows of 16 lanes, ds_bpermute across the wave)
// and float32 -> storage rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Element type traits: bytes per element and elements per 16-byte chunk.
template <int DT> struct Elem;
template <> struct Elem<PA_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
};
template <> struct Elem<PA_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
};
template <> struct Elem<PA_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
};

__device__ __forceinline__ u32x4 load_chunk(const void *base, int64_t byte_off) {
  return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(base) + byte_off);
}

__device__ __forceinline__ void store_chunk(void *base, int64_t byte_off, u32x4 v) {
  *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(base) + byte_off) = v;
}

// Element e of a 16-byte chunk, widened to float32 (exact).
template <int DT> __device__ __forceinline__ float chunk_elem(const u32x4 &c, int e);

// A vector element is copied to a scalar before any bit cast: __builtin_bit_cast
// applied directly to a vector-element lvalue reads element 0 with this compiler.
__device__ __forceinline__ uint32_t chunk_word(const u32x4 &c, int w) {
  const uint32_t v = c[w];
  return v;
}

template <> __device__ __forceinline__ float chunk_elem<PA_F32>(const u32x4 &c, int e) {
  return __builtin_bit_cast(float, chunk_word(c, e));
}
template <> __device__ __forceinline__ float chunk_elem<PA_F16>(const u32x4 &c, int e) {
  const uint32_t w = chunk_word(c, e >> 1);
  const uint16_t h = (e & 1) ? uint16_t(w >> 16) : uint16_t(w & 0xffffu);
  return float(__builtin_bit_cast(_Float16, h));
}
template <> __device__ __forceinline__ float chunk_elem<PA_BF16>(const u32x4 &c, int e) {
  const uint32_t w = chunk_word(c, e >> 1);
  return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// float32 -> storage bits, round to nearest even.
template <int DT> struct Store;
template <> struct Store<PA_F32> {
  using T = float;
  __device__ static T cvt(float x) { return x; }
};
template <> struct Store<PA_F16> {
  using T = _Float16;
  __device__ static T cvt(float x) { return _Float16(x); }
};
template <> struct Store<PA_BF16> {
  using T = uint16_t;
  __device__ static T cvt(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    if ((b & 0x7fffffffu) > 0x7f800000u) return uint16_t(0x7fc0);  // NaN
    return uint16_t((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
  }
};

// DPP moves inside rows of 16 lanes.
enum : int {
  kDppQuadXor1 = 0xB1,   // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,   // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
};

template <int CTRL> __device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum over the 16 lanes of each row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return v;
}

// Value of `v` held by lane `src` (0..63).
__device__ __forceinline__ float lane_read(float v, int src) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float lane_xor(float v, int mask) {
  const int lane = __lane_id();
  return lane_read(v, lane ^ mask);
}

__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
