// Device helpers for the gfx950 kernels: element-type traits, packed dot
// products, DPP / cross-lane reductions and round-to-nearest-even stores.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---- 16-bit element types -------------------------------------------------

template <bool BF16>
struct Elem;

template <>
struct Elem<false> {  // IEEE fp16
  static __device__ __forceinline__ float lo(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(half2_t, w)[0]);
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(half2_t, w)[1]);
  }
  // acc + a.lo*b.lo + a.hi*b.hi, fp32 accumulate.
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  acc, false);
  }
  // fp32 -> fp16, round to nearest even (the hardware default rounding mode).
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
};

template <>
struct Elem<true> {  // bfloat16: the upper half of an fp32
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return __uint_as_float(w & 0xffff0000u);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), acc, false);
  }
  // fp32 -> bf16, round to nearest even on the dropped 16 bits; NaN stays NaN.
  static __device__ __forceinline__ uint16_t from_float(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
};

// Sum of the eight products of two 16-byte vectors (8 elements each).
template <bool BF16>
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc) {
  acc = Elem<BF16>::dot2(a.x, b.x, acc);
  acc = Elem<BF16>::dot2(a.y, b.y, acc);
  acc = Elem<BF16>::dot2(a.z, b.z, acc);
  acc = Elem<BF16>::dot2(a.w, b.w, acc);
  return acc;
}

// ---- cross-lane ------------------------------------------------------------

// DPP controls (gfx9): quad permutations, mirrors inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N == 16) x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __int_as_float(
      __builtin_amdgcn_ds_bpermute(((lane ^ mask) & 63) << 2, __float_as_int(x)));
}

// Integer maximum over the wave; every lane gets it.
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1)
    x = max(x, __builtin_amdgcn_ds_bpermute(((__lane_id() ^ sh) & 63) << 2, x));
  return x;
}

// Integer sum over the wave; every lane gets it.
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1)
    x += __builtin_amdgcn_ds_bpermute(((__lane_id() ^ sh) & 63) << 2, x);
  return x;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan_i(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute(((lane - sh) & 63) << 2, x);
    if (lane >= sh) x += y;
  }
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Plain 16-byte global load (one dwordx4).
__device__ __forceinline__ uint4 load16(const void* p) {
  return *static_cast<const uint4*>(p);
}

// Word 3 of a raw buffer descriptor on gfx9 (32-bit data format, no
// swizzle): offsets at or past num_records read as zero without a memory
// access.
constexpr int kBufferFlags = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of a buffer load on gfx950: bit 1 is NT (non-temporal,
// streaming).  KV pages are read exactly once per step, so their loads carry
// NT; on MI355X this raised the read rate of the page stream by 10-13 % over
// the default policy (read-only probe over the same pages, one long row and
// the bimodal batch).
constexpr int kCachePolicyStream = 2;

// One 16-byte KV load through a page's buffer descriptor (streaming policy).
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int offset) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kCachePolicyStream);
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace pkv
