// Device helpers shared by the gfx950 kernels: storage types, bf16
// conversion, 16-byte vector loads and wave64 lane reductions (DPP within a
// row of 16 lanes, ds_bpermute across rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dqkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 is carried as its 16-bit pattern.
typedef uint16_t bf16;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16 h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

template <typename T> struct Elem;

template <> struct Elem<float> {
  static constexpr int kPer16 = 4;  // elements per 16-byte load
  __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
};

template <> struct Elem<bf16> {
  static constexpr int kPer16 = 8;
  __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ float to_f32(bf16 x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ bf16 from_f32(float x) { return f32_to_bf16(x); }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c for two packed bf16 pairs, fp32 accumulate
// (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (lo, hi) rounded to bf16 (nearest, ties to even) and packed, lo in bits 0-15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load: the nontemporal hint tells the caches the line is read
// once, which lets long sequential reads run closer to HBM bandwidth.
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- DPP
// dpp_ctrl encodings (GCN/CDNA): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror (reverse 8 lanes) = 0x141, row_mirror (reverse 16) = 0x140.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64);
// every lane of a group receives the group's sum.  Must be called with all
// lanes of the wave active.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);
  if constexpr (N >= 4) x += dpp<0x4E>(x);
  if constexpr (N >= 8) x += dpp<0x141>(x);
  if constexpr (N >= 16) x += dpp<0x140>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) { return group_max<64>(x); }

// Hardware base-2 exponential / logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace dqkv
