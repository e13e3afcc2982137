// Device-side helpers shared by the HIP kernels: element types, 16-byte
// vector loads, conversions, packed dot products and cross-lane reductions
// for 64-wide CDNA wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

struct u32x4 {
  uint32_t w[4];
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  u32x4 r;
  r.w[0] = v.x;
  r.w[1] = v.y;
  r.w[2] = v.z;
  r.w[3] = v.w;
  return r;
}

struct u32x2 {
  uint32_t w[2];
};

__device__ __forceinline__ u32x2 load8(const void* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  u32x2 r;
  r.w[0] = v.x;
  r.w[1] = v.y;
  return r;
}

// Streaming (non-temporal) loads: data read exactly once is not kept in the
// caches, which leaves L2 and the Infinity Cache to the data that is reused.
typedef uint32_t u32v4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32v2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  const u32v4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32v4_t*>(p));
  u32x4 r;
  r.w[0] = v[0];
  r.w[1] = v[1];
  r.w[2] = v[2];
  r.w[3] = v[3];
  return r;
}

__device__ __forceinline__ uint32_t load4_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

__device__ __forceinline__ u32x2 load8_stream(const void* p) {
  const u32v2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32v2_t*>(p));
  u32x2 r;
  r.w[0] = v[0];
  r.w[1] = v[1];
  return r;
}

__device__ __forceinline__ void store16(void* p, const u32x4& r) {
  uint4 v;
  v.x = r.w[0];
  v.y = r.w[1];
  v.z = r.w[2];
  v.w = r.w[3];
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// Element types.  `bytes` is the element size; a 32-bit word holds
// 4 / bytes elements; lo()/hi() widen the elements of one word to float.
struct TF32 {
  static constexpr int bytes = 4;
  static constexpr bool is_f16 = false;
  static constexpr bool is_fp8 = false;
  static __device__ __forceinline__ float lo(uint32_t u) { return u2f(u); }
  static __device__ __forceinline__ float store_cvt(float x) { return x; }
};

struct TF16 {
  static constexpr int bytes = 2;
  static constexpr bool is_f16 = true;
  static constexpr bool is_fp8 = false;
  static __device__ __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(half2_t, u).x;
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(half2_t, u).y;
  }
  // sum += a.x*b.x + a.y*b.y with the products and sum in fp32
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                  __builtin_bit_cast(half2_t, b), acc, false);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
  }
};

struct TBF16 {
  static constexpr int bytes = 2;
  static constexpr bool is_f16 = false;
  static constexpr bool is_fp8 = false;
  static __device__ __forceinline__ float lo(uint32_t u) { return u2f(u << 16); }
  static __device__ __forceinline__ float hi(uint32_t u) { return u2f(u & 0xffff0000u); }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), acc, false);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);    // round to nearest even
  }
};

// fp8 cache elements (OCP E4M3 / E5M2).  cvt2<QT, HI>(w) widens the two fp8
// values in bytes 0-1 (HI = false) or 2-3 (HI = true) of w into a packed
// pair of QT (f16 or bf16), low half from the lower byte.  Every E4M3 and
// E5M2 value is exact in f16 and in bf16, so the widening is exact.
struct TFP8E4M3 {
  static constexpr int bytes = 1;
  static constexpr bool is_f16 = false;
  static constexpr bool is_fp8 = true;
  static constexpr bool is_e4m3 = true;
  template <typename QT, bool HI>
  static __device__ __forceinline__ uint32_t cvt2(uint32_t w) {
    if constexpr (QT::is_f16)
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HI));
    else
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
  }
};

struct TFP8E5M2 {
  static constexpr int bytes = 1;
  static constexpr bool is_f16 = false;
  static constexpr bool is_fp8 = true;
  static constexpr bool is_e4m3 = false;
  template <typename QT, bool HI>
  static __device__ __forceinline__ uint32_t cvt2(uint32_t w) {
    if constexpr (QT::is_f16)
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.f, HI));
    else
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.f, HI));
  }
};

// Four fp32 values to four fp8 codes (byte e from y[e]): values beyond the
// largest finite one are clipped to it first (the conversion itself rounds
// to nearest even and does not saturate), NaN becomes 0x7F.
template <bool E4M3>
__device__ __forceinline__ uint32_t fp8_pack4(const float (&y)[4]) {
  constexpr float kMax = E4M3 ? 448.f : 57344.f;
  float c[4];
  uint32_t nan_mask = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    nan_mask |= (y[e] != y[e]) ? (0xffu << (8 * e)) : 0u;
    c[e] = fminf(fmaxf(y[e], -kMax), kMax);
  }
  uint32_t w;
  if constexpr (E4M3) {
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)w, true);
  } else {
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], (int)w, true);
  }
  return (w & ~nan_mask) | (0x7f7f7f7fu & nan_mask);
}

// Source element i of a 16-byte vector group, widened exactly to fp32.
template <typename ST>
__device__ __forceinline__ float src_elem(const u32x4 (&v)[4], int i);
template <>
__device__ __forceinline__ float src_elem<TF32>(const u32x4 (&v)[4], int i) {
  return u2f(v[i / 4].w[i % 4]);
}
template <>
__device__ __forceinline__ float src_elem<TF16>(const u32x4 (&v)[4], int i) {
  const uint32_t w = v[i / 8].w[(i % 8) / 2];
  return (i & 1) ? TF16::hi(w) : TF16::lo(w);
}
template <>
__device__ __forceinline__ float src_elem<TBF16>(const u32x4 (&v)[4], int i) {
  const uint32_t w = v[i / 8].w[(i % 8) / 2];
  return (i & 1) ? TBF16::hi(w) : TBF16::lo(w);
}

// Store one float as element type TT at p[idx].
template <typename TT>
__device__ __forceinline__ void store_elem(void* p, int64_t idx, float x);

template <>
__device__ __forceinline__ void store_elem<TF32>(void* p, int64_t idx, float x) {
  reinterpret_cast<float*>(p)[idx] = x;
}
template <>
__device__ __forceinline__ void store_elem<TF16>(void* p, int64_t idx, float x) {
  reinterpret_cast<uint16_t*>(p)[idx] = TF16::from_float(x);
}
template <>
__device__ __forceinline__ void store_elem<TBF16>(void* p, int64_t idx, float x) {
  reinterpret_cast<uint16_t*>(p)[idx] = TBF16::from_float(x);
}

// ---- cross-lane data movement inside a 64-lane wavefront ------------------

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowRor8 = 0x128;     // rotate right by 8 within 16 lanes (= xor 8)

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Sum over the 8 lanes {8j .. 8j+7}; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Order LDS accesses of one wavefront across lanes (writes before reads by
// other lanes of the same wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pkv
