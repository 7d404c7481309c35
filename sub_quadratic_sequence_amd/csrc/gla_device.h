// Device-side helpers for the gfx950 GLA kernels: element I/O for bf16/fp32,
// MFMA wrappers, wave64 DPP lane moves and exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- element types
struct BF16 {
  using storage = unsigned short;     // raw bf16 bits in HBM and LDS
  static constexpr int kBytes = 2;
};
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// Round-to-nearest-even pack of two floats into two bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(unsigned, r);
}
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float x) {
  return (unsigned short)(pack_bf16x2(x, 0.f) & 0xffffu);
}

// Load N consecutive elements (N*bytes is 8, 16 or 32) as floats.
template <typename E, int N>
__device__ __forceinline__ void load_vec(const typename E::storage* p, float* out);

template <>
__device__ __forceinline__ void load_vec<BF16, 8>(const unsigned short* p, float* out) {
  uint4 r = *reinterpret_cast<const uint4*>(p);
  unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load_vec<BF16, 4>(const unsigned short* p, float* out) {
  uint2 r = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(r.x << 16);
  out[1] = __uint_as_float(r.x & 0xffff0000u);
  out[2] = __uint_as_float(r.y << 16);
  out[3] = __uint_as_float(r.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load_vec<F32, 8>(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
template <>
__device__ __forceinline__ void load_vec<F32, 4>(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
}

// Store 4 consecutive elements from floats (RNE rounding for bf16).
template <typename E>
__device__ __forceinline__ void store4(typename E::storage* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<BF16>(unsigned short* p, float a, float b, float c, float d) {
  uint2 r = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<uint2*>(p) = r;
}
template <>
__device__ __forceinline__ void store4<F32>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Store 8 consecutive elements (16 B for bf16, 32 B for fp32).
template <typename E>
__device__ __forceinline__ void store8(typename E::storage* p, const float* x);
template <>
__device__ __forceinline__ void store8<BF16>(unsigned short* p, const float* x) {
  uint4 r = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  *reinterpret_cast<uint4*>(p) = r;
}
template <>
__device__ __forceinline__ void store8<F32>(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Store N (4 or 8) consecutive elements.
template <typename E, int N>
__device__ __forceinline__ void lds_store_n(typename E::storage* p, const float* x) {
  if constexpr (N == 8) {
    store8<E>(p, x);
  } else {
    static_assert(N == 4, "store width");
    store4<E>(p, x[0], x[1], x[2], x[3]);
  }
}

// ---------------------------------------------------------------- MFMA operands
// An "8-slot fragment" is what one lane contributes to a 16x16 tile over 32
// contraction indices: for bf16 one v_mfma_f32_16x16x32_bf16 consumes it, for
// fp32 eight v_mfma_f32_16x16x4_f32 consume one slot each.  A and B fragments
// built with the same slot -> index map contract correctly, whatever order the
// hardware assigns to the slots.
template <typename E>
struct Frag;
template <>
struct Frag<BF16> {
  bf16x8 v;
};
template <>
struct Frag<F32> {
  float v[8];
};

__device__ __forceinline__ void frag_from_f32(Frag<BF16>& f, const float* x) {
  uint4 r = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  f.v = __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ void frag_from_f32(Frag<F32>& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = x[i];
}

// 16 contiguous bytes (bf16) / 32 bytes (fp32) of LDS -> one fragment.
__device__ __forceinline__ void frag_ld8(Frag<BF16>& f, const unsigned short* p) {
  f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void frag_ld8(Frag<F32>& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// Two runs of 4 contiguous elements -> one fragment (slots 0-3 from p0, 4-7 from p1).
__device__ __forceinline__ void frag_ld4x2(Frag<BF16>& f, const unsigned short* p0,
                                           const unsigned short* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0);
  uint2 b = *reinterpret_cast<const uint2*>(p1);
  uint4 r = {a.x, a.y, b.x, b.y};
  f.v = __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ void frag_ld4x2(Frag<F32>& f, const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0);
  float4 b = *reinterpret_cast<const float4*>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// acc += A(16x32) * B(32x16) for one 8-slot fragment pair.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<BF16>& a, const Frag<BF16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<F32>& a, const Frag<F32>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

// ---------------------------------------------------------------- lane moves
// DPP moves inside a row of 16 lanes.  Lanes whose source falls outside the
// row read 0 (bound_ctrl), which lets the compiler fold the move into the
// instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118,
              kRowShr12 = 0x11C;
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128, kRowRor12 = 0x12C;
constexpr int kQuadBcast3 = 0xFF;  // quad_perm:[3,3,3,3]

// Value of lane `src` (0..3) of each group of four lanes (quad_perm broadcast).
template <int SRC>
__device__ __forceinline__ float quad_bcast_c(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), SRC * 0x55, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_bcast(float x, int src) {
  switch (src) {
    case 0: return quad_bcast_c<0>(x);
    case 1: return quad_bcast_c<1>(x);
    case 2: return quad_bcast_c<2>(x);
    default: return quad_bcast_c<3>(x);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gla
