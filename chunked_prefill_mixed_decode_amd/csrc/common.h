// Device helpers shared by the gfx950 kernels of libcb: element types, 8-element fragments
// and the matrix-core (MFMA) steps used for the attention contractions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cb {

using bf16_t = __bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// Float32 -> bfloat16 bits, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats -> two bfloat16 (round to nearest, ties to even) in one v_cvt_pk_bf16_f32; a in the
// low half.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// 2^x on the hardware exponential (v_exp_f32): exact at 0, 0 for -inf, results below the
// smallest normal flushed to 0.  Used for softmax weights, which are then rounded to bf16 or
// summed in float32.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight consecutive elements of T held by one lane.  For bf16 that is 16 bytes (one dwordx4),
// for float 32 bytes (two).
template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = u; }
  __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&u.x)[i >> 1];
    return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
  }
  // Pack 8 floats (rounded to nearest-even).
  __device__ __forceinline__ void set_all(const float* f) {
    u = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7]));
  }
  __device__ __forceinline__ bf16x8 vec() const { return __builtin_bit_cast(bf16x8, u); }
};

template <> struct Frag<float> {
  float f[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.f;
  }
  __device__ __forceinline__ float get(int i) const { return f[i]; }
  __device__ __forceinline__ void set_all(const float* g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = g[i];
  }
};

// One 32x32 output tile, contraction over 16 "slots": lane l supplies row/column l % 32 and
// slots 8 * (l / 32) + j, j = 0..7, of both operands.  bf16: one v_mfma_f32_32x32x16_bf16.
// float: eight v_mfma_f32_32x32x2_f32, the j-th taking slot j of every lane (so each pairs the
// same slots of A and B; the union over j covers all 16).
__device__ __forceinline__ void mma32_k16(f32x16& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.vec(), b.vec(), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32_k16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.f[j], b.f[j], acc, 0, 0, 0);
}

// One 16x16 output tile, contraction over 32 slots: lane l supplies row/column l % 16 and slots
// 8 * (l / 16) + j.  bf16: one v_mfma_f32_16x16x32_bf16; float: eight v_mfma_f32_16x16x4_f32.
__device__ __forceinline__ void mma16_k32(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.vec(), b.vec(), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16_k32(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[j], b.f[j], acc, 0, 0, 0);
}

// Output layouts of the accumulators (lane l, register r):
//   32x32: row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32
//   16x16: row 4 * (l / 16) + r,                    column l % 16
__device__ __forceinline__ int acc32_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc16_row(int lane, int r) { return 4 * (lane >> 4) + r; }

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_xor_sum(float v, int mask) { return v + __shfl_xor(v, mask, 64); }
// Maximum over lanes i and i ^ 32 with gfx950's v_permlane32_swap: the two 32-lane halves trade
// values inside the VALU (no LDS round trip, so no wait on the lane's other LDS traffic).  The
// pair it returns is {v[i], v[i ^ 32]} in either order; the maximum does not depend on which.
// The final maximum is one v_max_f32 from asm: the inputs are scores or -inf (never signalling
// NaNs), so the canonicalising moves fmaxf would add are not needed.
__device__ __forceinline__ float half_xor_max(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(sw[0]), "v"(sw[1]));
  return r;
}

constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace cb
