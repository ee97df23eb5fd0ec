// Device-side helpers shared by the librdt kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 storage
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;

#define RDT_DEV __device__ __forceinline__

RDT_DEV float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// float -> bfloat16 with the hardware conversion: round to nearest even, NaN
// kept quiet (checked on MI355X against the bit-level rounding for 4M values
// including ties, denormals, infinities and NaNs: identical).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
RDT_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two floats -> packed bfloat16 pair (low half = a), one instruction.
RDT_DEV uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct ST;
template <> struct ST<float> {
  static constexpr int VEC = 4;  // elements per 16-byte vector
  static RDT_DEV float to_f(float x) { return x; }
  static RDT_DEV float from_f(float x) { return x; }
};
template <> struct ST<bf16_t> {
  static constexpr int VEC = 8;
  static RDT_DEV float to_f(bf16_t x) { return bf2f(x); }
  static RDT_DEV bf16_t from_f(float x) { return f2bf(x); }
};

// A lane's share of one 16x16x32 MFMA operand: 8 consecutive k values.
// bf16: one 16-byte vector; float: two 16-byte vectors.
template <typename T> struct Frag { uint4 v[sizeof(T) / 2]; };

template <typename T> RDT_DEV Frag<T> frag_zero() {
  Frag<T> f;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) f.v[i] = make_uint4(0, 0, 0, 0);
  return f;
}

template <typename T> RDT_DEV Frag<T> frag_lds(const T* p) {  // p 16-byte aligned
  Frag<T> f;
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) f.v[i] = q[i];
  return f;
}

// acc[16x16] += A[16 x 32] * B[16 x 32]^T with the lane layout
// lane l: row/col (l % 16), k values 8*(l/16) .. 8*(l/16)+7.
// For float the 32-wide k-step is split over eight 16x16x4 MFMAs; the k order
// differs from the bf16 instruction but is the same for A and B.
RDT_DEV void mma(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v[0]),
                                                __builtin_bit_cast(bf16x8_t, b.v[0]), acc, 0, 0, 0);
}
RDT_DEV void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
  const float* fa = reinterpret_cast<const float*>(a.v);
  const float* fb = reinterpret_cast<const float*>(b.v);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[i], acc, 0, 0, 0);
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() also makes
// every wave wait until its global stores have completed; a GEMM epilogue that
// stages its tile through LDS chunk by chunk does not read those stores back,
// and waiting for them at every chunk cost a 256x256 tile about 20 us.
RDT_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// SiLU(g) * u of the SwiGLU experts, g / (1 + e^-g) * u, with the hardware
// 2^x and reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each; e^-g is
// 2^(-g log2 e)). Every expert epilogue uses this one definition, so tile
// shapes do not change results. The IEEE expf and division cost the 256x256
// gate/up launch on the wide MoE shape 6 % (662 -> 623 us).
RDT_DEV float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g)) * u;
}

// wave64 reductions
RDT_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
RDT_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 8 values of T <-> float
template <typename T> RDT_DEV void store8(T* dst, const float* v);
template <> RDT_DEV void store8<float>(float* dst, const float* v) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <> RDT_DEV void store8<bf16_t>(bf16_t* dst, const float* v) {
  uint4 o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  o.z = pack_bf16x2(v[4], v[5]);
  o.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(dst) = o;
}
template <typename T> RDT_DEV void load4f(const T* src, float* v);
template <> RDT_DEV void load4f<float>(const float* src, float* v) {
  float4 a = *reinterpret_cast<const float4*>(src);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <> RDT_DEV void load4f<bf16_t>(const bf16_t* src, float* v) {
  uint2 a = *reinterpret_cast<const uint2*>(src);
  v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xffff0000u);
  v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xffff0000u);
}
template <typename T> RDT_DEV void store4(T* dst, const float* v);
template <> RDT_DEV void store4<float>(float* dst, const float* v) {
  *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> RDT_DEV void store4<bf16_t>(bf16_t* dst, const float* v) {
  uint2 o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(dst) = o;
}
