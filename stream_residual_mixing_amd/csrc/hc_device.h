// Device-side helpers shared by the gfx950 kernels of libhc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

typedef uint16_t bf16_t;

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-to-nearest-even float -> bfloat16 bits (quiet NaN kept).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// The same rounding (to nearest even) in one instruction, v_cvt_pk_bf16_f32;
// NaNs come out as the instruction's quiet NaN.
__device__ __forceinline__ uint32_t pack_bf2_hw(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const b2_t r = __builtin_convertvector((f2_t){lo, hi}, b2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------- element access

template <typename T> struct Elem;

template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};

template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = (bf16_t)f2bf(v); }
};

// 8 consecutive elements; the pointer must be 16-byte aligned.
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  v[0] = bf2f(q.x & 0xffffu); v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = bf2f(q.y & 0xffffu); v[3] = __uint_as_float(q.y & 0xffff0000u);
  v[4] = bf2f(q.z & 0xffffu); v[5] = __uint_as_float(q.z & 0xffff0000u);
  v[6] = bf2f(q.w & 0xffffu); v[7] = __uint_as_float(q.w & 0xffff0000u);
}

// Nontemporal forms for state streamed once per pass (it does not displace what
// L2 holds for reuse).
__device__ __forceinline__ void load8_nt(const float* p, float v[8]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 a = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
  const f4 b = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p) + 1);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8_nt(const bf16_t* p, float v[8]) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  const u4 q = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  v[0] = bf2f(q.x & 0xffffu); v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = bf2f(q.y & 0xffffu); v[3] = __uint_as_float(q.y & 0xffff0000u);
  v[4] = bf2f(q.z & 0xffffu); v[5] = __uint_as_float(q.z & 0xffff0000u);
  v[6] = bf2f(q.w & 0xffffu); v[7] = __uint_as_float(q.w & 0xffff0000u);
}

__device__ __forceinline__ void store8_nt(float* p, const float v[8]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4*>(p));
  __builtin_nontemporal_store(f4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f4*>(p) + 1);
}

__device__ __forceinline__ void store8_nt(bf16_t* p, const float v[8]) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                 pack_bf2(v[6], v[7])},
                              reinterpret_cast<u4*>(p));
}

__device__ __forceinline__ void store8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  uint4 q;
  q.x = pack_bf2(v[0], v[1]);
  q.y = pack_bf2(v[2], v[3]);
  q.z = pack_bf2(v[4], v[5]);
  q.w = pack_bf2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = q;
}

// Up to 8 consecutive elements with a bounds count (scalar accesses).
template <typename T>
__device__ __forceinline__ void load8_tail(const T* p, int cnt, float v[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (e < cnt) ? Elem<T>::ld(p + e) : 0.f;
}

template <typename T>
__device__ __forceinline__ void store8_tail(T* p, int cnt, const float v[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < cnt) Elem<T>::st(p + e, v[e]);
}

// ------------------------------------------------------------ reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over the whole block; every thread gets the result. `red` holds one
// float per wave (blockDim.x / 64 <= 16). Contains two barriers.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < nw; ++w) s += red[w];
  return s;
}

// Lane exchange within rows of 16 lanes (DPP): quad permutations and row rotations.
constexpr int DPP_QXOR1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int DPP_QXOR2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROR4 = 0x124;  // row_ror:4
constexpr int DPP_ROR8 = 0x128;  // row_ror:8
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// the sum over a row of 16 lanes, in every lane of the row
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<DPP_QXOR1>(x);
  x += dpp<DPP_QXOR2>(x);
  x += dpp<DPP_ROR8>(x);
  x += dpp<DPP_ROR4>(x);
  return x;
}

// ------------------------------------------------------------ activations

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace hc
