// Device-side helpers shared by the libsnapstream kernels (gfx950 / CDNA4,
// wave64).  Storage types: float (fp32) or uint16_t holding bfloat16 bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// native 16-byte vector (HIP's uint4 class wrapper can keep register arrays
// from being promoted out of stack memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// fp64 -> bf16 in one rounding step (no fp32 intermediate): round the
// binary64 significand at bit 45 (keeping 8 significant bits) to nearest
// even, then the result is exact in fp32 and its top half is the bf16.
// Finite inputs with |x| >= 2^-126 (bf16 normal range) or x == 0.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  u += 0x0fffffffffffull + ((u >> 45) & 1ull);   // 2^44 - 1 + lsb of the kept part
  u &= ~0x1fffffffffffull;                         // clear the 45 dropped bits
  float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
  return static_cast<bf16_t>(__float_as_uint(f) >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

template <typename T> __device__ __forceinline__ T from_f64(double x);
template <> __device__ __forceinline__ float from_f64<float>(double x) { return static_cast<float>(x); }
template <> __device__ __forceinline__ bf16_t from_f64<bf16_t>(double x) { return f64_to_bf16(x); }

// ------------------------------------------------------------------ MFMA tile
// 16x16 output tiles.  Operand layout shared by A (M x K) and B (K x N):
// lane l supplies row/column (l % 16) and KPL consecutive k-values starting
// at (l / 16) * KPL; the accumulator lane l holds column (l % 16), rows
// 4 * (l / 16) + r, r = 0..3.
template <typename T> struct Mma;

template <> struct Mma<float> {  // v_mfma_f32_16x16x4_f32
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 4;
  typedef float frag;
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.f; }
};

template <> struct Mma<bf16_t> {  // v_mfma_f32_16x16x32_bf16 (gfx950)
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 32;
  typedef bf16x8_t frag;
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // 16-byte load of 8 consecutive bf16 values (p must be 16-byte aligned)
  static __device__ __forceinline__ frag load(const bf16_t* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4_t*>(p));
  }
  static __device__ __forceinline__ frag zero() {
    return __builtin_bit_cast(frag, u32x4_t{0u, 0u, 0u, 0u});
  }
};

// pack 8 bf16 bit patterns (low index in the low half of each dword)
__device__ __forceinline__ bf16x8_t pack_bf16x8(const bf16_t* e) {
  u32x4_t u;
  u.x = static_cast<uint32_t>(e[0]) | (static_cast<uint32_t>(e[1]) << 16);
  u.y = static_cast<uint32_t>(e[2]) | (static_cast<uint32_t>(e[3]) << 16);
  u.z = static_cast<uint32_t>(e[4]) | (static_cast<uint32_t>(e[5]) << 16);
  u.w = static_cast<uint32_t>(e[6]) | (static_cast<uint32_t>(e[7]) << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

// ---------------------------------------------------------- cross-lane reduce
// 2^x from the hardware instruction (v_exp_f32): no denormal results (they
// flush to 0), -inf gives 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, WAVE));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, WAVE);
}

// v + the value of lane l ^ 16 (resp. l ^ 32), through the gfx950 row-swap
// instructions (no LDS): v_permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second, so with both operands v
// the two results hold, in every lane, v and the partner's v.
__device__ __forceinline__ float sum_across_16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_across_32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// the maximum of v and the value of lane l ^ 16 (resp. l ^ 32), through the
// same row swaps
__device__ __forceinline__ float max_across_16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_across_32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace ss
