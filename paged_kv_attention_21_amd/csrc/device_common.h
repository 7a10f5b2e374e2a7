// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pka {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite "minus infinity" for running maxima: exp2(m - m') stays 0 or 1 and
// never becomes NaN when both maxima are still at their initial value.
constexpr float kNegBig = -1.0e30f;

struct F16 {};
struct BF16 {};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

template <typename T>
struct Elem;

// fp16: two elements per dword.  dot2 is v_dot2c_f32_f16 (fp32 accumulate).
template <>
struct Elem<F16> {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
  }
  static __device__ __forceinline__ float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
  // round to nearest even
  static __device__ __forceinline__ uint16_t from_float(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
  // two at once, round to nearest even (one v_cvt_pk_f16_f32)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, half2_t));
  }
};

// bf16: the upper half of an fp32.  dot2 is v_dot2c_f32_bf16.
template <>
struct Elem<BF16> {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), c,
                                           false);
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  static __device__ __forceinline__ uint16_t from_float(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
  // two at once, round to nearest even (one v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf162_t));
  }
};

// Lane move inside a 16-lane DPP row (bound_ctrl: out-of-row reads give 0,
// which the patterns below never do).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within 16

// Sum over aligned groups of N consecutive lanes (N in 8, 16, 32, 64);
// every lane of a group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group of 8..64 lanes");
  x += dpp_mov<kDppQuadSwap1>(x);
  x += dpp_mov<kDppQuadSwap2>(x);
  x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef int int4v_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: data read once (the decode K/V stream)
// should not displace reusable lines in L2 / Infinity Cache.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const int4v_t*>(p)));
}

__device__ __forceinline__ int uniform_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Combine lane l with lane l ^ 16 (resp. l ^ 32) without going through LDS:
// v_permlane16_swap / v_permlane32_swap exchange rows between two registers,
// so swapping two copies of x leaves, in every lane, x[l] in one register and
// x[l ^ 16] (resp. x[l ^ 32]) in the other; a symmetric combine of the two is
// the butterfly step whichever way the rows moved.  Written as inline asm
// (with the two wait states a VALU write needs before a permlane read)
// because this compiler's two-result builtins hand back one register twice.
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// v_max_f32 without the NaN-quieting copies fmaxf adds for operands the
// compiler cannot see into (the permlane results).
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float xor16_max(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float xor32_max(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float xor16_sum(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  return a + b;
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  return a + b;
}

// Index of this wavefront in the workgroup, in a scalar register: loops and
// branches that depend only on it compile to scalar control flow.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

}  // namespace pka
