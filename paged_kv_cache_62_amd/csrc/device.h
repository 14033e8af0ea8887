// device.h -- device-side helpers shared by the kernels of libpkv (append,
// decode and prefill translation units). Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "kernels.h"

namespace pkv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order: a
// loop whose index is a compile-time constant in every body, so that arrays
// indexed by it stay in registers.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int kWaves = 4;             // wavefronts per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = 16;             // tokens per unit of work (one MFMA tile of tokens)
constexpr int kRsrcWord3 = 0x00020000; // buffer descriptor word 3 for untyped dword loads (gfx9 family)
// sched_barrier mask: ALU, VALU, SALU and MFMA instructions may be scheduled
// across the barrier; memory instructions may not.
constexpr int kSchedAluOnly = 0x000F;
constexpr int kSlack = 4;              // the running max may trail the true maximum by this much (log2)
// The longest partition is 4 wavefronts x 64 units of 16 tokens, so one lane
// per unit holds a wavefront's bookkeeping.
static_assert(kMaxPartitionTokens == kWaves * 64 * kUnit, "partition bound");
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (DT == kF32) return ((const float*)p)[i];
  else if constexpr (DT == kF16) return f16_to_f32(((const uint16_t*)p)[i]);
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

// DPP moves inside a row of 16 lanes; lanes that would read outside the row
// read 0 (bound_ctrl).
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <- 7-i within 8
constexpr int kMirror = 0x140;     // lane i <- 15-i within 16
constexpr int kRowShl4 = 0x104;    // lane i <- i+4
constexpr int kRowShl8 = 0x108;    // lane i <- i+8
constexpr int kRowShr8 = 0x118;    // lane i <- i-8

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}

// Maximum over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kQuadXor1>(x));
  x = fmaxf(x, dpp_f<kQuadXor2>(x));
  x = fmaxf(x, dpp_f<kHalfMirror>(x));
  x = fmaxf(x, dpp_f<kMirror>(x));
  const int b = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Combine the four 16-lane rows holding the same column: lane l with lanes
// l^16, l^32, l^48 (the swaps exchange whole rows between two registers).
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)r16[0]), __builtin_bit_cast(float, (int)r16[1]));
  const int c = __builtin_bit_cast(int, x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r32[0]), __builtin_bit_cast(float, (int)r32[1]));
}
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = __builtin_bit_cast(float, (int)r16[0]) + __builtin_bit_cast(float, (int)r16[1]);
  const int c = __builtin_bit_cast(int, x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_bit_cast(float, (int)r32[0]) + __builtin_bit_cast(float, (int)r32[1]);
}

__device__ __forceinline__ int wave_max_int(int x) {
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// A float that is wave-uniform by construction, moved to a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// A pointer the compiler can treat as wave-uniform (it is, by construction,
// wherever this is used): buffer descriptors must live in scalar registers,
// and a value it cannot prove uniform costs a loop over the lanes per load.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

// INT8 V codes are stored biased (code + 128, i.e. code ^ 0x80). Four of them
// -> four fp16 values with two byte permutes, exactly: each byte becomes the
// low mantissa byte of 1024.0 (0x6400), giving 1152 + code.
__device__ __forceinline__ f16x4 biased_i8x4_to_f16x4_plus1152(uint32_t u) {
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  return __builtin_bit_cast(f16x4, make_uint2(lo, hi));
}
// The same with the 1152 subtracted (two packed fp16 subtractions, exact):
// the codes themselves.
__device__ __forceinline__ f16x4 biased_i8x4_to_f16x4(uint32_t u) {
  const f16x4 x = biased_i8x4_to_f16x4_plus1152(u);
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 a = f16x2{x[0], x[1]} - bias;
  const f16x2 b = f16x2{x[2], x[3]} - bias;
  return f16x4{a[0], a[1], b[0], b[1]};
}

// x0, x1 in [0, 2^14) as binary16 pairs hi + lo: hi is x rounded toward zero
// (one conversion instruction, which the compiler cannot fuse with anything,
// so every use sees the same hi); in the binary16 normal range that is x with
// the low 13 of its 23 fraction bits cleared, so lo = x - hi is exact in
// binary32 and is itself rounded toward zero into binary16. hi + lo carries
// about 21 significant bits (|x - hi - lo| < 2^-20 |x|); below 2^-14, where
// hi is subnormal, the remainder is dropped (|error| < 2^-24 absolute).
__device__ __forceinline__ void split_f16x2(float x0, float x1, f16x2& hi, f16x2& lo) {
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  const float h0 = __uint_as_float(__float_as_uint(x0) & 0xFFFFE000u);
  const float h1 = __uint_as_float(__float_as_uint(x1) & 0xFFFFE000u);
  lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0 - h0, x1 - h1));
}

// ---------------------------------------------------------------------------
// The per-(block, KV head) symmetric INT8 quantizer of "轻量级推理引擎实战：KV Cache
// 量化与连续批处理的底层优化" §三, shared by the append kernels and the decode step.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float scale_of(float max_abs) {
  return max_abs > 1e-6f ? max_abs / 127.0f : 1.0f;
}
__device__ __forceinline__ int8_t encode(float x, float scale) {
  const float y = x / scale;  // IEEE binary32 division (correctly rounded)
  const float rr = fminf(fmaxf(rintf(y), -127.0f), 127.0f);  // rintf: ties to even
  return (int8_t)(int)rr;
}
// Re-encode the bytes of a word of codes selected by `mask` from scale s_old
// to s_new (the bytes are stored XOR bias4).
__device__ __forceinline__ uint32_t requant_word(uint32_t w, uint32_t mask, float s_old, float s_new,
                                                 uint32_t bias4) {
  uint32_t x = w ^ bias4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (mask & (0xFFu << (8 * b))) {
      const int code = (int)(int8_t)(x >> (8 * b));
      const uint32_t q = (uint32_t)(uint8_t)encode((float)code * s_old, s_new);
      x = (x & ~(0xFFu << (8 * b))) | (q << (8 * b));
    }
  }
  return x ^ bias4;
}

}  // namespace
}  // namespace pkv
