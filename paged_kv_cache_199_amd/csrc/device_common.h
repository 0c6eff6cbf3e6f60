// Device-side helpers shared by the library's kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;                       // tokens per KV page
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max seed.  Finite on purpose: exp2(seed - seed) = 1 and exp2(-inf - seed) = 0, so the online
// softmax never forms inf - inf.  A row that sees no key keeps it and ends with a zero sum.
constexpr float kNegBig = -1.0e30f;
// Lazy rescale: the running max only moves when a score exceeds it by more than this (log2 units),
// so every exp2 argument stays <= kRescaleSlack and the sum stays far from fp32 overflow.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.  gfx950 converts in one instruction
// (v_cvt_pk_bf16_f32, two values at a time).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float float2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_v{lo, hi}), bf16x2_v));
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// DPP lane moves inside a 16-lane row (all source lanes valid for the controls used here).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // row_ror:4
constexpr int kRowRor8 = 0x128;   // row_ror:8

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_mov<kQuadXor1>(v);
  v += dpp_mov<kQuadXor2>(v);
  return v;
}

// Reduction over the 16 quads of a wave (lane bits 2..5); lanes of a quad hold equal values.
__device__ __forceinline__ float quads_max(float v) {
  v = fmaxf(v, dpp_mov<kRowRor4>(v));
  v = fmaxf(v, dpp_mov<kRowRor8>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float quads_sum(float v) {
  v += dpp_mov<kRowRor4>(v);
  v += dpp_mov<kRowRor8>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroups are handed to the 8 XCDs round robin (workgroup i runs on XCD i % 8).  This maps the
// hardware index to a work-unit index so that each XCD walks one contiguous range of units, keeping
// units that read the same data (row tiles of one KV stream, sequences sharing prefix pages) under
// one L2.
__device__ __forceinline__ int xcd_unit(int hw, int per_xcd) { return (hw & 7) * per_xcd + (hw >> 3); }

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Orders this wave's LDS writes before its following LDS reads of other lanes' data (LDS executes a
// wave's operations in issue order; this keeps the compiler from reordering them and waits for the
// writes to land).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace pkv
