// Shared device helpers for the qlin kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs

constexpr int kTile = 64;     // rows per layout tile: one row per lane of a wave
constexpr int kBlock = 64;    // codes per K-block (and per group)
constexpr uint32_t kMagic = 0x64006400u;  // two fp16 1024.0: OR a code into the mantissa

// A constant materialized once in a VGPR.  gfx9 VOP3 encodings take no
// literal operand, so (v & mask) | magic becomes one v_and_or_b32 only when
// the magic number already sits in a register.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Round-to-nearest of w / s, then clamped to [lo, hi], for w / s taken as the
// exact quotient: t = w * r with r = fl32(1/s) rounds the same way as the
// correctly rounded quotient everywhere except at exact half-way cases (an
// fp16/fp16 quotient that is not a tie sits much farther from a half-integer
// than the product's rounding error).  A tie is detected exactly: e = w - q0*s
// is computed without rounding by the fma, and |e| == s/2 only at a tie, where
// the even neighbour q0 +- 1/2 -> rint is chosen.  `fix` enables the tie path.
struct RtnParams {
  float s, r, hs, lo, hi;
};

__device__ __forceinline__ RtnParams rtn_params(float s, int z, int qmax) {
  RtnParams p;
  if (s == 0.f) {   // constant group: every code is 0 and z is 0
    p.s = 0.f; p.r = 0.f; p.hs = -1.f; p.lo = 0.f; p.hi = 0.f;
  } else {
    p.s = s;
    p.r = __fdiv_rn(1.0f, s);
    p.hs = 0.5f * s;
    p.lo = (float)(-z);
    p.hi = (float)(qmax - z);
  }
  return p;
}

// q0 = rint(w * r) without the tie correction, and whether w sits on a tie.
__device__ __forceinline__ float rtn_raw(float w, const RtnParams& p, bool& tie) {
  float q0 = __builtin_rintf(w * p.r);
  float e = __builtin_fmaf(-q0, p.s, w);
  tie = __builtin_fabsf(e) == p.hs;
  return q0;
}

__device__ __forceinline__ float rtn_fix(float w, float q0, const RtnParams& p) {
  float e = __builtin_fmaf(-q0, p.s, w);
  if (__builtin_fabsf(e) == p.hs) q0 = __builtin_rintf(q0 + __builtin_copysignf(0.5f, e));
  return q0;
}

// clamp to [lo, hi] (lo <= hi, v finite): one v_med3_f32
__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(v, lo, hi);
}


// Work-group barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for the wave's global loads still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace qlin
