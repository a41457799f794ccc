// Device helpers shared by the kvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// Widen the low / high bfloat16 of a packed dword to float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bfloat16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(bf16_t, h);
}

// Two floats -> packed bfloat16 pair (lo = a, hi = b), round to nearest even
// (one v_cvt_pk_bf16_f32).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// acc + a.lo*b.lo + a.hi*b.hi on packed bfloat16 pairs (v_dot2_f32_bf16, float32 accumulate).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         acc, false);
}

// One RoPE pair rotation in float32 (half-split pairs i and i + D/2):
// (x, y) -> (x c - y s, x s + y c).  Every kernel that rotates uses this one
// function, so that they all round the same way.  The fused multiply-adds are
// written out: left as x * c - y * s, which product the compiler fuses may
// differ from one call site (or unrolled copy) to another, and with it the
// last bit of the result.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float& xr, float& yr) {
  xr = fmaf(x, c, -(y * s));
  yr = fmaf(x, s, y * c);
}

// Byte permute: pick bytes of {hi_src:lo_src} (lo_src = bytes 0..3, hi_src = bytes 4..7).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}
// lo16(a) | lo16(b) << 16
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
// hi16(a) | hi16(b) << 16
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// DPP move within rows of 16 lanes (bound_ctrl: out-of-row sources read 0; all patterns here stay in-row).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // row_mirror: lane i <-> 15-i within 16

// Max / sum over all 64 lanes; every lane receives the result.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppMirror>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  x += dpp_f32<kDppMirror>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Order this wave's LDS accesses around a point (lanes exchange data through LDS).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void report(int32_t* dev_err, int32_t bit) {
  if (dev_err) atomicOr(dev_err, bit);
}

}  // namespace kvc
