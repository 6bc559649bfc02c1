// float32 -> OCP E4M3FN conversion shared by the append kernels and the
// conversion check in the probe library (which runs both forms below on
// every binary32 input).  Device-only; included inside each source's own namespace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
namespace {

// float32 -> OCP E4M3FN codes of two values (low byte: a): round to
// nearest, ties to even; |x| >= 448 (infinities included) saturates to
// +-448; NaN gives the NaN code with the input's sign.  gfx950's
// v_cvt_pk_fp8_f32 rounds to nearest even but does not saturate, so it is
// given the values clamped to [-448, 448] by v_med3_f32; the clamp turns a
// NaN into a number, so NaN codes are put back afterwards.  Over all 2^32
// binary32 inputs, in both halves of the pair, this equals the rounding of
// the binary32 fields written out from the format (pkv_probe_e4m3_check).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.f, 448.f),
                                                         __builtin_amdgcn_fmed3f(b, -448.f, 448.f), 0, false);
  if (a != a) w = (w & 0xFF00u) | ((__builtin_bit_cast(uint32_t, a) >> 24) & 0x80u) | 0x7Fu;
  if (b != b) w = (w & 0x00FFu) | ((((__builtin_bit_cast(uint32_t, b) >> 24) & 0x80u) | 0x7Fu) << 8);
  return w & 0xFFFFu;
}

// The same rounding for four values, byte i of the result for the i-th: the
// two pairs go into the two halves of one word through v_cvt_pk_fp8_f32's
// word select, and the NaN codes are put back only when one of the four is
// NaN (a branch the wave skips when no lane has one).
__device__ __forceinline__ uint32_t e4m3_nan_code(float x) {
  return ((__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u) | 0x7Fu;
}
__device__ __forceinline__ uint32_t e4m3_quad(float a, float b, float c, float d) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.f, 448.f),
                                                         __builtin_amdgcn_fmed3f(b, -448.f, 448.f), 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, -448.f, 448.f),
                                                __builtin_amdgcn_fmed3f(d, -448.f, 448.f), (int)w, true);
  if (__builtin_expect(__builtin_isunordered(a, b) || __builtin_isunordered(c, d), 0)) {
    if (a != a) w = (w & 0xFFFFFF00u) | e4m3_nan_code(a);
    if (b != b) w = (w & 0xFFFF00FFu) | (e4m3_nan_code(b) << 8);
    if (c != c) w = (w & 0xFF00FFFFu) | (e4m3_nan_code(c) << 16);
    if (d != d) w = (w & 0x00FFFFFFu) | (e4m3_nan_code(d) << 24);
  }
  return w;
}

}  // namespace
}  // namespace pkv
