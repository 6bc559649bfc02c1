// float32 -> OCP E4M3FN conversion shared by the append kernels and the
// conversion check in the probe library (which runs it on every binary32
// input).  Device-only; included inside each source's own namespace.
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

}  // namespace
}  // namespace pkv
