// KV append: scatter each new token's K and V into its cache slot.
//
// Habr KV-Cache article (habr.com/ru/articles/1021832), section 1 "Prefill
// and Decode": each decode step computes K and V for the new token only and
// appends them to the cache.  Section 4, step-by-step example: the token
// lands in the next slot of the sequence's last block (the host opened a
// fresh block when the last one was full).  A slot is block * B + offset for
// B tokens per block.
//
// One wave per (token, kv head).  K tiles are token-major, so a token's K
// row is D contiguous elements; V tiles are dim-major, so its V column is D
// elements B apart.  For an fp8 cache the bf16 input is divided by the kv
// head's float32 scale (IEEE division) and rounded to E4M3 below.

#include "pkv_internal.h"

#include <type_traits>

namespace pkv {
namespace {

// float32 -> OCP E4M3FN code: round to nearest, ties to even; |x| >= 448
// (infinities included) saturates to +-448; NaN gives the NaN code with the
// input's sign.  Works on the binary32 fields: the 24-bit significand is
// shifted so that its integer part counts E4M3 grid steps.  In the binade
// of 2^E (E >= -6) the grid step is 2^(E-3), i.e. the significand's top 4
// bits; below 2^-6 the step stays 2^-9 (subnormal codes 0..8).
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;        // NaN
  if (mag >= 0x43E00000u) return sign | 0x7Eu;       // >= 448: saturate
  const int e = (int)(mag >> 23);                    // biased binary32 exponent
  const uint32_t sig = e ? ((mag & 0x7FFFFFu) | 0x800000u) : (mag & 0x7FFFFFu);
  const int e_eff = e ? e : 1;
  const int shift = e_eff >= 121 ? 20 : 141 - e_eff; // 121 = 127 - 6
  if (shift > 24) return sign;                       // below half of 2^-9
  const uint32_t steps = sig >> shift;
  const uint32_t rem = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  const uint32_t q = steps + ((rem > half || (rem == half && (steps & 1u))) ? 1u : 0u);
  // normal binades: code = (E + 7) * 8 + (q - 8) with E = e_eff - 127
  const uint32_t code = e_eff >= 121 ? (uint32_t)(e_eff - 120) * 8u + q - 8u : q;
  return sign | code;
}

template <int KV, int D>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int item = blockIdx.x;
  const int i = item / a.num_kv_heads;
  const int h = item % a.num_kv_heads;
  const int64_t slot = a.slot_mapping[i];
  const int bs = a.block_size;
  if (slot < 0 || slot >= (int64_t)a.num_blocks * bs) return;  // padding
  const int64_t blk = slot / bs;
  const int off = (int)(slot - blk * bs);
  const size_t src = ((size_t)i * a.num_kv_heads + h) * D;
  const size_t ktile = ((size_t)blk * a.num_kv_heads + h) * bs * D;
  const size_t kdst = ktile + (size_t)off * D;     // token-major: row `off`
  const size_t vdst = ktile + off;                 // dim-major: column `off`
  for (int d = threadIdx.x; d < D; d += 64) {
    if constexpr (KV == kFP8) {
      const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
      const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
      const float kx = __builtin_bit_cast(float, (uint32_t)kn[src + d] << 16);
      const float vx = __builtin_bit_cast(float, (uint32_t)vn[src + d] << 16);
      static_cast<uint8_t*>(a.k_pool)[kdst + d] = (uint8_t)e4m3_from_f32(__fdiv_rn(kx, a.k_scale[h]));
      static_cast<uint8_t*>(a.v_pool)[vdst + (size_t)d * bs] =
          (uint8_t)e4m3_from_f32(__fdiv_rn(vx, a.v_scale[h]));
    } else {
      using E = typename std::conditional<KV == kF32, uint32_t, uint16_t>::type;
      static_cast<E*>(a.k_pool)[kdst + d] = static_cast<const E*>(a.k_new)[src + d];
      static_cast<E*>(a.v_pool)[vdst + (size_t)d * bs] = static_cast<const E*>(a.v_new)[src + d];
    }
  }
}

template <int KV, int D>
hipError_t launch_t(const AppendArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_tokens * (unsigned)a.num_kv_heads;
  hipLaunchKernelGGL((append_kernel<KV, D>), dim3(grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) {
    if (a.kv_dtype == kF32) return launch_t<kF32, 64>(a, stream);
    if (a.kv_dtype == kBF16) return launch_t<kBF16, 64>(a, stream);
    return launch_t<kFP8, 64>(a, stream);
  }
  if (a.kv_dtype == kF32) return launch_t<kF32, 128>(a, stream);
  if (a.kv_dtype == kBF16) return launch_t<kBF16, 128>(a, stream);
  return launch_t<kFP8, 128>(a, stream);
}

}  // namespace pkv
