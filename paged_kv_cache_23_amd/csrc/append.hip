// KV append: scatter each new token's K and V into its cache slot.
//
// Habr KV-Cache article (habr.com/ru/articles/1021832), section 1 "Prefill
// and Decode": each decode step computes K and V for the new token only and
// appends them to the cache.  Section 4, step-by-step example: the token
// lands in the next slot of the sequence's last block (the host opened a
// fresh block when the last one was full).  A slot is block * B + offset for
// B tokens per block.
//
// K tiles are token-major, so a token's K row is D contiguous elements; V
// tiles are dim-major, so its V column is D elements B apart.  For an fp8
// cache the bf16 input is divided by the kv head's float32 scale (IEEE
// division) and rounded to E4M3 below.

#include "pkv_internal.h"

#include <type_traits>

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// A 16-byte vector viewed as its elements.
template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  typedef uint16_t type __attribute__((ext_vector_type(8)));
};
template <>
struct Vec16<uint32_t> {
  typedef uint32_t type __attribute__((ext_vector_type(4)));
};

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

// Value stored for new element x of kv head h: a bit copy, or for an fp8
// cache the E4M3 code of x / scale[h].
template <int KV>
struct Store;
template <>
struct Store<kF32> {
  using In = uint32_t;
  using Out = uint32_t;
  __device__ static Out put(In x, float) { return x; }
};
template <>
struct Store<kBF16> {
  using In = uint16_t;
  using Out = uint16_t;
  __device__ static Out put(In x, float) { return x; }
};
template <>
struct Store<kFP8> {
  using In = uint16_t;   // bf16
  using Out = uint8_t;
  __device__ static Out put(In x, float s) {
    return (Out)e4m3_from_f32(__fdiv_rn(__builtin_bit_cast(float, (uint32_t)x << 16), s));
  }
};

// Few new tokens (a decode step: one per sequence, each into its own
// block): one wave per (token, kv head), so every token's quantisation and
// scattered V column run in parallel across the machine.
template <int KV, int D>
__global__ __launch_bounds__(64) void append_scatter_kernel(AppendArgs a) {
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

constexpr int kGroup = 16;          // new tokens per workgroup
constexpr int kAppendThreads = 256;

// One workgroup per (16 consecutive new tokens, kv head).  When the 16
// tokens' slots are 16 consecutive rows of one block (a prefill chunk's
// appends), the K rows form one contiguous run of the block's K tile and
// the V columns 16-token pieces of every row of its V tile: K is written
// as that run, V is transposed through LDS and written row by row.  Any
// other slots (one token per sequence in a decode step, padding, a run
// that crosses a block) take the element-wise scatter: K row `off`, V
// column `off` of the slot's block.
template <int KV, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  using S = Store<KV>;
  using In = typename S::In;
  using Out = typename S::Out;
  const int g0 = blockIdx.x * kGroup;   // first new token of the group
  const int h = blockIdx.y;
  const int Hkv = a.num_kv_heads;
  const int bs = a.block_size;
  const int n = min(kGroup, a.num_tokens - g0);
  const int tid = threadIdx.x;
  const In* kn = static_cast<const In*>(a.k_new);
  const In* vn = static_cast<const In*>(a.v_new);
  Out* kp = static_cast<Out*>(a.k_pool);
  Out* vp = static_cast<Out*>(a.v_pool);
  float ks = 1.f, vs = 1.f;
  if constexpr (KV == kFP8) {
    ks = a.k_scale[h];
    vs = a.v_scale[h];
  }
  const int64_t limit = (int64_t)a.num_blocks * bs;

  __shared__ int64_t slot[kGroup];
  __shared__ __attribute__((aligned(16))) Out vt[D][kGroup + 16 / sizeof(Out)];   // V transposed: [dim][token], rows padded by 16 bytes
  if (tid < kGroup) slot[tid] = tid < n ? a.slot_mapping[g0 + tid] : -1;
  __syncthreads();

  const int64_t base = slot[0];
  bool run = n == kGroup && base >= 0 && base + kGroup <= limit && (base % bs) % kGroup == 0;
  for (int k = 1; k < kGroup && run; ++k) run = slot[k] == base + k;

  if (run) {
    const int64_t blk = base / bs;
    const int off = (int)(base - blk * bs);
    const size_t tile = ((size_t)blk * Hkv + h) * bs * D;   // the (block, head) tile, in elements
    // 16-byte input vectors: kVec elements of one new token's row
    constexpr int kVec = 16 / sizeof(In);
    constexpr int kRowVecs = D / kVec;
    // K: rows off .. off+15 of the tile are kGroup * D contiguous elements
    Out* kdst = kp + tile + (size_t)off * D;
    for (int v = tid; v < kGroup * kRowVecs; v += kAppendThreads) {
      const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
      const u32x4 w = *reinterpret_cast<const u32x4*>(kn + ((size_t)(g0 + k) * Hkv + h) * D + d0);
      if constexpr (KV == kFP8) {
        const auto x = __builtin_bit_cast(typename Vec16<In>::type, w);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) lo |= (uint32_t)S::put(x[e], ks) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi |= (uint32_t)S::put(x[4 + e], ks) << (8 * e);
        *reinterpret_cast<u32x2*>(kdst + (size_t)k * D + d0) = u32x2{lo, hi};
      } else {
        *reinterpret_cast<u32x4*>(kdst + (size_t)k * D + d0) = w;
      }
    }
    // V: element (token k, dim d) goes to row d, column off + k, through LDS
    for (int v = tid; v < kGroup * kRowVecs; v += kAppendThreads) {
      const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
      const u32x4 w = *reinterpret_cast<const u32x4*>(vn + ((size_t)(g0 + k) * Hkv + h) * D + d0);
      const auto x = __builtin_bit_cast(typename Vec16<In>::type, w);
#pragma unroll
      for (int e = 0; e < kVec; ++e) vt[d0 + e][k] = S::put(x[e], vs);
    }
    __syncthreads();
    // 16-byte pieces of the V rows: kOut tokens of one dim
    constexpr int kOut = 16 / sizeof(Out);
    constexpr int kRowPieces = kGroup / kOut;
    Out* vdst = vp + tile + off;
    for (int v = tid; v < D * kRowPieces; v += kAppendThreads) {
      const int d = v / kRowPieces, k0 = (v - d * kRowPieces) * kOut;
      *reinterpret_cast<u32x4*>(vdst + (size_t)d * bs + k0) = *reinterpret_cast<const u32x4*>(&vt[d][k0]);
    }
    return;
  }

  // element-wise scatter
  for (int e = tid; e < n * D; e += kAppendThreads) {
    const int k = e / D, d = e - k * D;
    const int64_t sl = slot[k];
    if (sl < 0 || sl >= limit) continue;   // padding
    const int64_t blk = sl / bs;
    const int off = (int)(sl - blk * bs);
    const size_t tile = ((size_t)blk * Hkv + h) * bs * D;
    const size_t src = ((size_t)(g0 + k) * Hkv + h) * D + d;
    kp[tile + (size_t)off * D + d] = S::put(kn[src], ks);
    vp[tile + (size_t)d * bs + off] = S::put(vn[src], vs);
  }
}

// Token count from which the tiled kernel runs: below it the appends are a
// decode step's (one token per sequence), which the one-wave-per-token
// kernel spreads over more of the machine; from it on, prefill chunks whose
// consecutive slots the tiled kernel writes tile by tile.
constexpr int kTileMinTokens = 1024;

template <int KV, int D>
hipError_t launch_t(const AppendArgs& a, hipStream_t stream) {
  if (a.num_tokens < kTileMinTokens) {
    const unsigned grid = (unsigned)a.num_tokens * (unsigned)a.num_kv_heads;
    hipLaunchKernelGGL((append_scatter_kernel<KV, D>), dim3(grid), dim3(64), 0, stream, a);
  } else {
    const dim3 grid((unsigned)((a.num_tokens + kGroup - 1) / kGroup), (unsigned)a.num_kv_heads);
    hipLaunchKernelGGL((append_kernel<KV, D>), grid, dim3(kAppendThreads), 0, stream, a);
  }
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
