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
// cache the bf16 input is divided by the kv head's float32 scale and
// rounded to E4M3, with the result of the IEEE division followed by E4M3
// rounding (below).

#include "e4m3.h"
#include "pkv_internal.h"

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

// x / s for the E4M3 rounding above, equal in code to the correctly rounded
// binary32 quotient (IEEE division, then E4M3 rounding).  The quotient is
// taken as q0 = x * r with r = 1/s correctly rounded: for a normal s and r
// (and no underflow), q0 is within (2^-23 + 2^-48) |x/s| of x/s and the
// correctly rounded quotient within 2^-24 |x/s|, so the two are within
// 1.5 * 2^-23 |x/s|, i.e. 3 units in the last place of q0, of each other.
// Where the E4M3 rounding cannot tell them apart, q0 is used:
//  - |q0| < 2^-11: both round to a signed zero (below half of 2^-9);
//  - 2^-6 <= |q0| <= 2^16: every E4M3 rounding boundary in that range (the
//    midpoints between neighbouring codes, which keep 4 significand bits)
//    has its 20 low significand bits equal to 0x80000; q0 more than 4 units
//    from that pattern lies strictly on the same side of every boundary as
//    the correctly rounded quotient (values past 448 all saturate).
// Otherwise (the E4M3 subnormal range, near a boundary, huge values, NaN,
// or a scale whose reciprocal is not a normal number) the quotient is the
// IEEE division itself.  The fast case replaces a division sequence by one
// multiply in all but a few inputs in 10^4.
struct Fp8Scale {
  float s, r;
  bool fast;
};
__device__ __forceinline__ Fp8Scale fp8_scale(float s) {
  return Fp8Scale{s, __fdiv_rn(1.f, s), s >= 0x1p-125f && s <= 0x1p125f};
}
__device__ __forceinline__ float fp8_quotient(float x, const Fp8Scale& q) {
  if (q.fast) {
    const float q0 = x * q.r;
    const float m = fabsf(q0);
    const int dm = (int)(__builtin_bit_cast(uint32_t, m) & 0xFFFFFu) - 0x80000;
    if (m < 0x1p-11f) return q0;
    if (m >= 0x1p-6f && m <= 0x1p16f && (dm > 4 || dm < -4)) return q0;
  }
  return __fdiv_rn(x, q.s);
}

// Value stored for new element x of kv head h: a bit copy, or for an fp8
// cache the E4M3 code of x / scale[h].
template <int KV>
struct Store;
template <>
struct Store<kF32> {
  using In = uint32_t;
  using Out = uint32_t;
  using Scale = float;
  __device__ static Out put(In x, const Scale&) { return x; }
};
template <>
struct Store<kBF16> {
  using In = uint16_t;
  using Out = uint16_t;
  using Scale = float;
  __device__ static Out put(In x, const Scale&) { return x; }
};
template <>
struct Store<kFP8> {
  using In = uint16_t;   // bf16
  using Out = uint8_t;
  using Scale = Fp8Scale;
  __device__ static float widen(In x) { return __builtin_bit_cast(float, (uint32_t)x << 16); }
  __device__ static Out put(In x, const Scale& s) { return (Out)e4m3_pair(fp8_quotient(widen(x), s), 0.f); }
  // codes of two elements: low byte x0
  __device__ static uint32_t put2(In x0, In x1, const Scale& s) {
    return e4m3_pair(fp8_quotient(widen(x0), s), fp8_quotient(widen(x1), s));
  }
};
template <int KV>
__device__ __forceinline__ typename Store<KV>::Scale store_scale(const float* scales, int h) {
  if constexpr (KV == kFP8) return fp8_scale(scales[h]);
  else return 1.f;
}

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
  using S = Store<KV>;
  const typename S::In* kn = static_cast<const typename S::In*>(a.k_new);
  const typename S::In* vn = static_cast<const typename S::In*>(a.v_new);
  typename S::Out* kp = static_cast<typename S::Out*>(a.k_pool);
  typename S::Out* vp = static_cast<typename S::Out*>(a.v_pool);
  const typename S::Scale ks = store_scale<KV>(a.k_scale, h), vs = store_scale<KV>(a.v_scale, h);
  // Non-temporal stores: the bytes go out to HBM at once.  A V column
  // touches D / (lines per block row) cache lines for D elements; left
  // cached, those partly written lines were written back later in the middle
  // of the decode's read stream and slowed it (measured on MI355X: 256
  // sequences, fp8 cache, append + decode 183.7 -> 174.5 us).
  for (int d = threadIdx.x; d < D; d += 64) {
    __builtin_nontemporal_store(S::put(kn[src + d], ks), &kp[kdst + d]);
    __builtin_nontemporal_store(S::put(vn[src + d], vs), &vp[vdst + (size_t)d * bs]);
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
  // the new tokens' K/V and the pools do not overlap
  const In* __restrict__ kn = static_cast<const In*>(a.k_new);
  const In* __restrict__ vn = static_cast<const In*>(a.v_new);
  Out* __restrict__ kp = static_cast<Out*>(a.k_pool);
  Out* __restrict__ vp = static_cast<Out*>(a.v_pool);
  const typename S::Scale ks = store_scale<KV>(a.k_scale, h), vs = store_scale<KV>(a.v_scale, h);
  const int64_t limit = (int64_t)a.num_blocks * bs;

  __shared__ int64_t slot[kGroup];
  __shared__ __attribute__((aligned(16))) Out vt[D][kGroup + 16 / sizeof(Out)];   // V transposed: [dim][token], rows padded by 16 bytes
  if (tid < kGroup) slot[tid] = tid < n ? a.slot_mapping[g0 + tid] : -1;
  __syncthreads();

  const int64_t base = slot[0];
  bool run = n == kGroup && base >= 0 && base + kGroup <= limit && (base % bs) % kGroup == 0;
  for (int k = 1; k < kGroup && run; ++k) run = slot[k] == base + k;

  // The run's stores are non-temporal (65,536 bf16 tokens: 109.9 -> 97.0 us on
  // MI355X); the element-wise scatter below keeps cached stores (4,096
  // scattered tokens: 36 us cached, 61 us non-temporal).
  if (run) {
    const int64_t blk = base / bs;
    const int off = (int)(base - blk * bs);
    const size_t tile = ((size_t)blk * Hkv + h) * bs * D;   // the (block, head) tile, in elements
    // 16-byte input vectors: kVec elements of one new token's row
    constexpr int kVec = 16 / sizeof(In);
    constexpr int kRowVecs = D / kVec;
    // Every thread's K and V input vectors are loaded first, so both loads
    // are in flight together (kGroup * kRowVecs <= 2 kAppendThreads).
    constexpr int kPer = (kGroup * kRowVecs + kAppendThreads - 1) / kAppendThreads;
    static_assert(kPer <= 2, "input vectors per thread");
    u32x4 kin[kPer], vin[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = tid + i * kAppendThreads;
      if (v < kGroup * kRowVecs) {
        const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
        const size_t src = ((size_t)(g0 + k) * Hkv + h) * D + d0;
        kin[i] = *reinterpret_cast<const u32x4*>(kn + src);
        vin[i] = *reinterpret_cast<const u32x4*>(vn + src);
      }
    }
    // K: rows off .. off+15 of the tile are kGroup * D contiguous elements
    Out* kdst = kp + tile + (size_t)off * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = tid + i * kAppendThreads;
      if (v >= kGroup * kRowVecs) break;
      const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
      const u32x4 w = kin[i];
      if constexpr (KV == kFP8) {
        const auto x = __builtin_bit_cast(typename Vec16<In>::type, w);
        const uint32_t lo = S::put2(x[0], x[1], ks) | (S::put2(x[2], x[3], ks) << 16);
        const uint32_t hi = S::put2(x[4], x[5], ks) | (S::put2(x[6], x[7], ks) << 16);
        __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(kdst + (size_t)k * D + d0));
      } else {
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(kdst + (size_t)k * D + d0));
      }
    }
    // V: element (token k, dim d) goes to row d, column off + k, through LDS
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = tid + i * kAppendThreads;
      if (v >= kGroup * kRowVecs) break;
      const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
      const u32x4 w = vin[i];
      const auto x = __builtin_bit_cast(typename Vec16<In>::type, w);
      if constexpr (KV == kFP8) {
#pragma unroll
        for (int e = 0; e < kVec; e += 2) {
          const uint32_t c = S::put2(x[e], x[e + 1], vs);
          vt[d0 + e][k] = (Out)c;
          vt[d0 + e + 1][k] = (Out)(c >> 8);
        }
      } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) vt[d0 + e][k] = S::put(x[e], vs);
      }
    }
    __syncthreads();
    // 16-byte pieces of the V rows: kOut tokens of one dim
    constexpr int kOut = 16 / sizeof(Out);
    constexpr int kRowPieces = kGroup / kOut;
    Out* vdst = vp + tile + off;
    for (int v = tid; v < D * kRowPieces; v += kAppendThreads) {
      const int d = v / kRowPieces, k0 = (v - d * kRowPieces) * kOut;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&vt[d][k0]),
                                  reinterpret_cast<u32x4*>(vdst + (size_t)d * bs + k0));
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
