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
//  - |q0| >= 2^-6: every E4M3 rounding boundary from 2^-6 up (the
//    midpoints between neighbouring codes, which keep 4 significand bits)
//    has its 20 low significand bits equal to 0x80000, and from 448 up
//    every value saturates to 448, so there is no boundary there; q0 more
//    than 4 units from that pattern lies strictly on the same side of every
//    boundary as the correctly rounded quotient.  An infinite q0 means
//    |x * r| overflowed, so both saturate.
// Otherwise (the E4M3 subnormal range, near a boundary, NaN, or a scale
// whose reciprocal is not a normal number) the quotient is the IEEE division
// itself.  For most scales the fast case replaces a division sequence by one
// multiply in all but a few inputs in 10^4.
struct Fp8Scale {
  float s, r;
  bool fast;
};
__device__ __forceinline__ Fp8Scale fp8_scale(float s) {
  return Fp8Scale{s, __fdiv_rn(1.f, s), s >= 0x1p-125f && s <= 0x1p125f};
}
// Whether the product q0 = x * (1/s) rounds to the same E4M3 code as the IEEE
// quotient x / s: one of the two cases above.  False for NaN.
__device__ __forceinline__ bool fp8_product_ok(float q0) {
  const float m = fabsf(q0);
  // the 20 low significand bits minus 0x7FFFC, modulo 2^20: at most 8
  // exactly when they lie within 4 units of 0x80000
  const uint32_t near = (__builtin_bit_cast(uint32_t, q0) - 0x7FFFCu) & 0xFFFFFu;
  const bool tiny = m < 0x1p-11f, normal = m >= 0x1p-6f, far = near > 8u;
  return tiny | (normal & far);   // no branches: all three are cheap
}
__device__ __forceinline__ float fp8_quotient(float x, const Fp8Scale& q) {
  if (q.fast) {
    const float q0 = x * q.r;
    if (fp8_product_ok(q0)) return q0;
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
  // codes of the eight elements of a 16-byte input vector, byte e for
  // element e: fp8_quotient's codes, with the test of all eight products
  // made first and the division then taken only for the elements that
  // failed it (a branch per element that the wave skips when no lane
  // needs it).  Such elements are not rare for every scale: with
  // s = 4/448, for one, every bf16 input with significand 1.5 gives a
  // product on a rounding boundary.
  __device__ static u32x2 put8(u32x4 w, const Scale& s) {
    float x[8], q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = widen((In)(w[e >> 1] >> (16 * (e & 1))));
    if (s.fast) {   // the same for every lane: one scale per kv head
      bool bad[8];
      bool any = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        q[e] = x[e] * s.r;
        bad[e] = !fp8_product_ok(q[e]);
        any |= bad[e];
      }
      if (any) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (bad[e]) {
            // an empty asm statement keeps the division inside its branch
            // (the compiler would otherwise compute all eight for every
            // lane and select)
            asm volatile("");
            q[e] = __fdiv_rn(x[e], s.s);
          }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = __fdiv_rn(x[e], s.s);
    }
    return u32x2{e4m3_quad(q[0], q[1], q[2], q[3]), e4m3_quad(q[4], q[5], q[6], q[7])};
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
  using S = Store<KV>;
  const int item = blockIdx.x;
  const int i = item / a.num_kv_heads;
  const int h = item % a.num_kv_heads;
  const typename S::In* kn = static_cast<const typename S::In*>(a.k_new);
  const typename S::In* vn = static_cast<const typename S::In*>(a.v_new);
  typename S::Out* kp = static_cast<typename S::Out*>(a.k_pool);
  typename S::Out* vp = static_cast<typename S::Out*>(a.v_pool);
  // The token's K and V rows do not depend on its slot: they are loaded
  // first, so that their loads and the slot's are in flight together.
  const size_t src = ((size_t)i * a.num_kv_heads + h) * D;
  constexpr int kPer = D / 64;
  typename S::In kx[kPer], vx[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    kx[j] = kn[src + threadIdx.x + 64 * j];
    vx[j] = vn[src + threadIdx.x + 64 * j];
  }
  const typename S::Scale ks = store_scale<KV>(a.k_scale, h), vs = store_scale<KV>(a.v_scale, h);
  // keeps the compiler from moving those loads below the padding test
  asm volatile("" ::: "memory");
  const int64_t slot = a.slot_mapping[i];
  const int bs = a.block_size;
  if (slot < 0 || slot >= (int64_t)a.num_blocks * bs) return;  // padding
  const int64_t blk = slot >> __builtin_ctz(bs);   // block sizes are powers of two
  const int off = (int)(slot & (bs - 1));
  const size_t ktile = ((size_t)blk * a.num_kv_heads + h) * bs * D;
  const size_t kdst = ktile + (size_t)off * D;     // token-major: row `off`
  const size_t vdst = ktile + off;                 // dim-major: column `off`
  // Non-temporal stores: the bytes go out to HBM at once.  A V column
  // touches D / (lines per block row) cache lines for D elements; left
  // cached, those partly written lines were written back later in the middle
  // of the decode's read stream and slowed it (measured on MI355X: 256
  // sequences, fp8 cache, append + decode 183.7 -> 174.5 us).
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = threadIdx.x + 64 * j;
    __builtin_nontemporal_store(S::put(kx[j], ks), &kp[kdst + d]);
    __builtin_nontemporal_store(S::put(vx[j], vs), &vp[vdst + (size_t)d * bs]);
  }
}

constexpr int kGroup = 16;          // new tokens per group
constexpr int kAppendThreads = 256;
// Workgroups of the tiled kernel for an fp8 cache, over all kv heads, each
// walking its share of the 16-token groups (65,536 tokens, 8 kv heads on
// MI355X: 2,048 workgroups 95.4 us, 3,072 89.3, 4,096 85.5, 8,192 88.0).
constexpr int kAppendWorkgroups = 4096;

// One 16-token group's inputs as one wave holds them: lane k < 16 has token
// k's slot (-1 past the last token), and each thread kPer 16-byte vectors
// of the group's K and V rows.
template <int KV, int D>
struct AppendGroup {
  using In = typename Store<KV>::In;
  static constexpr int kVec = 16 / sizeof(In);   // elements per input vector
  static constexpr int kRowVecs = D / kVec;
  static constexpr int kVecs = kGroup * kRowVecs;
  static constexpr int kPer = (kVecs + kAppendThreads - 1) / kAppendThreads;
  static_assert(kPer <= 2, "input vectors per thread");
  int64_t my_slot;
  u32x4 kin[kPer], vin[kPer];
};

template <int KV, int D>
__device__ __forceinline__ void load_group(AppendGroup<KV, D>& G, const AppendArgs& a, int g0, int h,
                                           int tid) {
  using AG = AppendGroup<KV, D>;
  using In = typename AG::In;
  const In* __restrict__ kn = static_cast<const In*>(a.k_new);
  const In* __restrict__ vn = static_cast<const In*>(a.v_new);
  const int n = min(kGroup, a.num_tokens - g0);
  const int lane = tid & 63;
  // Every load is made, on clamped indices where the group is short (its
  // extra values are never stored), so that the number of loads issued is
  // the same on every path: the compiler can then wait for one group's
  // loads while the next group's are still in flight.
  const int64_t sl = a.slot_mapping[g0 + min(lane, n - 1)];
  G.my_slot = lane < n ? sl : -1;
#pragma unroll
  for (int i = 0; i < AG::kPer; ++i) {
    const int v = min(tid + i * kAppendThreads, AG::kVecs - 1);
    const int k = min(v / AG::kRowVecs, n - 1), d0 = (v % AG::kRowVecs) * AG::kVec;
    const size_t src = ((size_t)(g0 + k) * a.num_kv_heads + h) * D + d0;
    G.kin[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kn + src));
    G.vin[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vn + src));
  }
}

// Each workgroup takes kv head blockIdx.y and the 16-token groups
// blockIdx.x, blockIdx.x + gridDim.x, ...; the next group's inputs are
// loaded before the current group is converted and stored, so each wave
// keeps loads in flight while it computes.  Each 16-byte input vector of a
// token's K goes to its slot's K row as one piece.  When the 16 tokens'
// slots are 16 consecutive rows of one block (a prefill chunk's appends),
// those K rows are one contiguous run of the block's K tile and the V
// columns 16-token pieces of every row of its V tile: V is transposed
// through LDS and written row by row.  Any other slots (one token per
// sequence in a decode step, padding, a run that crosses a block) get their
// V columns element by element.
template <int KV, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  using S = Store<KV>;
  using In = typename S::In;
  using Out = typename S::Out;
  using AG = AppendGroup<KV, D>;
  constexpr int kVec = AG::kVec, kRowVecs = AG::kRowVecs, kVecs = AG::kVecs, kPer = AG::kPer;
  const int h = blockIdx.y;
  const int Hkv = a.num_kv_heads;
  const int bs = a.block_size;
  const int bshift = __builtin_ctz(bs);   // block sizes are powers of two
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int groups = (a.num_tokens + kGroup - 1) / kGroup;
  Out* __restrict__ kp = static_cast<Out*>(a.k_pool);
  Out* __restrict__ vp = static_cast<Out*>(a.v_pool);
  const int64_t limit = (int64_t)a.num_blocks * bs;
  const typename S::Scale ks = store_scale<KV>(a.k_scale, h), vs = store_scale<KV>(a.v_scale, h);

  // A group's V in LDS.  For a run: transposed, [dim][token], each row
  // padded by one 4-byte word, which spreads a wave's element writes over
  // the LDS banks; otherwise as it is, [token][dim].  Two buffers, used by
  // turns from one group to the next: the barrier between a group's LDS
  // writes and reads then also orders the previous group's reads of the
  // other buffer before that buffer's next writes.
  constexpr int kPitch = kGroup * (int)sizeof(Out) / 4 + 1;   // words per row
  constexpr int kPitchE = kPitch * 4 / (int)sizeof(Out);      // elements per row
  static_assert(D * kPitch >= kGroup * D * (int)sizeof(Out) / 4, "a group's V fits a buffer");
  __shared__ __attribute__((aligned(16))) uint32_t vt_buf[2][D * kPitch];
  int turn = 0;   // groups that used LDS so far

  // converts and stores one group
  auto process = [&](const AG& cur, int g) {
    const int n = min(kGroup, a.num_tokens - g * kGroup);

    // K: token k's row goes to row `off` of its slot's block tile, one
    // 16-byte input vector (8 bytes of E4M3 codes) per store; token k's
    // slot comes from lane k.  Non-temporal: the bytes go out to HBM at once
    // (65,536 bf16 tokens into consecutive slots: 109.9 -> 97.0 us on MI355X).
    int64_t sl[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = tid + i * kAppendThreads;
      const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
      sl[i] = (int64_t)(uint32_t)__shfl((int)(uint32_t)cur.my_slot, k) |
              ((int64_t)__shfl((int)((uint64_t)cur.my_slot >> 32), k) << 32);
      if (v >= kVecs || k >= n || sl[i] < 0 || sl[i] >= limit) {   // padding
        sl[i] = -1;
        continue;
      }
      const size_t tile = ((size_t)(sl[i] >> bshift) * Hkv + h) * bs * D;
      Out* kd = kp + tile + (size_t)(sl[i] & (bs - 1)) * D + d0;
      if constexpr (KV == kFP8) {
        __builtin_nontemporal_store(S::put8(cur.kin[i], ks), reinterpret_cast<u32x2*>(kd));
      } else {
        __builtin_nontemporal_store(cur.kin[i], reinterpret_cast<u32x4*>(kd));
      }
    }

    // run: 16 tokens, slots base .. base + 15 inside the pool, base on a
    // 16-row boundary of its block (block sizes are powers of two from 16,
    // so all 16 rows lie in that block)
    const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)cur.my_slot) |
                         ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)cur.my_slot >> 32)) << 32);
    const bool in_run = lane >= kGroup || cur.my_slot == base + lane;
    const bool run = n == kGroup && base >= 0 && base + kGroup <= limit && (base & (kGroup - 1)) == 0 &&
                     __builtin_amdgcn_ballot_w64(!in_run) == 0;

    if (run) {
      // V columns off .. off+15 of every row of the tile, through LDS, then
      // written as 16-byte pieces of the rows, non-temporal like K
      const int off = (int)(base & (bs - 1));
      const size_t tile = ((size_t)(base >> bshift) * Hkv + h) * bs * D;
      uint32_t* vt = vt_buf[turn & 1];
      ++turn;
      Out* vte = reinterpret_cast<Out*>(vt);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int v = tid + i * kAppendThreads;
        if (v >= kVecs) break;
        const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
        if constexpr (KV == kFP8) {
          const u32x2 c = S::put8(cur.vin[i], vs);
#pragma unroll
          for (int e = 0; e < kVec; ++e) vte[(d0 + e) * kPitchE + k] = (Out)(c[e >> 2] >> (8 * (e & 3)));
        } else {
          const auto x = __builtin_bit_cast(typename Vec16<In>::type, cur.vin[i]);
#pragma unroll
          for (int e = 0; e < kVec; ++e) vte[(d0 + e) * kPitchE + k] = x[e];
        }
      }
      __syncthreads();
      constexpr int kOut = 16 / sizeof(Out);   // tokens per 16-byte piece
      constexpr int kRowPieces = kGroup / kOut;
      Out* vdst = vp + tile + off;
      for (int v = tid; v < D * kRowPieces; v += kAppendThreads) {
        const int d = v / kRowPieces, k0 = (v - d * kRowPieces) * kOut;
        const uint32_t* r = vt + d * kPitch + k0 * (int)sizeof(Out) / 4;
        __builtin_nontemporal_store(u32x4{r[0], r[1], r[2], r[3]},
                                    reinterpret_cast<u32x4*>(vdst + (size_t)d * bs + k0));
      }
    } else {
      // V scatter: the group's V rows go to LDS as they are ([token][dim]),
      // then each token's column is written element by element with
      // consecutive lanes on consecutive dims, so one store instruction
      // covers a run of rows of one tile (a few cache lines) rather than
      // rows of several tiles; cached stores (4,096 scattered tokens: 36 us
      // cached, 61 us non-temporal on MI355X).
      uint32_t* vt = vt_buf[turn & 1];
      ++turn;
      Out* vte = reinterpret_cast<Out*>(vt);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int v = tid + i * kAppendThreads;
        if (v >= kVecs) break;
        const int k = v / kRowVecs, d0 = (v - k * kRowVecs) * kVec;
        if constexpr (KV == kFP8) {
          *reinterpret_cast<u32x2*>(vte + k * D + d0) = S::put8(cur.vin[i], vs);
        } else {
          *reinterpret_cast<u32x4*>(vte + k * D + d0) = cur.vin[i];
        }
      }
      __syncthreads();
      // D is 64 or 128: the token of element e = tid + 256 j is the same
      // across a wave, so its slot is read from that lane of the wave
      for (int e = tid; e < n * D; e += kAppendThreads) {
        const int k = __builtin_amdgcn_readfirstlane(e / D), d = e - k * D;
        const int64_t slk =
            (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)cur.my_slot, k) |
            ((int64_t)__builtin_amdgcn_readlane((int)((uint64_t)cur.my_slot >> 32), k) << 32);
        if (slk < 0 || slk >= limit) continue;   // padding
        const size_t tile = ((size_t)(slk >> bshift) * Hkv + h) * bs * D;
        vp[tile + (size_t)d * bs + (slk & (bs - 1))] = vte[k * D + d];
      }
    }
  };

  // The loop's loads are unconditional (the last group is taken after it),
  // which keeps the next group's loads in flight during process().
  int g = blockIdx.x;
  AG cur;
  load_group(cur, a, g * kGroup, h, tid);
  for (; g + (int)gridDim.x < groups; g += (int)gridDim.x) {
    AG nxt;
    load_group(nxt, a, (g + (int)gridDim.x) * kGroup, h, tid);
    process(cur, g);
    cur = nxt;
  }
  process(cur, g);
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
    const int groups = (a.num_tokens + kGroup - 1) / kGroup;
    // A bit copy has little to overlap with its loads: one group per
    // workgroup (65,536 bf16 tokens: 89.4 us, against 95.5 with 2,048
    // workgroups).  The fp8 quantiser's arithmetic is worth overlapping.
    const int per_head = KV == kFP8 ? max(1, kAppendWorkgroups / a.num_kv_heads) : groups;
    const dim3 grid((unsigned)min(groups, per_head), (unsigned)a.num_kv_heads);
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
