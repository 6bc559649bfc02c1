// Measurement and check kernels beside the attention library (not part of
// its path).  (1) The read-stream ceiling probe (bench.py --tile-probe times
// it).  It measures how fast HBM serves the paged
// decode's access pattern with no arithmetic: whole tiles of a few KiB read
// at random positions of a large buffer, 16 bytes per lane, a set number of
// KiB in flight per wave.  The decode reads one such tile per (block, kv
// head) for K and one for V.  (2) A check of the float32 -> E4M3 conversion
// the append kernels use (e4m3.h) on every binary32 input, and that
// conversion on a caller's array, for comparison with the CPU oracle.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e4m3.h"
#include "pkv_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

// The work is a list of 1 KiB pieces: piece p is KiB (p mod tile_kib) of
// tile ids[p / tile_kib] (tile_kib = 2^tile_shift).  Wave w reads pieces [w * per, (w + 1) * per) in
// groups of kInst (one wave instruction each); the next group's loads are
// issued before the current group is folded into the checksum, so about
// kInst KiB stay in flight.  Tile ids are clamped into the buffer.
template <bool NT, int kInst>
__global__ __launch_bounds__(256) void read_tiles_kernel(const uint8_t* __restrict__ buf,
                                                        const uint32_t* __restrict__ ids, int64_t pieces,
                                                        int32_t tile_shift, int64_t buf_tiles, int64_t per,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t p0 = wave * per;
  const int64_t p1 = p0 + per < pieces ? p0 + per : pieces;
  const int64_t in_tile = ((int64_t)1 << tile_shift) - 1;
  auto tile_of = [&](int64_t p) -> uint32_t {   // a scalar load (p is the same for the whole wave)
    const uint32_t id = ids[p >> tile_shift];
    return id < buf_tiles ? id : (uint32_t)(buf_tiles - 1);
  };
  auto addr = [&](uint32_t id, int64_t p) -> const uint8_t* {
    return buf + ((size_t)id << (tile_shift + 10)) + ((size_t)(p & in_tile) << 10) + lane * 16;
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 cur[kInst], nxt[kInst];
  uint32_t id_next[kInst];   // tile ids of the next group, fetched one group ahead (as the decode does)
  int64_t p = p0;
  const int64_t full = p0 + (p1 - p0) / kInst * kInst;   // pieces in whole groups
  if (p < full) {
#pragma unroll
    for (int i = 0; i < kInst; ++i) cur[i] = ld<NT>(addr(tile_of(p + i), p + i));
    p += kInst;
#pragma unroll
    for (int i = 0; i < kInst; ++i) id_next[i] = p < full ? tile_of(p + i) : 0u;
    for (; p < full; p += kInst) {
#pragma unroll
      for (int i = 0; i < kInst; ++i) nxt[i] = ld<NT>(addr(id_next[i], p + i));
      if (p + kInst < full) {
#pragma unroll
        for (int i = 0; i < kInst; ++i) id_next[i] = tile_of(p + kInst + i);
      }
#pragma unroll
      for (int i = 0; i < kInst; ++i) acc ^= cur[i];
#pragma unroll
      for (int i = 0; i < kInst; ++i) cur[i] = nxt[i];
    }
#pragma unroll
    for (int i = 0; i < kInst; ++i) acc ^= cur[i];
  }
  for (; p < p1; ++p) acc ^= ld<NT>(addr(tile_of(p), p));
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (p0 < pieces) sink[wave * 64 + lane] = v;
}

template <bool NT>
hipError_t launch_nt(const uint8_t* buf, const uint32_t* ids, int64_t pieces, int32_t tile_shift, int64_t buf_tiles,
                     int64_t per, int32_t inst, unsigned grid, uint32_t* sink, hipStream_t s) {
  switch (inst) {
    case 4: hipLaunchKernelGGL((read_tiles_kernel<NT, 4>), dim3(grid), dim3(256), 0, s, buf, ids, pieces, tile_shift, buf_tiles, per, sink); break;
    case 8: hipLaunchKernelGGL((read_tiles_kernel<NT, 8>), dim3(grid), dim3(256), 0, s, buf, ids, pieces, tile_shift, buf_tiles, per, sink); break;
    case 16: hipLaunchKernelGGL((read_tiles_kernel<NT, 16>), dim3(grid), dim3(256), 0, s, buf, ids, pieces, tile_shift, buf_tiles, per, sink); break;
    case 32: hipLaunchKernelGGL((read_tiles_kernel<NT, 32>), dim3(grid), dim3(256), 0, s, buf, ids, pieces, tile_shift, buf_tiles, per, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// OCP E4M3FN rounding of a binary32 value written out from the format in
// integer arithmetic: sign kept; NaN -> 0x7F; magnitudes >= 448 (infinities
// included) -> 448 (0x7E); otherwise the nearest multiple, ties to even, of
// the spacing 2^(E - 3) of the value's binade E (E = -6 for everything
// below 2^-6: the subnormal grid), code (E + 7) * 8 + steps - 8, so a
// round-up across a binade edge lands on the next exponent's first code.
__device__ __forceinline__ uint32_t e4m3_fields(uint32_t x) {
  const uint32_t s = (x >> 24) & 0x80u;
  const uint32_t a = x & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return s | 0x7Fu;     // NaN
  if (a >= 0x43E00000u) return s | 0x7Eu;    // 448 = 1.75 * 2^8 and above
  const int ef = (int)(a >> 23);
  const uint64_t m = (a & 0x7FFFFFu) | (ef ? 0x800000u : 0u);   // value = m * 2^(e - 23)
  const int e = ef ? ef - 127 : -126;
  const int bin = e < -6 ? -6 : e;
  const int sh = 20 + bin - e;               // steps = m / 2^sh (>= 20)
  uint64_t q = 0;
  if (sh <= 40) {                            // else the value is below 2^-17 spacings: 0
    q = m >> sh;
    const uint64_t rem = m & ((uint64_t(1) << sh) - 1), half = uint64_t(1) << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
  }
  return s | (uint32_t)((bin + 7) * 8 + (int)q - 8);
}

// Every input x in [first, first + count) (as binary32 bit patterns) through
// e4m3_pair in both halves of the pair and through e4m3_quad in each of its
// four places, against e4m3_fields; e4m3_quad's other three values are 1.0
// (code 0x38) and then NaN with the sign bit set (code 0xFF), which must keep
// their codes.  Mismatches are counted, and the smallest mismatching x kept.
__global__ __launch_bounds__(256) void e4m3_check_kernel(uint64_t first, uint64_t count,
                                                         unsigned long long* __restrict__ bad,
                                                         uint32_t* __restrict__ first_bad) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint32_t x = (uint32_t)(first + i);
    const float f = __builtin_bit_cast(float, x);
    const uint32_t want = e4m3_fields(x);
    const uint32_t lo = pkv::e4m3_pair(f, 0.f) & 0xFFu;
    const uint32_t hi = (pkv::e4m3_pair(0.f, f) >> 8) & 0xFFu;
    bool quad_ok = true;
    const float nan = __builtin_bit_cast(float, 0xFFC00000u);
#pragma unroll
    for (int other = 0; other < 2; ++other) {
      const float o = other ? nan : 1.f;
      const uint32_t oc = other ? 0xFFu : 0x38u;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t got = pkv::e4m3_quad(p == 0 ? f : o, p == 1 ? f : o, p == 2 ? f : o, p == 3 ? f : o);
        const uint32_t expect = (oc * 0x01010101u & ~(0xFFu << (8 * p))) | (want << (8 * p));
        quad_ok &= got == expect;
      }
    }
    if (lo != want || hi != want || !quad_ok) {
      atomicAdd(bad, 1ull);
      atomicMin(first_bad, x);
    }
  }
}

__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)(pkv::e4m3_pair(in[i], 0.f) & 0xFFu);
}

}  // namespace

extern "C" {

int pkv_probe_read_tiles(const void* buf, size_t buf_bytes, const uint32_t* tile_ids, int64_t num_tiles,
                         int32_t tile_kib, int32_t kib_in_flight, int32_t waves, int32_t nontemporal,
                         uint32_t* sink, void* stream) {
  if (!buf || !tile_ids || !sink || num_tiles <= 0 || waves <= 0 || waves % 4 != 0) return -1;
  int tile_shift = 0;
  while (tile_shift <= 6 && (1 << tile_shift) != tile_kib) ++tile_shift;
  if (tile_shift > 6 || buf_bytes < ((size_t)tile_kib << 10)) return -1;   // 1, 2, 4, ... 64 KiB
  if (kib_in_flight != 4 && kib_in_flight != 8 && kib_in_flight != 16 && kib_in_flight != 32) return -1;
  const int64_t pieces = num_tiles * tile_kib;
  const int64_t per = (pieces + waves - 1) / waves;
  const int64_t buf_tiles = (int64_t)(buf_bytes / ((size_t)tile_kib << 10));
  const unsigned grid = (unsigned)(waves / 4);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = nontemporal ? launch_nt<true>(b, tile_ids, pieces, tile_shift, buf_tiles, per, kib_in_flight, grid, sink, s)
                                   : launch_nt<false>(b, tile_ids, pieces, tile_shift, buf_tiles, per, kib_in_flight, grid, sink, s);
  return e == hipSuccess ? 0 : -4;
}

int pkv_probe_e4m3_check(uint64_t first, uint64_t count, unsigned long long* mismatches, uint32_t* first_mismatch,
                         void* stream) {
  if (!mismatches || !first_mismatch || count == 0 || count > (uint64_t(1) << 32) ||
      first + count > (uint64_t(1) << 32))
    return -1;
  hipLaunchKernelGGL(e4m3_check_kernel, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), first, count,
                     mismatches, first_mismatch);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int pkv_probe_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (!in || !out || n <= 0 || n > (int64_t(1) << 40)) return -1;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(e4m3_encode_kernel, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream), in,
                     out, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
