// Read-stream ceiling probe (not part of the attention path; bench.py
// --tile-probe times it).  It measures how fast HBM serves the paged
// decode's access pattern with no arithmetic: whole tiles of a few KiB read
// at random positions of a large buffer, 16 bytes per lane, a set number of
// KiB in flight per wave.  The decode reads one such tile per (block, kv
// head) for K and one for V.

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // extern "C"
