/*
 * pkv_probe.h - measurement and check kernels for MI355X (gfx950), built as
 * libpkv_probe.so.  Not part of the attention library.  The read-stream
 * ceiling probe measures how fast
 * HBM serves the access pattern of the paged decode (Habr KV-Cache article,
 * section 4: the cache's blocks lie scattered over GPU memory; "Chapter 8 -
 * Next-generation KV cache", 8.1: the kernel reaches them by indirect
 * addressing) with no arithmetic, so the decode's rate can be set against it.
 */
#ifndef PKV_PROBE_H_
#define PKV_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read num_tiles tiles of tile_kib KiB each (a power of two up to 64): tile i is the tile_kib KiB at
 * buf + tile_ids[i] * tile_kib KiB (ids past the buffer are clamped to its
 * last tile).  `waves` worker waves (a multiple of 4; 1024 is one per SIMD on
 * MI355X) each read a contiguous share of the list, 1 KiB per wave
 * instruction (16 bytes per lane), keeping kib_in_flight KiB (4, 8, 16 or 32)
 * of loads outstanding; nontemporal != 0 streams them past the caches.  Each
 * wave writes a checksum to sink[wave * 64 + lane], so sink must hold
 * waves * 64 uint32.  All pointers are device memory, 16-byte aligned.
 * Returns 0, -1 on a bad argument, -4 on a launch error.  Asynchronous on
 * `stream`. */
int pkv_probe_read_tiles(const void* buf, size_t buf_bytes, const uint32_t* tile_ids, int64_t num_tiles,
                         int32_t tile_kib, int32_t kib_in_flight, int32_t waves, int32_t nontemporal,
                         uint32_t* sink, void* stream);

/* Check of the float32 -> OCP E4M3FN conversion the append kernels use (the
 * fp8 cache format; Habr KV-Cache article, section 2: an fp8 cache stores
 * one byte per element): every binary32 bit pattern x in [first, first +
 * count) (first + count <= 2^32) is converted in both halves of the
 * kernels' two-value conversion and compared with the format's rounding
 * written out on the binary32 fields (nearest, ties to even, +-448
 * saturation, NaN kept).  Adds the number of mismatching inputs to
 * *mismatches and lowers *first_mismatch to the smallest one; both device
 * memory, initialised by the caller (0 and 0xFFFFFFFF).  Returns 0, -1 on
 * a bad argument, -4 on a launch error.  Asynchronous on `stream`. */
int pkv_probe_e4m3_check(uint64_t first, uint64_t count, unsigned long long* mismatches, uint32_t* first_mismatch,
                         void* stream);

/* The same conversion applied to n float32 values: out[i] = E4M3FN code of
 * in[i] (device memory).  Returns 0, -1 on a bad argument, -4 on a launch
 * error.  Asynchronous on `stream`. */
int pkv_probe_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H_ */
