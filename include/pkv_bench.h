/*
 * pkv_bench.h -- measurement helper of bench.py (libpkv_bench.so), not part
 * of the attention library.
 *
 * pkvb_gather_read reads n_tiles K tiles and the V tiles at the same byte
 * offsets (tile_offsets[i], int64, device memory, each a multiple of 1 KiB
 * inside both pools) of tile_bytes (4096 or 2048) each, with no arithmetic,
 * on `stream` (a hipStream_t), using `waves` single-wave workgroups that each
 * read an equal share.  It writes waves * 64 * 16 bytes of XOR checksums to
 * `sink` (device, caller-owned).  Its run time is the cost of moving the same
 * bytes as the attention step without any compute: the reference for the
 * achieved bandwidth of the attention kernel (page 3 "xf_kv_cache": decode
 * time is, to first order, cache bytes read divided by memory bandwidth).
 * Returns 0, -1 on a bad argument (nothing launched), -5 if the launch failed.
 */
#ifndef PKV_BENCH_H
#define PKV_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pkvb_gather_read(const void* k_pool, const void* v_pool, const int64_t* tile_offsets,
                     int64_t n_tiles, int32_t tile_bytes, int32_t waves, void* sink,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BENCH_H */
