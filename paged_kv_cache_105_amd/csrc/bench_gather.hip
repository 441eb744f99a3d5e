// Measurement kernel (not part of the attention path): read a list of K/V
// tiles once, with no arithmetic, to measure what a pure gather of the same
// bytes achieves on this device.  bench.py passes the tiles the attention
// step reads (every (request, KV head, block) of the batch), so the figure is
// the ceiling for that access pattern and size.
//
// Wave w reads tiles [floor(w n / W), floor((w + 1) n / W)), two tiles (K
// and V of each) in flight, non-temporal loads like the attention kernel,
// and XORs what it read into sink[w][lane] so no load is dead.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_bench.h"

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CHUNKS>  // 16-byte chunks per lane per tile: 4 = 4 KiB tiles, 2 = 2 KiB
__global__ __launch_bounds__(64) void gather_kernel(const char* __restrict__ kp,
                                                    const char* __restrict__ vp,
                                                    const int64_t* __restrict__ offs,
                                                    int64_t n, u32x4* __restrict__ sink) {
  const int w = blockIdx.x, W = gridDim.x, lane = threadIdx.x;
  const int64_t lo = static_cast<int64_t>(w) * n / W, hi = static_cast<int64_t>(w + 1) * n / W;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = lo;
  for (; i + 2 <= hi; i += 2) {
    u32x4 r[2][2 * CHUNKS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t o = offs[i + u];
#pragma unroll
      for (int s = 0; s < CHUNKS; ++s) {
        r[u][s] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kp + o + s * 1024 + lane * 16));
        r[u][CHUNKS + s] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vp + o + s * 1024 + lane * 16));
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int s = 0; s < 2 * CHUNKS; ++s) acc ^= r[u][s];
  }
  for (; i < hi; ++i) {
    const int64_t o = offs[i];
#pragma unroll
    for (int s = 0; s < CHUNKS; ++s) {
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + o + s * 1024 + lane * 16));
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + o + s * 1024 + lane * 16));
    }
  }
  sink[static_cast<size_t>(w) * 64 + lane] = acc;
}
}  // namespace

extern "C" int pkvb_gather_read(const void* k_pool, const void* v_pool, const int64_t* tile_offsets,
                                int64_t n_tiles, int32_t tile_bytes, int32_t waves, void* sink,
                                void* stream) {
  if (!k_pool || !v_pool || !tile_offsets || !sink || n_tiles < 1 || waves < 1 ||
      (tile_bytes != 4096 && tile_bytes != 2048))
    return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const char* k = static_cast<const char*>(k_pool);
  const char* v = static_cast<const char*>(v_pool);
  u32x4* o = static_cast<u32x4*>(sink);
  if (tile_bytes == 4096) {
    hipLaunchKernelGGL(gather_kernel<4>, dim3(waves), dim3(64), 0, s, k, v, tile_offsets, n_tiles, o);
  } else {
    hipLaunchKernelGGL(gather_kernel<2>, dim3(waves), dim3(64), 0, s, k, v, tile_offsets, n_tiles, o);
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
