// Block copies for copy-on-write (page 1 "KV cache: Generation state,
// latency, and allocation", section 21.5, the paragraph after the walk: a
// shared, partly filled block is copied before a writer changes it, so the
// other requests keep their view).
//
// One workgroup per (src, dst) pair: every stored byte of block src -- all KV
// heads, all slots, K and V -- and its fp8 scales go to block dst, in 16-byte
// chunks when the block size allows it.  Pairs whose ids fall outside the
// pool are skipped.

#include "pkv_device.h"

namespace pkv {

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                          char* __restrict__ v_cache,
                                                          float* __restrict__ k_scale,
                                                          float* __restrict__ v_scale,
                                                          const int32_t* __restrict__ pairs,
                                                          size_t block_bytes, int H_KV,
                                                          int num_blocks) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const size_t so = static_cast<size_t>(src) * block_bytes;
  const size_t dof = static_cast<size_t>(dst) * block_bytes;
  if (block_bytes % 16 == 0) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const size_t n = block_bytes / 16;
    for (size_t i = threadIdx.x; i < n; i += blockDim.x) {
      reinterpret_cast<u32x4*>(k_cache + dof)[i] = reinterpret_cast<const u32x4*>(k_cache + so)[i];
      reinterpret_cast<u32x4*>(v_cache + dof)[i] = reinterpret_cast<const u32x4*>(v_cache + so)[i];
    }
  } else {
    for (size_t i = threadIdx.x; i < block_bytes; i += blockDim.x) {
      k_cache[dof + i] = k_cache[so + i];
      v_cache[dof + i] = v_cache[so + i];
    }
  }
  if (k_scale) {
    for (int h = threadIdx.x; h < H_KV; h += blockDim.x) {
      k_scale[static_cast<size_t>(dst) * H_KV + h] = k_scale[static_cast<size_t>(src) * H_KV + h];
      v_scale[static_cast<size_t>(dst) * H_KV + h] = v_scale[static_cast<size_t>(src) * H_KV + h];
    }
  }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int n_pairs, size_t block_bytes, int H_KV,
                              int num_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs), dim3(256), 0, stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), k_scale, v_scale,
                     pairs, block_bytes, H_KV, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
