// Block swap between the device pools and a record buffer in host memory
// (page 1 "KV cache: Generation state, latency, and allocation", section
// 21.3: offloading moves retained cache state to CPU memory and a later
// operation brings the needed blocks back; page 3 "xf_kv_cache", "End-to-end
// flow": a preempted request's blocks are swapped to pinned host memory and
// copied back when it resumes).
//
// Record i of the buffer holds block blocks[i]: its K bytes ([H_KV][bs][d_h]
// as stored), its V bytes, then for fp8 caches its K and V scales ([H_KV]
// float32 each), padded to a multiple of 256 bytes (padding untouched).
// One kernel does both directions: a workgroup per (record, slice); the
// K/V bytes move in W-byte units (16 when sizes and addresses allow).  The
// buffer is read or written directly through its device mapping, so no
// staging copy is needed.  Records whose block id is out of range are
// skipped.

#include "pkv_device.h"

namespace pkv {

namespace {

template <int W>
struct Unit;
template <>
struct Unit<16> {
  using type = uint4;
};
template <>
struct Unit<4> {
  using type = uint32_t;
};
template <>
struct Unit<1> {
  using type = uint8_t;
};

}  // namespace

template <int W, bool TO_HOST>
__global__ __launch_bounds__(256) void swap_kernel(char* __restrict__ k_cache,
                                                   char* __restrict__ v_cache,
                                                   float* __restrict__ k_scale,
                                                   float* __restrict__ v_scale,
                                                   const int32_t* __restrict__ blocks,
                                                   char* __restrict__ records, size_t blk_bytes,
                                                   size_t rec_bytes, int H_KV, int num_blocks) {
  using T = typename Unit<W>::type;
  const int i = blockIdx.x;
  const int b = blocks[i];
  if (b < 0 || b >= num_blocks) return;
  char* rec = records + static_cast<size_t>(i) * rec_bytes;
  const size_t units = blk_bytes / W;  // per K or V
  for (size_t u = static_cast<size_t>(blockIdx.y) * blockDim.x + threadIdx.x; u < 2 * units;
       u += static_cast<size_t>(gridDim.y) * blockDim.x) {
    const bool is_v = u >= units;
    const size_t o = (is_v ? u - units : u) * W;
    char* pool = (is_v ? v_cache : k_cache) + static_cast<size_t>(b) * blk_bytes + o;
    char* host = rec + (is_v ? blk_bytes : 0) + o;
    if constexpr (TO_HOST) {
      *reinterpret_cast<T*>(host) = *reinterpret_cast<const T*>(pool);
    } else {
      *reinterpret_cast<T*>(pool) = *reinterpret_cast<const T*>(host);
    }
  }
  if (k_scale && blockIdx.y == 0) {
    float* hs = reinterpret_cast<float*>(rec + 2 * blk_bytes);
    for (int t = threadIdx.x; t < 2 * H_KV; t += blockDim.x) {
      float* ps = (t < H_KV ? k_scale : v_scale) + static_cast<size_t>(b) * H_KV + t % H_KV;
      if constexpr (TO_HOST) {
        hs[t] = *ps;
      } else {
        *ps = hs[t];
      }
    }
  }
}

hipError_t launch_swap(bool to_host, void* k_cache, void* v_cache, float* k_scale,
                       float* v_scale, const int32_t* blocks, int n, size_t blk_bytes,
                       size_t rec_bytes, int H_KV, int num_blocks, void* records,
                       hipStream_t stream) {
  const uintptr_t mis = reinterpret_cast<uintptr_t>(k_cache) |
                        reinterpret_cast<uintptr_t>(v_cache) |
                        reinterpret_cast<uintptr_t>(records) | blk_bytes;
  const int w = (mis & 15) == 0 ? 16 : (mis & 3) == 0 ? 4 : 1;
  const size_t units = 2 * blk_bytes / w;
  const unsigned slices = static_cast<unsigned>(std::min<size_t>((units + 255) / 256, 64));
  const dim3 grid(n, slices), block(256);
  char* k = static_cast<char*>(k_cache);
  char* v = static_cast<char*>(v_cache);
  char* r = static_cast<char*>(records);
#define PKV_SWAP(W, DIR)                                                                       \
  hipLaunchKernelGGL((swap_kernel<W, DIR>), grid, block, 0, stream, k, v, k_scale, v_scale,   \
                     blocks, r, blk_bytes, rec_bytes, H_KV, num_blocks)
  if (to_host) {
    if (w == 16) PKV_SWAP(16, true); else if (w == 4) PKV_SWAP(4, true); else PKV_SWAP(1, true);
  } else {
    if (w == 16) PKV_SWAP(16, false); else if (w == 4) PKV_SWAP(4, false); else PKV_SWAP(1, false);
  }
#undef PKV_SWAP
  return hipGetLastError();
}

}  // namespace pkv
