// kv_append: write each request's new K and V into the slot of its newest
// position (page 1 "KV cache: Generation state, latency, and allocation",
// section 21.6, Eq. 21.6: the cache grows by appending the processed token;
// section 21.5: position t sits in logical block t / bs, slot t % bs, and the
// block table gives the physical block).
//
// One workgroup per request, one thread per (KV head, element) pair of the
// K or V row.  Bit copies for equal dtypes, OCP E4M3 quantisation with the
// per-(block, head) scale for fp8 caches.  A request whose slot would fall
// outside the table or the pool writes nothing.

#include "pkv_device.h"

namespace pkv {

template <int IN, int KV>
__global__ void kv_append_kernel(const void* __restrict__ k_new, const void* __restrict__ v_new,
                                 void* __restrict__ k_cache, void* __restrict__ v_cache,
                                 const float* __restrict__ k_scale,
                                 const float* __restrict__ v_scale,
                                 const int32_t* __restrict__ block_table, int max_blocks_per_seq,
                                 const int32_t* __restrict__ context_lens, int H_KV, int d_h,
                                 int block_size, int num_blocks) {
  const int b = blockIdx.x;
  const int n = context_lens[b];
  if (n < 1 || n > max_blocks_per_seq * block_size) return;
  const int t = n - 1;
  const int p = block_table[static_cast<size_t>(b) * max_blocks_per_seq + t / block_size];
  if (p < 0 || p >= num_blocks) return;
  const int r = t % block_size;
  const int row = H_KV * d_h;
  for (int i = threadIdx.x; i < 2 * row; i += blockDim.x) {
    const bool is_v = i >= row;
    const int e = is_v ? i - row : i;
    const int h = e / d_h, d = e % d_h;
    const void* src = is_v ? v_new : k_new;
    void* dst = is_v ? v_cache : k_cache;
    const size_t si = static_cast<size_t>(b) * row + e;
    const size_t di = ((static_cast<size_t>(p) * H_KV + h) * block_size + r) * d_h + d;
    if constexpr (IN == KV) {
      if constexpr (KV == DT_F32) {
        static_cast<uint32_t*>(dst)[di] = static_cast<const uint32_t*>(src)[si];
      } else {
        static_cast<uint16_t*>(dst)[di] = static_cast<const uint16_t*>(src)[si];
      }
    } else {
      static_assert(KV == DT_FP8, "only fp8 caches convert on append");
      const float x = load_elem<IN>(src, si);
      const float s = (is_v ? v_scale : k_scale)[static_cast<size_t>(p) * H_KV + h];
      // IEEE division (correctly rounded; the library is built without fast math)
      static_cast<uint8_t*>(dst)[di] = static_cast<uint8_t>(f32_to_e4m3(x / s));
    }
  }
}

hipError_t launch_kv_append(int in_dtype, int kv_dtype, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const float* k_scale,
                            const float* v_scale, const int32_t* block_table,
                            int max_blocks_per_seq, const int32_t* context_lens, int B, int H_KV,
                            int d_h, int block_size, int num_blocks, hipStream_t stream) {
  const int threads = 2 * H_KV * d_h >= 256 ? 256 : 64;
  const dim3 grid(B), block(threads);
#define PKV_APPEND(IN, KV)                                                                    \
  hipLaunchKernelGGL((kv_append_kernel<IN, KV>), grid, block, 0, stream, k_new, v_new,        \
                     k_cache, v_cache, k_scale, v_scale, block_table, max_blocks_per_seq,     \
                     context_lens, H_KV, d_h, block_size, num_blocks)
  if (in_dtype == DT_F32 && kv_dtype == DT_F32) PKV_APPEND(DT_F32, DT_F32);
  else if (in_dtype == DT_BF16 && kv_dtype == DT_BF16) PKV_APPEND(DT_BF16, DT_BF16);
  else if (in_dtype == DT_BF16 && kv_dtype == DT_FP8) PKV_APPEND(DT_BF16, DT_FP8);
  else if (in_dtype == DT_F32 && kv_dtype == DT_FP8) PKV_APPEND(DT_F32, DT_FP8);
  else return hipErrorInvalidValue;
#undef PKV_APPEND
  return hipGetLastError();
}

}  // namespace pkv
