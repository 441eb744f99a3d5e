// kv_append: write each request's new K and V into the slot of its newest
// position (page 1 "KV cache: Generation state, latency, and allocation",
// section 21.6, Eq. 21.6: the cache grows by appending the processed token;
// section 21.5: position t sits in logical block t / bs, slot t % bs, and the
// block table gives the physical block).
//
// Chunks of new tokens (page 1 section 21.3) use the same kernel: with a
// query_start array, row r of k_new / v_new belongs to the request b whose
// range [query_start[b], query_start[b + 1]) holds it and goes to position
// context_lens[b] - n_b + (r - query_start[b]), n_b the request's new
// tokens; without one, row b is request b's single new token.
//
// Grid (row, chunk of the row's K and V elements); each thread moves a run
// of consecutive elements of one head's row with one load and one store.  Bit copies for equal dtypes, OCP E4M3 quantisation with the
// per-(block, head) scale for fp8 caches.  A request whose slot would fall
// outside the table or the pool writes nothing.

#include "pkv_device.h"

namespace pkv {

template <int BYTES>
struct Chunk;  // an aligned run of BYTES bytes moved as one access
template <>
struct Chunk<16> {
  using type = uint4;
};
template <>
struct Chunk<8> {
  using type = uint2;
};
template <>
struct Chunk<4> {
  using type = uint32_t;
};
template <>
struct Chunk<2> {
  using type = uint16_t;
};
template <>
struct Chunk<1> {
  using type = uint8_t;
};

// EPT consecutive elements of one (K or V, head) row per thread; grid.y
// splits a request's 2 * H_KV * d_h elements into workgroup-sized chunks.
// d_h % EPT == 0, so a thread's elements never straddle two heads.
template <int IN, int KV, int EPT>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, void* __restrict__ k_cache,
    void* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    int max_blocks_per_seq, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ query_start, int B, int total_rows, int H_KV, int d_h,
    int block_size, int num_blocks) {
  constexpr int IB = IN == DT_F32 ? 4 : 2;   // input bytes per element
  constexpr int OB = KV == DT_F32 ? 4 : KV == DT_BF16 ? 2 : 1;
  const int row_id = blockIdx.x;
  int b = row_id, t;
  if (query_start) {
    b = request_of_row(query_start, B, row_id);
    const int qs0 = query_start[b], qs1 = query_start[b + 1];
    const int n = context_lens[b];
    if (qs0 < 0 || qs1 > total_rows || row_id < qs0 || row_id >= qs1 || qs1 - qs0 > n ||
        n > max_blocks_per_seq * block_size)
      return;
    t = n - (qs1 - qs0) + (row_id - qs0);
  } else {
    const int n = context_lens[b];
    if (n < 1 || n > max_blocks_per_seq * block_size) return;
    t = n - 1;
  }
  const int p = block_table[static_cast<size_t>(b) * max_blocks_per_seq + t / block_size];
  if (p < 0 || p >= num_blocks) return;
  const int r = t % block_size;
  const int row = H_KV * d_h;
  const int i = (blockIdx.y * blockDim.x + threadIdx.x) * EPT;  // first element of this thread
  if (i >= 2 * row) return;
  const bool is_v = i >= row;
  const int e = is_v ? i - row : i;
  const int h = e / d_h, d = e % d_h;
  const char* src = static_cast<const char*>(is_v ? v_new : k_new) +
                    (static_cast<size_t>(row_id) * row + e) * IB;
  char* dst = static_cast<char*>(is_v ? v_cache : k_cache) +
              (((static_cast<size_t>(p) * H_KV + h) * block_size + r) * d_h + d) * OB;
  if constexpr (IN == KV) {
    using T = typename Chunk<EPT * IB>::type;
    *reinterpret_cast<T*>(dst) = *reinterpret_cast<const T*>(src);
  } else {
    static_assert(KV == DT_FP8, "only fp8 caches convert on append");
    const float s = (is_v ? v_scale : k_scale)[static_cast<size_t>(p) * H_KV + h];
    union {
      typename Chunk<EPT * IB>::type v;
      uint16_t h16[EPT];
      float f32[EPT];
    } xin;
    xin.v = *reinterpret_cast<const typename Chunk<EPT * IB>::type*>(src);
    union {
      typename Chunk<EPT>::type v;
      uint8_t c[EPT];
    } xout;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const float x = IN == DT_F32 ? xin.f32[k] : bf16_to_f32(xin.h16[k]);
      // IEEE division (correctly rounded; the library is built without fast math)
      xout.c[k] = static_cast<uint8_t>(f32_to_e4m3(x / s));
    }
    *reinterpret_cast<typename Chunk<EPT>::type*>(dst) = xout.v;
  }
}

hipError_t launch_kv_append(int in_dtype, int kv_dtype, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const float* k_scale,
                            const float* v_scale, const int32_t* block_table,
                            int max_blocks_per_seq, const int32_t* context_lens,
                            const int32_t* query_start, int B, int rows, int H_KV, int d_h,
                            int block_size, int num_blocks, hipStream_t stream) {
  // elements per thread: a 16-byte input access where d_h and the buffers'
  // alignment allow it (4 for fp8 output from fp32), else one element
  const int in_b = in_dtype == DT_F32 ? 4 : 2;
  const int want = 16 / in_b;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                        reinterpret_cast<uintptr_t>(k_cache) |
                        reinterpret_cast<uintptr_t>(v_cache);
  const bool vec = d_h % want == 0 && (mis & 15) == 0;
  const int ept = vec ? want : 1;
  const int total = 2 * H_KV * d_h / ept;  // threads per request
  const int threads = total >= 256 ? 256 : 64;
  const dim3 grid(rows, (total + threads - 1) / threads), block(threads);
#define PKV_APPEND(IN, KV, EPT)                                                              \
  hipLaunchKernelGGL((kv_append_kernel<IN, KV, EPT>), grid, block, 0, stream, k_new, v_new,  \
                     k_cache, v_cache, k_scale, v_scale, block_table, max_blocks_per_seq,    \
                     context_lens, query_start, B, rows, H_KV, d_h, block_size, num_blocks)
#define PKV_APPEND_EPT(IN, KV, W) \
  do {                            \
    if (vec) PKV_APPEND(IN, KV, W); \
    else PKV_APPEND(IN, KV, 1);   \
  } while (0)
  if (in_dtype == DT_F32 && kv_dtype == DT_F32) PKV_APPEND_EPT(DT_F32, DT_F32, 4);
  else if (in_dtype == DT_BF16 && kv_dtype == DT_BF16) PKV_APPEND_EPT(DT_BF16, DT_BF16, 8);
  else if (in_dtype == DT_BF16 && kv_dtype == DT_FP8) PKV_APPEND_EPT(DT_BF16, DT_FP8, 8);
  else if (in_dtype == DT_F32 && kv_dtype == DT_FP8) PKV_APPEND_EPT(DT_F32, DT_FP8, 4);
  else return hipErrorInvalidValue;
#undef PKV_APPEND_EPT
#undef PKV_APPEND
  return hipGetLastError();
}

}  // namespace pkv
