// Split-K combine: merge the per-partition partial results of one (request,
// query head) into the attention output with the log-sum-exp rule.
//
// A partition p of a request holds m_p = max of its scores (log2 units),
// l_p = sum of 2^(s - m_p) and o_p = sum of 2^(s - m_p) v.  With
// M = max_p m_p the exact softmax over all positions is
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// the same normalisation and value mixture as one pass over the whole
// request (page 1 "KV cache: Generation state, latency, and allocation",
// section 21.1); only the order of additions changes.
//
// One wave per (query head, request).  Requests with a single partition were
// written by the partition kernel and are skipped.

#include "pkv_device.h"

namespace pkv {

template <int D_STEP>
__global__ __launch_bounds__(64) void combine_kernel(float* __restrict__ out,
                                                     const int32_t* __restrict__ context_lens,
                                                     Workspace ws, int H_Q, int d_h,
                                                     int partition_tokens, int max_parts) {
  extern __shared__ float w_s[];  // [max_parts] weights 2^(m_p - M) / L
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  // same partition count as the partition kernel
  const int n = context_lens[b];
  const int P = min((n + partition_tokens - 1) / partition_tokens, max_parts);
  if (P <= 1) return;
  const size_t base = (static_cast<size_t>(b) * H_Q + hq) * max_parts;

  float M = -INFINITY;
  for (int p = lane; p < P; p += 64) M = fmaxf(M, ws.ml[2 * (base + p)]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float L = 0.f;
  for (int p = lane; p < P; p += 64) {
    const float w = exp2f(ws.ml[2 * (base + p)] - M);
    w_s[p] = w;
    L = fmaf(w, ws.ml[2 * (base + p) + 1], L);
  }
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
  __syncthreads();
  const float inv = 1.0f / L;
  for (int d0 = lane * D_STEP; d0 < d_h; d0 += 64 * D_STEP) {
    float acc[D_STEP];
#pragma unroll
    for (int k = 0; k < D_STEP; ++k) acc[k] = 0.f;
    for (int p = 0; p < P; ++p) {
      const float w = w_s[p];
      const float* o = ws.o + (base + p) * d_h + d0;
#pragma unroll
      for (int k = 0; k < D_STEP; ++k) acc[k] = fmaf(w, o[k], acc[k]);
    }
    float* dst = out + (static_cast<size_t>(b) * H_Q + hq) * d_h + d0;
#pragma unroll
    for (int k = 0; k < D_STEP; ++k) dst[k] = acc[k] * inv;
  }
}

hipError_t launch_combine(float* out, const int32_t* context_lens, Workspace ws, int B, int H_Q,
                          int d_h, int partition_tokens, int max_parts, hipStream_t stream) {
  const dim3 grid(H_Q, B), block(64);
  const size_t lds = sizeof(float) * static_cast<size_t>(max_parts);
  if (d_h % 128 == 0) {
    hipLaunchKernelGGL((combine_kernel<2>), grid, block, lds, stream, out, context_lens, ws, H_Q,
                       d_h, partition_tokens, max_parts);
  } else {
    hipLaunchKernelGGL((combine_kernel<1>), grid, block, lds, stream, out, context_lens, ws, H_Q,
                       d_h, partition_tokens, max_parts);
  }
  return hipGetLastError();
}

}  // namespace pkv
