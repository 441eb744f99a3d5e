// Split-K combine: merge the partial results of one (request, query head)
// into the attention output with the log-sum-exp rule.
//
// A piece p of a request's positions holds m_p = max of its scores (log2
// units), l_p = sum of 2^(s - m_p) and o_p = sum of 2^(s - m_p) v.  With
// M = max_p m_p the exact softmax over all positions is
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// the same normalisation and value mixture as one pass over the whole
// request (page 1 "KV cache: Generation state, latency, and allocation",
// section 21.1); only the order of additions changes.
//
// One wave per (query head, request).  The workspace header says which
// layout the partition kernel wrote (see pkv_device.h).  Requests whose
// result the partition kernel wrote directly are skipped.

#include "pkv_device.h"

namespace pkv {

template <int D_STEP>
__global__ __launch_bounds__(64) void combine_kernel(float* __restrict__ out,
                                                     const int32_t* __restrict__ context_lens,
                                                     const char* __restrict__ ws, int H_Q,
                                                     int H_KV, int d_h, int partition_tokens,
                                                     int max_parts) {
  const int hq = blockIdx.x, b = blockIdx.y, B = gridDim.y, lane = threadIdx.x;
  const WsHeader hd = *reinterpret_cast<const WsHeader*>(ws);
  float* dst = out + (static_cast<size_t>(b) * H_Q + hq) * d_h;

  // Locate the pieces: piece k (k < P) has its (m, l) at ml + k * ml_step
  // and its o at o + k * o_step, after a per-piece base offset.
  int P = 0;
  const float* ml = nullptr;
  const float* o = nullptr;
  // flat layout: pieces come from consecutive waves, each in slot 0 except
  // the first wave's piece when that wave started in an earlier sequence
  int first_wave = 0, first_slot = 0, g = 1, j = 0;
  if (hd.mode == kWsPartition) {
    const int n = context_lens[b];
    P = min((n + partition_tokens - 1) / partition_tokens, max_parts);
    if (P <= 1) return;
    const PartitionLayout PL = partition_layout(B, H_Q, max_parts, d_h);
    const size_t base = (static_cast<size_t>(b) * H_Q + hq) * max_parts;
    ml = reinterpret_cast<const float*>(ws + PL.ml) + 2 * base;
    o = reinterpret_cast<const float*>(ws + PL.o) + base * d_h;
  } else if (hd.mode == kWsFlat) {
    const int W = hd.waves, C = hd.chunks;
    g = hd.g;
    const int h = hq / g;
    j = hq % g;
    const FlatLayout FL = flat_layout(B, W, g, d_h);
    const int32_t* prefix = reinterpret_cast<const int32_t*>(ws + FL.prefix);
    const int nb = prefix[b + 1] - prefix[b];
    if (nb <= 0) return;
    const long long T = static_cast<long long>(H_KV) * prefix[B];
    const long long S = static_cast<long long>(H_KV) * prefix[b] + static_cast<long long>(h) * nb;
    first_wave = flat_wave_of(S, T, C);
    const int last_wave = flat_wave_of(S + nb - 1, T, C);
    if (first_wave == last_wave) return;  // written final by its wave
    first_slot = flat_chunk_lo(first_wave, T, C) == S ? 0 : 1;
    P = last_wave - first_wave + 1;
    ml = reinterpret_cast<const float*>(ws + FL.ml);
    o = reinterpret_cast<const float*>(ws + FL.o);
  } else {
    return;
  }

  // piece k -> partial index in the chosen layout
  auto ml_at = [&](int k) -> const float* {
    if (hd.mode == kWsPartition) return ml + 2 * k;
    const int slot = (k == 0) ? first_slot : 0;
    return ml + 2 * ((static_cast<size_t>(first_wave + k) * 2 + slot) * g + j);
  };
  auto o_at = [&](int k) -> const float* {
    if (hd.mode == kWsPartition) return o + static_cast<size_t>(k) * d_h;
    const int slot = (k == 0) ? first_slot : 0;
    return o + ((static_cast<size_t>(first_wave + k) * 2 + slot) * g + j) * d_h;
  };

  float M = -INFINITY;
  for (int k = lane; k < P; k += 64) M = fmaxf(M, ml_at(k)[0]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float Lsum = 0.f;
  for (int k = lane; k < P; k += 64) Lsum = fmaf(exp2f(ml_at(k)[0] - M), ml_at(k)[1], Lsum);
  for (int off = 32; off > 0; off >>= 1) Lsum += __shfl_xor(Lsum, off, 64);
  const float inv = 1.0f / Lsum;

  for (int d0 = lane * D_STEP; d0 < d_h; d0 += 64 * D_STEP) {
    float acc[D_STEP];
#pragma unroll
    for (int k = 0; k < D_STEP; ++k) acc[k] = 0.f;
    for (int k = 0; k < P; ++k) {
      const float w = exp2f(ml_at(k)[0] - M);
      const float* src = o_at(k) + d0;
#pragma unroll
      for (int e = 0; e < D_STEP; ++e) acc[e] = fmaf(w, src[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < D_STEP; ++e) dst[d0 + e] = acc[e] * inv;
  }
}

hipError_t launch_combine(float* out, const int32_t* context_lens, const void* ws, int B, int H_Q,
                          int H_KV, int d_h, int partition_tokens, int max_parts,
                          hipStream_t stream) {
  const dim3 grid(H_Q, B), block(64);
  const char* w = static_cast<const char*>(ws);
  if (d_h % 128 == 0) {
    hipLaunchKernelGGL((combine_kernel<2>), grid, block, 0, stream, out, context_lens, w, H_Q,
                       H_KV, d_h, partition_tokens, max_parts);
  } else {
    hipLaunchKernelGGL((combine_kernel<1>), grid, block, 0, stream, out, context_lens, w, H_Q,
                       H_KV, d_h, partition_tokens, max_parts);
  }
  return hipGetLastError();
}

}  // namespace pkv
