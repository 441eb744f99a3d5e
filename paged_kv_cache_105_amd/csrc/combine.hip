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

constexpr int kChunk = 1024;   // piece weights held in LDS at a time
constexpr int kMaxStep = 4;    // output elements per lane: d_h <= 256 = 64 lanes x 4

template <int D_STEP>
__global__ __launch_bounds__(64) void combine_kernel(float* __restrict__ out,
                                                     const int32_t* __restrict__ context_lens,
                                                     const char* __restrict__ ws, int H_Q,
                                                     int H_KV, int d_h, int partition_tokens,
                                                     int max_parts) {
  __shared__ float w_s[kChunk];
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

  // piece k -> its (m, l) pair and its o row in the chosen layout
  size_t ml_step = 2, o_step = d_h;  // partition layout: pieces are contiguous
  size_t ml_first = 0, o_first = 0;  // offset of piece 0 when it sits in another slot
  if (hd.mode == kWsFlat) {
    // piece k > 0 lives in slot 0 of wave first_wave + k; piece 0 in first_slot
    const size_t base = (static_cast<size_t>(first_wave) * 2) * g + j;
    ml += 2 * base;
    o += base * d_h;
    ml_step = 2 * 2 * static_cast<size_t>(g);
    o_step = 2 * static_cast<size_t>(g) * d_h;
    ml_first = 2 * static_cast<size_t>(first_slot) * g;
    o_first = static_cast<size_t>(first_slot) * g * d_h;
  }
  auto ml_at = [&](int k) { return ml + k * ml_step + (k == 0 ? ml_first : 0); };
  auto o_at = [&](int k) { return o + k * o_step + (k == 0 ? o_first : 0); };

  // pass 1 (lane-parallel): M = max_k m_k and L = sum_k 2^(m_k - M) l_k
  float M = -INFINITY;
  for (int k = lane; k < P; k += 64) M = fmaxf(M, ml_at(k)[0]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float Lsum = 0.f;
  for (int k = lane; k < P; k += 64) Lsum = fmaf(exp2f(ml_at(k)[0] - M), ml_at(k)[1], Lsum);
  for (int off = 32; off > 0; off >>= 1) Lsum += __shfl_xor(Lsum, off, 64);
  const float inv = 1.0f / Lsum;

  // pass 2: weights of up to kChunk pieces at a time in LDS, then every lane
  // sums its output elements over the chunk with independent loads
  constexpr int R = kMaxStep / D_STEP;  // element groups per lane (static: acc stays in VGPRs)
  float acc[kMaxStep];
#pragma unroll
  for (int e = 0; e < kMaxStep; ++e) acc[e] = 0.f;
  const int d0 = lane * D_STEP;
  for (int k0 = 0; k0 < P; k0 += kChunk) {
    const int kn = min(kChunk, P - k0);
    for (int k = lane; k < kn; k += 64) w_s[k] = exp2f(ml_at(k0 + k)[0] - M) * inv;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the weights are in LDS
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int d = d0 + r * 64 * D_STEP;
      if (d >= d_h) continue;
      int k = 0;
      for (; k + 4 <= kn; k += 4) {
        const float* s0 = o_at(k0 + k) + d;
        const float* s1 = o_at(k0 + k + 1) + d;
        const float* s2 = o_at(k0 + k + 2) + d;
        const float* s3 = o_at(k0 + k + 3) + d;
#pragma unroll
        for (int e = 0; e < D_STEP; ++e) {
          const float x0 = s0[e], x1 = s1[e], x2 = s2[e], x3 = s3[e];
          acc[r * D_STEP + e] = fmaf(w_s[k], x0, acc[r * D_STEP + e]);
          acc[r * D_STEP + e] = fmaf(w_s[k + 1], x1, acc[r * D_STEP + e]);
          acc[r * D_STEP + e] = fmaf(w_s[k + 2], x2, acc[r * D_STEP + e]);
          acc[r * D_STEP + e] = fmaf(w_s[k + 3], x3, acc[r * D_STEP + e]);
        }
      }
      for (; k < kn; ++k) {
        const float* s0 = o_at(k0 + k) + d;
#pragma unroll
        for (int e = 0; e < D_STEP; ++e) acc[r * D_STEP + e] = fmaf(w_s[k], s0[e], acc[r * D_STEP + e]);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the next chunk rewrites w_s
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int d = d0 + r * 64 * D_STEP;
    if (d >= d_h) continue;
#pragma unroll
    for (int e = 0; e < D_STEP; ++e) dst[d + e] = acc[r * D_STEP + e];
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
