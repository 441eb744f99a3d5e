// Generic paged decode attention, one workgroup per (partition, KV head,
// request), plain VALU arithmetic.  Covers every supported shape (any d_h up
// to 256, any block size, any group size) and is the path for fp32 caches.
//
// Page 1 "KV cache: Generation state, latency, and allocation": section 21.1
// (each query head of a group normalises its own scores over the cached keys
// of its request and mixes the values), section 21.5 (attention follows the
// block table; logical position t is block t / bs, slot t % bs).
//
// Work of one workgroup, over the positions [t0, t1) of one partition:
//   1. stage the g query rows of the group in LDS as fp32;
//   2. one thread per (head, position) pair forms s2 = log2(e) * scale * q.k;
//   3. one wave per head turns the scores into 2^(s2 - m) and their sum;
//   4. one thread per (head, element) forms sum_t 2^(s2_t - m) v_t.
// Positions >= n are never read.  The partial (m, l, o) goes to the
// workspace, or out = o / l directly when the request has one partition.

#include "pkv_device.h"

namespace pkv {

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int QT, int KV>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = a.g, d_h = a.d_h, bs = a.block_size, PT = a.partition_tokens;
  if (part == 0 && h == 0 && b == 0 && threadIdx.x == 0 && a.ws) {
    WsHeader* hd = reinterpret_cast<WsHeader*>(a.ws);
    hd->mode = kWsPartition;
    hd->waves = 0;
    hd->B = a.B;
    hd->g = g;
  }
  const int n_raw = a.context_lens[b];
  const int n = min(n_raw, a.max_blocks_per_seq * bs);   // never read past the table row
  const int t0 = part * PT;
  if (t0 >= n) return;
  const int T = min(n - t0, PT);
  const int nparts = min((n_raw + PT - 1) / PT, a.max_parts);

  float* q_s = smem;                   // [g][d_h]
  float* s_s = q_s + g * d_h;          // [g][PT]
  float* ml_s = s_s + g * PT;          // [g][2]
  const int tid = threadIdx.x, nth = blockDim.x;
  const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  const size_t head_stride = static_cast<size_t>(bs) * d_h;          // elements
  const size_t block_stride = head_stride * a.H_KV;

  for (int i = tid; i < g * d_h; i += nth)
    q_s[i] = load_elem<QT>(a.q, (static_cast<size_t>(b) * a.H_Q + h * g) * d_h + i);
  __syncthreads();

  // 2. scores
  for (int idx = tid; idx < g * T; idx += nth) {
    const int j = idx / T, i = idx % T, t = t0 + i;
    const int p = min(max(row[t / bs], 0), a.num_blocks - 1);
    const size_t base = p * block_stride + h * head_stride + static_cast<size_t>(t % bs) * d_h;
    const float* qj = q_s + j * d_h;
    float acc = 0.f;
    for (int d = 0; d < d_h; ++d) acc = fmaf(qj[d], load_elem<KV>(a.k_cache, base + d), acc);
    if constexpr (KV == DT_FP8) acc *= a.k_scale[static_cast<size_t>(p) * a.H_KV + h];
    s_s[j * PT + i] = acc * a.scale_log2;
  }
  __syncthreads();

  // 3. softmax numerators per head
  const int wave = tid >> 6, lane = tid & 63, nwaves = nth >> 6;
  for (int j = wave; j < g; j += nwaves) {
    float m = -INFINITY;
    for (int i = lane; i < T; i += 64) m = fmaxf(m, s_s[j * PT + i]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < T; i += 64) {
      const float e = exp2f(s_s[j * PT + i] - m);
      s_s[j * PT + i] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      ml_s[2 * j] = m;
      ml_s[2 * j + 1] = l;
    }
  }
  __syncthreads();

  // 4. value mixture
  for (int idx = tid; idx < g * d_h; idx += nth) {
    const int j = idx / d_h, d = idx % d_h;
    float acc = 0.f;
    for (int i = 0; i < T; ++i) {
      const int t = t0 + i;
      const int p = min(max(row[t / bs], 0), a.num_blocks - 1);
      const size_t base = p * block_stride + h * head_stride + static_cast<size_t>(t % bs) * d_h;
      float v = load_elem<KV>(a.v_cache, base + d);
      if constexpr (KV == DT_FP8) v *= a.v_scale[static_cast<size_t>(p) * a.H_KV + h];
      acc = fmaf(s_s[j * PT + i], v, acc);
    }
    const size_t hq = static_cast<size_t>(b) * a.H_Q + h * g + j;
    if (nparts == 1) {
      a.out[hq * d_h + d] = acc / ml_s[2 * j + 1];
    } else {
      const PartitionLayout PL = partition_layout(a.B, a.H_Q, a.max_parts, d_h);
      float* wo = reinterpret_cast<float*>(a.ws + PL.o);
      float* wml = reinterpret_cast<float*>(a.ws + PL.ml);
      const size_t slot = hq * a.max_parts + part;
      wo[slot * d_h + d] = acc;
      if (d == 0) {
        wml[2 * slot] = ml_s[2 * j];
        wml[2 * slot + 1] = ml_s[2 * j + 1];
      }
    }
  }
}

size_t generic_lds_bytes(int g, int d_h, int partition_tokens) {
  return sizeof(float) * (static_cast<size_t>(g) * d_h + static_cast<size_t>(g) * partition_tokens +
                          2 * static_cast<size_t>(g));
}

hipError_t launch_decode_generic(int q_dtype, int kv_dtype, const DecodeArgs& a,
                                 hipStream_t stream) {
  const dim3 grid(a.max_parts, a.H_KV, a.B), block(256);
  const size_t lds = generic_lds_bytes(a.g, a.d_h, a.partition_tokens);
#define PKV_GEN(QT, KV) \
  hipLaunchKernelGGL((decode_generic_kernel<QT, KV>), grid, block, lds, stream, a)
  if (q_dtype == DT_F32 && kv_dtype == DT_F32) PKV_GEN(DT_F32, DT_F32);
  else if (q_dtype == DT_BF16 && kv_dtype == DT_BF16) PKV_GEN(DT_BF16, DT_BF16);
  else if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) PKV_GEN(DT_BF16, DT_FP8);
  else return hipErrorInvalidValue;
#undef PKV_GEN
  return hipGetLastError();
}

}  // namespace pkv
