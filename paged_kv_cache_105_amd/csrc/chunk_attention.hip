// Chunk attention: every new token of a chunk attends to the positions up to
// and including its own.
//
// Page 1 "KV cache: Generation state, latency, and allocation", section 21.3:
// a prompt can be processed in chunks, and later chunks keep the earlier
// chunks' positions and cached state; section 21.1: a query reads the keys
// of earlier positions and its own.  Page 3 "xf_kv_cache", "End-to-end
// flow": after a prefix hit the request's new tokens attend to the shared
// prefix blocks and to their own chunk through one block table.  Request b
// brings n_b = query_start[b + 1] - query_start[b] new tokens at positions
// ctx_b - n_b .. ctx_b - 1 (ctx_b = context_lens[b], after the chunk's
// append); query row query_start[b] + i sits at position ctx_b - n_b + i.
//
// Two kernels:
//   * chunk_mfma_kernel (bf16 queries, bf16 or fp8 caches, d_h 128, 16-slot
//     blocks): one wave per (tile of 16 NG columns, KV head, request), a
//     column being one (new token, query head of the group) pair, columns
//     ordered token-major.  The wave walks blocks 0 .. (its last position) /
//     16 with the shared MFMA step (mfma_tiles.h); each column masks the
//     positions after its own.  No split: every wave writes final outputs.
//   * chunk_generic_kernel (any supported dtype pair, d_h <= 256, any block
//     size): one wave per (query row, query head); two passes over the
//     positions (max and sum, then weights and values).  A reference path.
//
// Requests whose query_start entries or lengths are out of range
// (n_b > ctx_b, rows past total_q) write nothing.

#include "mfma_tiles.h"

namespace pkv {

namespace {

// Clamped bounds of request b's chunk; false if the request has nothing to
// do or its entries are out of range.
__device__ __forceinline__ bool chunk_bounds(const DecodeArgs& a, int b, int& qs0, int& n_new,
                                             int& ctx) {
  qs0 = a.query_start[b];
  const int qs1 = a.query_start[b + 1];
  n_new = qs1 - qs0;
  ctx = min(a.context_lens[b], a.max_blocks_per_seq * a.block_size);
  return qs0 >= 0 && qs1 <= a.total_q && n_new > 0 && n_new <= ctx;
}

}  // namespace

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

template <int KV, int NG>
__global__ __launch_bounds__(64, 2) void chunk_mfma_kernel(DecodeArgs a) {
  __shared__ u32x4 lds_k[kBS * 16];
  const LaneMap L = lane_map();
  // one-dimensional grid over (request, KV head, tile), tile fastest, laid
  // out so that the tiles of a (request, KV head) share an XCD's L2
  const int item = xcd_block(blockIdx.x, gridDim.x);
  const int tile = item % a.chunk_tiles;
  const int h = (item / a.chunk_tiles) % a.H_KV, b = item / a.chunk_tiles / a.H_KV;
  int qs0, n_new, ctx;
  if (!chunk_bounds(a, b, qs0, n_new, ctx)) return;
  const int g = a.g, cols = n_new * g, c0 = tile * 16 * NG;
  if (c0 >= cols) return;
  const int first = ctx - n_new;                   // position of the chunk's first token
  const int c_last = min(c0 + 16 * NG, cols) - 1;  // last real column of this wave
  const int p_first = first + c0 / g, p_last = first + c_last / g;

  // B operand of QK: lane l holds Q[column 16G + c][dims 32j + 8q .. +7];
  // columns past the chunk read zeros and are never written
  bf16x8 qop[NG][4];
  int pcol[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const int col = c0 + 16 * G + L.c;
    pcol[G] = first + min(col, c_last) / g;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(qs0 + col / g) * a.H_Q + h * g + col % g) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col < cols) v = *reinterpret_cast<const u32x4*>(qrow + 32 * j + 8 * L.q4);
      qop[G][j] = __builtin_bit_cast(bf16x8, v);
    }
  }
  Acc<NG> acc;
  acc_init<NG>(acc);
  const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  run_blocks<KV, NG, 1, false>(a, L, lds_k, qop, acc, row, ctx, h, 0, p_last / kBS + 1, p_first,
                               pcol);

  // normalised outputs: lane l holds column 16G + c, dims 32q + 8i + n
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float l_tot = acc.l[G] + __shfl_xor(acc.l[G], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int col = c0 + 16 * G + L.c;
    if (col >= cols) continue;
    float* dst = a.out + (static_cast<size_t>(qs0 + col / g) * a.H_Q + h * g + col % g) * kD;
    const float mul = 1.0f / l_tot;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const f32x4 w0 = {acc.o[G][0][ii], acc.o[G][1][ii], acc.o[G][2][ii], acc.o[G][3][ii]};
      const f32x4 w1 = {acc.o[G][4][ii], acc.o[G][5][ii], acc.o[G][6][ii], acc.o[G][7][ii]};
      *reinterpret_cast<f32x4*>(dst + 32 * L.q4 + 8 * ii) = w0 * mul;
      *reinterpret_cast<f32x4*>(dst + 32 * L.q4 + 8 * ii + 4) = w1 * mul;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic kernel
// ---------------------------------------------------------------------------

constexpr int kGenMaxDh = 256;

template <int QD, int KV>
__global__ __launch_bounds__(64) void chunk_generic_kernel(DecodeArgs a) {
  __shared__ float q_s[kGenMaxDh];
  __shared__ float w_s[64];
  const int r = blockIdx.x, hq = blockIdx.y, lane = threadIdx.x;
  const int b = request_of_row(a.query_start, a.B, r);
  int qs0, n_new, ctx;
  if (!chunk_bounds(a, b, qs0, n_new, ctx)) return;
  if (r < qs0 || r >= qs0 + n_new) return;
  const int p = ctx - n_new + (r - qs0);  // this query's position
  const int h = hq / a.g, d_h = a.d_h, bs = a.block_size;
  const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  for (int d = lane; d < d_h; d += 64)
    q_s[d] = load_elem<QD>(a.q, (static_cast<size_t>(r) * a.H_Q + hq) * d_h + d);
  __syncthreads();

  // element offset of (position t, dim 0) of KV head h, and its fp8 scale
  auto slot_base = [&](int t, float& ks, float& vs) {
    const int blk = min(max(row[t / bs], 0), a.num_blocks - 1);
    if constexpr (KV == DT_FP8) {
      ks = a.k_scale[static_cast<size_t>(blk) * a.H_KV + h];
      vs = a.v_scale[static_cast<size_t>(blk) * a.H_KV + h];
    }
    return ((static_cast<size_t>(blk) * a.H_KV + h) * bs + t % bs) * d_h;
  };
  auto score = [&](int t) {
    float ks = 1.f, vs = 1.f;
    const size_t base = slot_base(t, ks, vs);
    float s = 0.f;
    for (int d = 0; d < d_h; ++d) s = fmaf(q_s[d], load_elem<KV>(a.k_cache, base + d), s);
    return s * ks * a.scale_log2;
  };

  // pass 1: M = max score, L = sum 2^(s - M) (log2 units), lanes over positions
  float m = -INFINITY, l = 0.f;
  for (int t = lane; t <= p; t += 64) {
    const float s = score(t);
    const float mn = fmaxf(m, s);
    l = l * exp2f(m - mn) + exp2f(s - mn);
    m = mn;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, m2);
    const float x = (m == mn) ? l : l * exp2f(m - mn);
    const float y = (m2 == mn) ? l2 : l2 * exp2f(m2 - mn);
    l = x + y;
    m = mn;
  }
  const float M = m, inv = 1.0f / l;

  // pass 2: 64 positions at a time, weights through LDS, lanes over dims
  float acc[kGenMaxDh / 64] = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 <= p; t0 += 64) {
    const int t = t0 + lane;
    w_s[lane] = t <= p ? exp2f(score(t) - M) * inv : 0.f;
    __syncthreads();
    const int kn = min(64, p + 1 - t0);
    for (int k = 0; k < kn; ++k) {
      float ks = 1.f, vs = 1.f;
      const size_t base = slot_base(t0 + k, ks, vs);
      const float wk = w_s[k] * vs;
#pragma unroll
      for (int e = 0; e < kGenMaxDh / 64; ++e) {
        const int d = lane + 64 * e;
        if (d < d_h) acc[e] = fmaf(wk, load_elem<KV>(a.v_cache, base + d), acc[e]);
      }
    }
    __syncthreads();
  }
  float* dst = a.out + (static_cast<size_t>(r) * a.H_Q + hq) * d_h;
#pragma unroll
  for (int e = 0; e < kGenMaxDh / 64; ++e) {
    const int d = lane + 64 * e;
    if (d < d_h) dst[d] = acc[e];
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

bool chunk_mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size) {
  return q_dtype == DT_BF16 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && d_h == kD &&
         block_size == kBS;
}

constexpr int kChunkNG = 2;  // columns per wave: 16 x kChunkNG

hipError_t launch_chunk_mfma(int kv_dtype, int max_q_len, const DecodeArgs& a,
                             hipStream_t stream) {
  const long long cols = static_cast<long long>(max_q_len) * a.g;
  const long long tiles = (cols + 16 * kChunkNG - 1) / (16 * kChunkNG);
  const long long items = tiles * a.H_KV * a.B;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  DecodeArgs ta = a;
  ta.chunk_tiles = static_cast<int32_t>(tiles);
  const dim3 grid(static_cast<unsigned>(items));
  if (kv_dtype == DT_BF16)
    hipLaunchKernelGGL((chunk_mfma_kernel<DT_BF16, kChunkNG>), grid, dim3(64), 0, stream, ta);
  else
    hipLaunchKernelGGL((chunk_mfma_kernel<DT_FP8, kChunkNG>), grid, dim3(64), 0, stream, ta);
  return hipGetLastError();
}

hipError_t launch_chunk_generic(int q_dtype, int kv_dtype, const DecodeArgs& a,
                                hipStream_t stream) {
  const dim3 grid(a.total_q, a.H_Q);
#define PKV_CHUNK_GEN(QD, KV) \
  hipLaunchKernelGGL((chunk_generic_kernel<QD, KV>), grid, dim3(64), 0, stream, a)
  if (q_dtype == DT_F32 && kv_dtype == DT_F32) PKV_CHUNK_GEN(DT_F32, DT_F32);
  else if (q_dtype == DT_BF16 && kv_dtype == DT_BF16) PKV_CHUNK_GEN(DT_BF16, DT_BF16);
  else if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) PKV_CHUNK_GEN(DT_BF16, DT_FP8);
  else return hipErrorInvalidValue;
#undef PKV_CHUNK_GEN
  return hipGetLastError();
}

}  // namespace pkv
