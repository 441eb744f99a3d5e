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
// One wave per (query head, request), or per two query heads of one KV head
// (combine_pair_kernel, below).  The workspace header says which
// layout the partition kernel wrote (see pkv_device.h).  Requests whose
// result the partition kernel wrote directly are skipped.  In a cascade
// over a shared prefix (prefix_splits > 0, flat layout only) every request
// has pieces: the flat kernel's over its private blocks (or one piece when
// no wave cut its sequence) and the prefix kernel's prefix_splits pieces
// over the shared blocks, all merged by the same rule.
//
// The kernel is latency bound (a few KiB per wave), so it is organised to
// keep the number of dependent memory round trips small: each lane loads
// the (m, l) pair of one piece at a time and merges them into its own
// running pair, one wave reduction gives (M, L), the weights stay in the
// lanes that computed them and are read with a lane shuffle, and the o rows
// are read as VW-wide vectors, several pieces per wave instruction, with
// kUnroll loads issued before any of them is used.

#include "pkv_device.h"

namespace pkv {

namespace {

// Loads of kUnroll iterations go out before any is used.  Measured on
// MI355X, combine trace us with 8 / 4 / 2: 8B-style batch 5.24 / 4.76 /
// 4.76, fp8 MQA 7.88 / 7.20 / 6.92, fp8 GQA 8.24 / 7.44 / 6.80, 32K
// contexts (17 pieces per sequence) 5.28 / 5.40 / 5.92: unused load slots
// cost instructions in every one of the many waves, too few starve the
// waves with many pieces.  (Choosing 2, 4 or 8 per wave from its piece
// count was slower still on fp8 MQA and 32K: the kernel with three copies of
// the loop ran 8.04 and 6.76 us.)
constexpr int kUnroll = 4;

template <int VW>
struct VecT;
template <>
struct VecT<1> {
  using type = float;
};
template <>
struct VecT<4> {
  typedef float type __attribute__((ext_vector_type(4)));
};

// merge (m2, l2) into (m, l): both are (max, sum of 2^(s - max)) of a set.
// The exponentials here have arguments <= 0 and results in (0, 1]; the
// hardware instruction is used directly (the library form adds steps for
// results below 2^-126, whose share of any sum is below 2^-126 as well).
__device__ inline void lse_merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  const float a = (m == mn) ? 1.f : __builtin_amdgcn_exp2f(m - mn);  // also covers m = m2 = -inf
  const float b = (m2 == mn) ? 1.f : __builtin_amdgcn_exp2f(m2 - mn);
  l = l * a + l2 * b;
  m = mn;
}

}  // namespace

// Where the pieces of (request b, query head hq) are.  Piece k < P1 has its
// (m, l) at ml + k * ml_step and its o at o + k * o_step, piece 0 shifted by
// (ml_first, o_first); a cascade's prefix pieces k = P1 .. P - 1 follow at
// ml2, o2.
struct PieceSet {
  const float* ml = nullptr;
  const float* o = nullptr;
  const float* ml2 = nullptr;
  const float* o2 = nullptr;
  size_t ml_step = 2, o_step = 0, ml_first = 0, o_first = 0, ml2_step = 0, o2_step = 0;
  int P1 = 0, P = 0;
  __device__ const float* ml_at(int k) const {
    return k < P1 ? ml + k * ml_step + (k == 0 ? ml_first : 0) : ml2 + (k - P1) * ml2_step;
  }
  __device__ const float* o_at(int k) const {
    return k < P1 ? o + k * o_step + (k == 0 ? o_first : 0) : o2 + (k - P1) * o2_step;
  }
};

// Locate the pieces of (b, hq); false when there is nothing to merge (the
// attention launch wrote the row final, or the request is empty).  One round
// trip for everything the lookup needs: the header, this request's length
// and (flat layout) the block prefix, which starts right after the header;
// the prefix words are read whenever they lie inside the workspace, whatever
// the layout, and used only for the flat one.  Every value but the head's
// own offsets is the same for all query heads of one KV head.
__device__ __forceinline__ bool locate_pieces(const int32_t* __restrict__ context_lens,
                                              const char* __restrict__ ws, size_t ws_bytes,
                                              int B, int b, int hq, int H_Q, int H_KV, int d_h,
                                              int partition_tokens, int max_parts,
                                              int prefix_splits, PieceSet& ps) {
  const WsHeader hd = *reinterpret_cast<const WsHeader*>(ws);
  const int n_b = context_lens[b];
  int pre_b = 0, pre_b1 = 0, pre_B = 0;
  if (kWsHeader + sizeof(int32_t) * (static_cast<size_t>(B) + 1) <= ws_bytes) {
    const int32_t* pre = reinterpret_cast<const int32_t*>(ws + kWsHeader);
    pre_b = pre[b];
    pre_b1 = pre[b + 1];
    pre_B = pre[B];
  }
  int P = 0, P2 = 0;
  ps.o_step = d_h;  // partition layout: pieces are contiguous
  if (hd.mode == kWsPartition) {
    P = min((n_b + partition_tokens - 1) / partition_tokens, max_parts);
    if (P <= 1) return false;
    const PartitionLayout PL = partition_layout(B, H_Q, max_parts, d_h);
    const size_t base = (static_cast<size_t>(b) * H_Q + hq) * max_parts;
    ps.ml = reinterpret_cast<const float*>(ws + PL.ml) + 2 * base;
    ps.o = reinterpret_cast<const float*>(ws + PL.o) + base * d_h;
  } else if (hd.mode == kWsFlat) {
    // flat layout: pieces come from consecutive waves, each in slot 0 except
    // the first wave's piece when that wave started in an earlier sequence
    const int W = hd.waves, C = hd.chunks, g = hd.g;
    const int h = hq / g, j = hq % g;
    const FlatLayout FL = flat_layout(B, W, g, d_h);
    const int nb = pre_b1 - pre_b;  // (a cascade: private blocks only)
    const size_t rowi = static_cast<size_t>(b) * H_Q + hq;
    if (prefix_splits > 0) {
      if (n_b < 1) return false;
      const CascadeLayout CL = cascade_layout(B, H_Q, W, g, d_h, prefix_splits);
      const size_t rows = static_cast<size_t>(B) * H_Q;
      P2 = prefix_splits;
      ps.ml2 = reinterpret_cast<const float*>(ws + CL.pre_ml) + 2 * rowi;
      ps.o2 = reinterpret_cast<const float*>(ws + CL.pre_o) + rowi * d_h;
      ps.ml2_step = 2 * rows;
      ps.o2_step = rows * d_h;
      // the private part: one piece for an uncut sequence (below), else as
      // in the plain layout
      ps.ml = reinterpret_cast<const float*>(ws + CL.seq_ml) + 2 * rowi;
      ps.o = reinterpret_cast<const float*>(ws + CL.seq_o) + rowi * d_h;
      P = nb > 0 ? 1 : 0;
    } else if (nb <= 0) {
      return false;
    }
    if (nb > 0) {
      const long long T = static_cast<long long>(H_KV) * pre_B;
      const long long S = static_cast<long long>(H_KV) * pre_b + static_cast<long long>(h) * nb;
      const int first_wave = flat_wave_of(S, T, C);
      const int last_wave = flat_wave_of(S + nb - 1, T, C);
      if (first_wave == last_wave) {
        if (prefix_splits == 0) return false;  // written final by its wave
      } else {
        const int first_slot = flat_chunk_lo(first_wave, T, C) == S ? 0 : 1;
        P = last_wave - first_wave + 1;
        const size_t base = (static_cast<size_t>(first_wave) * 2) * g + j;
        ps.ml = reinterpret_cast<const float*>(ws + FL.ml) + 2 * base;
        ps.o = reinterpret_cast<const float*>(ws + FL.o) + base * d_h;
        ps.ml_step = 2 * 2 * static_cast<size_t>(g);
        ps.o_step = 2 * static_cast<size_t>(g) * d_h;
        ps.ml_first = 2 * static_cast<size_t>(first_slot) * g;
        ps.o_first = static_cast<size_t>(first_slot) * g * d_h;
      }
    }
  } else {
    return false;
  }
  ps.P1 = P;
  ps.P = P + P2;
  return true;
}

// VW: floats per vector load (4 when d_h % 4 == 0, else 1).  R: vector
// columns per lane when a row has more than 64 of them (only VW = 1).
template <int VW, int R>
__global__ __launch_bounds__(64) void combine_kernel(float* __restrict__ out,
                                                     const int32_t* __restrict__ context_lens,
                                                     const char* __restrict__ ws,
                                                     size_t ws_bytes, int H_Q, int H_KV, int d_h,
                                                     int partition_tokens, int max_parts,
                                                     int prefix_splits) {
  using Vec = typename VecT<VW>::type;
  __shared__ Vec red_s[64 * R];
  const int hq = blockIdx.x, b = blockIdx.y, B = gridDim.y, lane = threadIdx.x;
  float* dst = out + (static_cast<size_t>(b) * H_Q + hq) * d_h;

  PieceSet ps;
  if (!locate_pieces(context_lens, ws, ws_bytes, B, b, hq, H_Q, H_KV, d_h, partition_tokens,
                     max_parts, prefix_splits, ps))
    return;
  const int P = ps.P;
  auto ml_at = [&](int k) { return ps.ml_at(k); };
  auto o_at = [&](int k) { return ps.o_at(k); };

  // pass 2's lane layout: lanes are split into PPI groups of LP lanes; group
  // s reads piece i * PPI + s of a chunk of 64 pieces on iteration i, lane c
  // of a group reads vector columns c, c + 64, ... of that piece's row
  const int ncol = d_h / VW;
  const int LP = ncol < 64 ? ncol : 64;
  const int PPI = 64 / LP;
  const int sub = lane / LP, c = lane % LP;
  const bool on = sub < PPI;
  // the o rows of the first kUnroll iterations go out together with the
  // (m, l) loads of pass 1 (their addresses do not depend on any weight)
  const int kn0 = min(64, P);
  Vec x0[kUnroll][R];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int kk = u * PPI + sub;
    const bool valid = on && kk < kn0;
    const Vec* row = reinterpret_cast<const Vec*>(o_at(valid ? kk : 0));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int col = c + r * 64;
      x0[u][r] = (valid && col < ncol) ? row[col] : Vec(0.f);
    }
  }

  // pass 1: every lane merges the pieces lane, lane + 64, ... into its own
  // (m, l); the first chunk's m stays in a register for pass 2
  float m_own = -INFINITY, m_lane = -INFINITY, l_lane = 0.f;
  if (lane < P) {
    const float2 x = *reinterpret_cast<const float2*>(ml_at(lane));
    m_own = m_lane = x.x;
    l_lane = x.y;
  }
  for (int k = lane + 64; k < P; k += 64) {
    const float2 x = *reinterpret_cast<const float2*>(ml_at(k));
    lse_merge(m_lane, l_lane, x.x, x.y);
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m_lane, off, 64), l2 = __shfl_xor(l_lane, off, 64);
    lse_merge(m_lane, l_lane, m2, l2);
  }
  const float M = m_lane, inv = 1.0f / l_lane;

  // pass 2: weights 2^(m_k - M) / L, held by lane k of each chunk of 64
  // pieces and read with a lane shuffle
  Vec acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = Vec(0.f);
  for (int k0 = 0; k0 < P; k0 += 64) {
    const int kn = min(64, P - k0);
    const float mk = (k0 == 0) ? m_own : (lane < kn ? ml_at(k0 + lane)[0] : -INFINITY);
    const float w = lane < kn ? __builtin_amdgcn_exp2f(mk - M) * inv : 0.f;
    const int iters = (kn + PPI - 1) / PPI;
    for (int i0 = 0; i0 < iters; i0 += kUnroll) {
      Vec x[kUnroll][R];
      float wk[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kk = (i0 + u) * PPI + sub;     // piece within the chunk
        const bool valid = on && kk < kn;
        wk[u] = __shfl(w, valid ? kk : 0, 64);
        if (k0 == 0 && i0 == 0) {
#pragma unroll
          for (int r = 0; r < R; ++r) x[u][r] = x0[u][r];
        } else {
          const Vec* row = reinterpret_cast<const Vec*>(o_at(k0 + (valid ? kk : 0)));
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int col = c + r * 64;
            x[u][r] = (valid && col < ncol) ? row[col] : Vec(0.f);
          }
        }
        if (!valid) wk[u] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += wk[u] * x[u][r];
    }
  }

  // sum the PPI groups' partial rows
  if (PPI > 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) red_s[lane + 64 * r] = acc[r];
    __syncthreads();
    if (sub == 0) {
      for (int s = 1; s < PPI; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += red_s[s * LP + c + 64 * r];
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int col = c + r * 64;
      if (col < ncol) reinterpret_cast<Vec*>(dst)[col] = acc[r];
    }
  }
}

// Two query heads per wave, for d_h = 128 (a head's row is 32 vectors of 4
// floats: half a wave) and an even group size: half s merges head
// 2 * blockIdx.x + s.  Both heads read the same KV head and so have the same
// pieces, so the lookup is done once for both and the wave count halves;
// with many (request, head) rows the waves share SIMDs, and the per-wave
// instructions are what the launch waits for.
__global__ __launch_bounds__(64) void combine_pair_kernel(float* __restrict__ out,
                                                          const int32_t* __restrict__ context_lens,
                                                          const char* __restrict__ ws,
                                                          size_t ws_bytes, int H_Q, int H_KV,
                                                          int partition_tokens, int max_parts,
                                                          int prefix_splits) {
  using Vec = typename VecT<4>::type;
  constexpr int kDh = 128;
  const int lane = threadIdx.x, s = lane >> 5, c = lane & 31;
  const int hq = 2 * blockIdx.x + s, b = blockIdx.y, B = gridDim.y;
  PieceSet ps;
  if (!locate_pieces(context_lens, ws, ws_bytes, B, b, hq, H_Q, H_KV, kDh, partition_tokens,
                     max_parts, prefix_splits, ps))
    return;  // the same for both halves: they share the sequence
  const int P = ps.P;
  // the rows of the first kUnroll pieces go out with the (m, l) loads
  Vec x0[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    x0[u] = u < P ? reinterpret_cast<const Vec*>(ps.o_at(u))[c] : Vec(0.f);

  // pass 1: lane c of each half merges its head's pieces c, c + 32, ...
  float m_own = -INFINITY, m_lane = -INFINITY, l_lane = 0.f;
  if (c < P) {
    const float2 x = *reinterpret_cast<const float2*>(ps.ml_at(c));
    m_own = m_lane = x.x;
    l_lane = x.y;
  }
  for (int k = c + 32; k < P; k += 32) {
    const float2 x = *reinterpret_cast<const float2*>(ps.ml_at(k));
    lse_merge(m_lane, l_lane, x.x, x.y);
  }
  for (int off = 16; off > 0; off >>= 1) {  // within the half
    const float m2 = __shfl_xor(m_lane, off, 64), l2 = __shfl_xor(l_lane, off, 64);
    lse_merge(m_lane, l_lane, m2, l2);
  }
  const float M = m_lane, inv = 1.0f / l_lane;

  // pass 2: the weight of piece k0 + k is held by lane k of the half
  Vec acc = Vec(0.f);
  for (int k0 = 0; k0 < P; k0 += 32) {
    const int kn = min(32, P - k0);
    const float mk = (k0 == 0) ? m_own : (c < kn ? ps.ml_at(k0 + c)[0] : -INFINITY);
    const float w = c < kn ? __builtin_amdgcn_exp2f(mk - M) * inv : 0.f;
    for (int i0 = 0; i0 < kn; i0 += kUnroll) {
      Vec x[kUnroll];
      float wk[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kk = i0 + u;
        const bool valid = kk < kn;
        wk[u] = __shfl(w, 32 * s + (valid ? kk : 0), 64);
        if (k0 == 0 && i0 == 0)
          x[u] = x0[u];
        else
          x[u] = valid ? reinterpret_cast<const Vec*>(ps.o_at(k0 + kk))[c] : Vec(0.f);
        if (!valid) wk[u] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc += wk[u] * x[u];
    }
  }
  reinterpret_cast<Vec*>(out + (static_cast<size_t>(b) * H_Q + hq) * kDh)[c] = acc;
}

hipError_t launch_combine(float* out, const int32_t* context_lens, const void* ws,
                          size_t ws_bytes, int B, int H_Q, int H_KV, int d_h, int partition_tokens,
                          int max_parts, int prefix_splits, hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  // Two heads per wave where the rows are many and each has few pieces: with
  // at least 128 (request, KV head) sequences the balanced split cuts each
  // into a few pieces.  With few long sequences (the 32K batch: 64 of them,
  // 17 pieces each) a whole wave per head keeps twice the loads in flight.
  // Measured on MI355X, step us one head / two heads per wave: fp8 MQA
  // 41.3-41.5 / 39.9-40.1, fp8 GQA 165.0-165.6 / 163.0-164.1, shared prefix
  // 55.1-55.4 / 54.8 per layer, 8B batch 61.0-61.2 / 60.7-61.5, 32K batch
  // 171.6-172.8 / 172.8-173.3.
  if (d_h == 128 && (H_Q / H_KV) % 2 == 0 && static_cast<long long>(B) * H_KV >= 128) {
    hipLaunchKernelGGL(combine_pair_kernel, dim3(H_Q / 2, B), dim3(64), 0, stream, out,
                       context_lens, w, ws_bytes, H_Q, H_KV, partition_tokens, max_parts,
                       prefix_splits);
    return hipGetLastError();
  }
  const dim3 grid(H_Q, B), block(64);
#define PKV_COMBINE(VW, R)                                                                    \
  hipLaunchKernelGGL((combine_kernel<VW, R>), grid, block, 0, stream, out, context_lens, w,        \
                     ws_bytes, H_Q, H_KV, d_h, partition_tokens, max_parts, prefix_splits)
  if (d_h % 4 == 0) {
    PKV_COMBINE(4, 1);  // d_h <= 256: at most 64 columns of 4
  } else if (d_h <= 64) {
    PKV_COMBINE(1, 1);
  } else if (d_h <= 128) {
    PKV_COMBINE(1, 2);
  } else if (d_h <= 192) {
    PKV_COMBINE(1, 3);
  } else {
    PKV_COMBINE(1, 4);
  }
#undef PKV_COMBINE
  return hipGetLastError();
}

}  // namespace pkv
