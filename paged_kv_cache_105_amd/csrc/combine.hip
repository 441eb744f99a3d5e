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

  // One round trip for everything the piece lookup needs: the header, this
  // request's length and (flat layout) the block prefix, which starts right
  // after the header; the prefix words are read whenever they lie inside the
  // workspace, whatever the layout, and used only for the flat one.
  const WsHeader hd = *reinterpret_cast<const WsHeader*>(ws);
  const int n_b = context_lens[b];
  int pre_b = 0, pre_b1 = 0, pre_B = 0;
  if (kWsHeader + sizeof(int32_t) * (static_cast<size_t>(B) + 1) <= ws_bytes) {
    const int32_t* pre = reinterpret_cast<const int32_t*>(ws + kWsHeader);
    pre_b = pre[b];
    pre_b1 = pre[b + 1];
    pre_B = pre[B];
  }

  // Locate the pieces: piece k (k < P) has its (m, l) at ml + k * ml_step
  // and its o at o + k * o_step, piece 0 shifted by (ml_first, o_first);
  // a cascade's prefix pieces k = P .. P + P2 - 1 follow at ml2, o2.
  int P = 0, P2 = 0;
  const float* ml = nullptr;
  const float* o = nullptr;
  const float* ml2 = nullptr;
  const float* o2 = nullptr;
  size_t ml_step = 2, o_step = d_h;  // partition layout: pieces are contiguous
  size_t ml_first = 0, o_first = 0;
  size_t ml2_step = 0, o2_step = 0;
  if (hd.mode == kWsPartition) {
    P = min((n_b + partition_tokens - 1) / partition_tokens, max_parts);
    if (P <= 1) return;
    const PartitionLayout PL = partition_layout(B, H_Q, max_parts, d_h);
    const size_t base = (static_cast<size_t>(b) * H_Q + hq) * max_parts;
    ml = reinterpret_cast<const float*>(ws + PL.ml) + 2 * base;
    o = reinterpret_cast<const float*>(ws + PL.o) + base * d_h;
  } else if (hd.mode == kWsFlat) {
    // flat layout: pieces come from consecutive waves, each in slot 0 except
    // the first wave's piece when that wave started in an earlier sequence
    const int W = hd.waves, C = hd.chunks, g = hd.g;
    const int h = hq / g, j = hq % g;
    const FlatLayout FL = flat_layout(B, W, g, d_h);
    const int nb = pre_b1 - pre_b;  // (a cascade: private blocks only)
    const size_t rowi = static_cast<size_t>(b) * H_Q + hq;
    if (prefix_splits > 0) {
      if (n_b < 1) return;
      const CascadeLayout CL = cascade_layout(B, H_Q, W, g, d_h, prefix_splits);
      const size_t rows = static_cast<size_t>(B) * H_Q;
      P2 = prefix_splits;
      ml2 = reinterpret_cast<const float*>(ws + CL.pre_ml) + 2 * rowi;
      o2 = reinterpret_cast<const float*>(ws + CL.pre_o) + rowi * d_h;
      ml2_step = 2 * rows;
      o2_step = rows * d_h;
      // the private part: one piece for an uncut sequence (below), else as
      // in the plain layout
      ml = reinterpret_cast<const float*>(ws + CL.seq_ml) + 2 * rowi;
      o = reinterpret_cast<const float*>(ws + CL.seq_o) + rowi * d_h;
      P = nb > 0 ? 1 : 0;
    } else if (nb <= 0) {
      return;
    }
    if (nb > 0) {
      const long long T = static_cast<long long>(H_KV) * pre_B;
      const long long S = static_cast<long long>(H_KV) * pre_b + static_cast<long long>(h) * nb;
      const int first_wave = flat_wave_of(S, T, C);
      const int last_wave = flat_wave_of(S + nb - 1, T, C);
      if (first_wave == last_wave) {
        if (prefix_splits == 0) return;  // written final by its wave
      } else {
        const int first_slot = flat_chunk_lo(first_wave, T, C) == S ? 0 : 1;
        P = last_wave - first_wave + 1;
        const size_t base = (static_cast<size_t>(first_wave) * 2) * g + j;
        ml = reinterpret_cast<const float*>(ws + FL.ml) + 2 * base;
        o = reinterpret_cast<const float*>(ws + FL.o) + base * d_h;
        ml_step = 2 * 2 * static_cast<size_t>(g);
        o_step = 2 * static_cast<size_t>(g) * d_h;
        ml_first = 2 * static_cast<size_t>(first_slot) * g;
        o_first = static_cast<size_t>(first_slot) * g * d_h;
      }
    }
  } else {
    return;
  }
  const int P1 = P;
  auto ml_at = [=](int k) {
    return k < P1 ? ml + k * ml_step + (k == 0 ? ml_first : 0) : ml2 + (k - P1) * ml2_step;
  };
  auto o_at = [=](int k) {
    return k < P1 ? o + k * o_step + (k == 0 ? o_first : 0) : o2 + (k - P1) * o2_step;
  };
  P += P2;

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

hipError_t launch_combine(float* out, const int32_t* context_lens, const void* ws,
                          size_t ws_bytes, int B, int H_Q, int H_KV, int d_h, int partition_tokens,
                          int max_parts, int prefix_splits, hipStream_t stream) {
  const dim3 grid(H_Q, B), block(64);
  const char* w = static_cast<const char*>(ws);
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
