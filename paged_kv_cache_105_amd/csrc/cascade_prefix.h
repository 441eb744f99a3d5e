// Cascade decode over a shared prefix, the prefix part: the blocks every
// request of the batch shares are read once per (KV head, column tile) for
// all of the batch's query heads, instead of once per request.
//
// Page 3 "xf_kv_cache", "End-to-end flow" and page 1 "KV cache: Generation
// state, latency, and allocation", section 21.5 step 3: requests that share
// a prompt prefix map the same physical blocks; the keys and values of
// those blocks are the same for all of them, so their scores against each
// request's query can be computed from one read of each block.  The
// softmax over a request's positions is then assembled from pieces with the
// log-sum-exp rule (section 21.1's normalisation, split by position): these
// pieces over the shared blocks, the flat decode kernel's over the rest,
// merged by the combine.
//
// The flat decode kernel runs this on its first prefix_waves workgroups
// (the others walk the private blocks), so the short prefix waves share the
// chip with the memory-bound ones instead of taking a launch of their own.
// Work item id -> (split of the shared blocks, tile of 32 columns, KV head);
// a column is one (request, query head of the group) pair, request-major.
// A column's positions end at min(n_r, shared positions) - 1.  Each item
// writes one unnormalised (m, l, o) piece per column into the cascade's
// prefix region.

#pragma once

#include "mfma_tiles.h"

namespace pkv {

template <int KV>
__device__ __forceinline__ void prefix_wave(const DecodeArgs& a, const LaneMap& L,
                                            u32x4* lds_k, int id) {
  constexpr int NG = 2;
  const int S = a.prefix_splits;
  const int split = id % S, h = (id / S) % a.H_KV, tile = id / S / a.H_KV;
  const int g = a.g, cols = a.B * g, c0 = tile * 16 * NG;
  if (c0 >= cols) return;
  const int SB = a.shared_blocks, end_pos = a.prefix_end;
  const int bps = (SB + S - 1) / S;
  const int jb = split * bps, je = min(SB, jb + bps);
  const int cap_pos = a.max_blocks_per_seq * kBS;

  // columns: Q rows, position limits; columns past the batch read zeros
  bf16x8 qop[NG][4];
  int pcol[NG];
  int pmin = INT32_MAX;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const int col = c0 + 16 * G + L.c;
    const bool real = col < cols;
    const int r = real ? col / g : 0;
    const int n_r = min(max(a.context_lens[r], 0), cap_pos);
    pcol[G] = min(n_r, SB * kBS) - 1;
    if (real) pmin = min(pmin, pcol[G]);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(r) * a.H_Q + h * g + col % g) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (real) v = *reinterpret_cast<const u32x4*>(qrow + 32 * j + 8 * L.q4);
      qop[G][j] = __builtin_bit_cast(bf16x8, v);
    }
  }
  for (int off = 32; off > 0; off >>= 1) pmin = min(pmin, __shfl_xor(pmin, off, 64));

  Acc<NG> acc;
  acc_init<NG>(acc);
  // every table row starts with the same shared blocks: read request 0's
  run_blocks<KV, NG, 1, false>(a, L, lds_k, qop, acc, a.block_table, end_pos, h, jb, je, pmin,
                               pcol);

  const CascadeLayout CL = cascade_layout(a.B, a.H_Q, a.waves_for_layout, g, kD, S);
  float* pre_ml = reinterpret_cast<float*>(a.ws + CL.pre_ml);
  float* pre_o = reinterpret_cast<float*>(a.ws + CL.pre_o);
  const size_t rows = static_cast<size_t>(a.B) * a.H_Q;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float l_tot = acc.l[G] + __shfl_xor(acc.l[G], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int col = c0 + 16 * G + L.c;
    if (col >= cols) continue;
    const size_t rowi = static_cast<size_t>(col / g) * a.H_Q + h * g + col % g;
    const size_t piece = static_cast<size_t>(split) * rows + rowi;
    if (L.q4 == 0) {
      pre_ml[piece * 2] = acc.m[G];
      pre_ml[piece * 2 + 1] = l_tot;
    }
    float* dst = pre_o + piece * kD;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const f32x4 w0 = {acc.o[G][0][ii], acc.o[G][1][ii], acc.o[G][2][ii], acc.o[G][3][ii]};
      const f32x4 w1 = {acc.o[G][4][ii], acc.o[G][5][ii], acc.o[G][6][ii], acc.o[G][7][ii]};
      *reinterpret_cast<f32x4*>(dst + 32 * L.q4 + 8 * ii) = w0;
      *reinterpret_cast<f32x4*>(dst + 32 * L.q4 + 8 * ii + 4) = w1;
    }
  }
}

}  // namespace pkv
