// MFMA tiles of paged attention on gfx950 (d_h = 128, 16-slot blocks, bf16
// or fp8 E4M3 caches, bf16 queries): the per-block step shared by the decode
// kernels and the chunk kernel.
//
// Page 1 "KV cache: Generation state, latency, and allocation", section 21.1:
// the query heads of a group read the same KV head but keep separate scores
// and normalise them over the positions they see; section 21.5: positions
// are read through the block table.  A wave holds up to NG x 16 "columns"
// (a query head of one query position each) and folds every K/V block it
// loads into all of them:
//
//   S[token][column] = K_blk[16 x 128] . Q^T[128 x 16]     (4 x MFMA 16x16x32)
//   O^T[dim][column] += V_pair^T[128 x 32] . P^T[32 x 16]  (8 x 2 x MFMA 16x16x32
//                                                           per pair of blocks)
//
// Lane l = 16 q + c (q = l / 16, c = l % 16).  Layouts:
//   * A coalesced 1 KiB load s (s = 0..3) of a bf16 block gives lane l the
//     8 dims 8c..8c+7 of token 4s + q.  fp8 blocks use 512 B loads with the
//     same token/dim assignment (8 codes per lane), widened to bf16.
//   * QK uses row r of the MFMA A operand for token pi(r) = r/4 + 4(r%4)
//     and reads K through LDS (16 B per lane, XOR-swizzled by chunk so that
//     both the row-major writes and the per-row reads are conflict free).
//     Its result then gives lane l the scores of tokens q + 4i (i = 0..3)
//     for column c -- exactly the B operand layout of the PV product with
//     the same token permutation, so P never moves between lanes.
//   * PV runs once per pair of blocks (a, b), with K = 32: step n
//     (n = 0..7) uses A-operand row c for dim 8c + n and k-index 8q + i for
//     token q + 4i of block a (i < 4) or q + 4(i - 4) of block b (i >= 4):
//     lane l already holds V[q + 4i][8c + n] of both blocks from load
//     s = i, so V needs one byte-permute per pair of values and no LDS
//     (fp8: one permute pairs two tokens' codes of two dims, and the
//     widening conversion turns each half into one operand word).
//     (The K = 16 product runs at half the K = 32 product's rate on gfx950.)
//   * The accumulator of step n gives lane l column c, dims 32q + 8i + n:
//     every lane owns one column's running max and sum, and rescales its own
//     accumulators.
// Probabilities enter the bf16 MFMA as a hi + lo pair of bf16 values, so
// the weights keep ~16 significant bits; the running max moves only when a
// block exceeds it by more than 2^8, which spares most rescales.  Positions
// a column must not see get probability 0, and V rows past the cached
// positions are zeroed before the product, so garbage or NaN in unused
// slots is never mixed in.

#pragma once

#include "pkv_device.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kBS = 16;

// 4 E4M3 codes -> 4 bf16 values (two packed dwords), exact: gfx950 converts
// a pair of OCP E4M3 codes to bf16 in one instruction (scale 1.0; every E4M3
// value is a bf16 value).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

template <int KV>
struct Raw;  // one block of K or V as loaded by a lane
template <>
struct Raw<DT_BF16> {
  u32x4 w[4];
};
template <>
struct Raw<DT_FP8> {
  u32x2 w[4];
  float scale;  // the block's scale for this KV head, loaded with the block
};

// One lane's part of one stored row (8 dims of one token), as loaded.
template <int KV>
struct RawWord;
template <>
struct RawWord<DT_BF16> {
  using type = u32x4;
};
template <>
struct RawWord<DT_FP8> {
  using type = u32x2;
};

// The new token of a decode step whose append is fused into the attention
// launch (bf16 caches): its K and V rows, this lane's 8 dims (loaded when
// the wave starts the sequence), and where they go.  blk is the block's
// index within the sequence (-1: none in this wave); the lanes with
// q == slot % 4 hold that slot in load slot / 4.  When the walk reaches the
// block, those lanes store the row into the cache (the append) and put it
// into the loaded tile in place of the slot's old contents.
struct NewRow {
  int blk;
  int slot;
  u32x4 k, v;
  u32x4* k_dst;  // this lane's 16 bytes of the slot in the K and V pools
  u32x4* v_dst;
};

// A decode step streams the cache: each tile is read once, so the loads
// carry the non-temporal hint (NT) and do not displace other data from the
// L2 and last-level caches (measured: +10-12% gather bandwidth on MI355X).
// Chunk attention reads each tile once per column tile and keeps the hint
// off, so the other column tiles of the same request find it in L2.
template <int KV, bool NT>
__device__ __forceinline__ void load_raw(Raw<KV>& r, const char* base, int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (KV == DT_BF16) {
      const u32x4* src = reinterpret_cast<const u32x4*>(base + s * 1024 + lane * 16);
      r.w[s] = NT ? __builtin_nontemporal_load(src) : *src;
    } else {
      const u32x2* src = reinterpret_cast<const u32x2*>(base + s * 512 + lane * 8);
      r.w[s] = NT ? __builtin_nontemporal_load(src) : *src;
    }
  }
}

// chunk s as 8 bf16 values (4 dwords: dims 8c+2k, 8c+2k+1 in dword k)
template <int KV>
__device__ __forceinline__ u32x4 as_bf16x8(const Raw<KV>& r, int s) {
  if constexpr (KV == DT_BF16) {
    return r.w[s];
  } else {
    const u32x2 lo = fp8x4_to_bf16x4(r.w[s].x), hi = fp8x4_to_bf16x4(r.w[s].y);
    u32x4 o;
    o.x = lo.x;
    o.y = lo.y;
    o.z = hi.x;
    o.w = hi.y;
    return o;
  }
}

// LDS ordering inside one wave: LDS instructions of a wave execute in issue
// order, so only the compiler must be kept from moving LDS accesses across
// this point, and the writes must have completed.  No s_barrier and no wait
// on outstanding global loads (a workgroup fence would add vmcnt(0) and
// drain the prefetched blocks).
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Running softmax state of one wave for the g heads of its KV head.
template <int NG>
struct Acc {
  f32x4 o[NG][8];
  float m[NG], l[NG];
};

// Per-lane constants of the K transpose through LDS.
struct LaneMap {
  int lane, q4, c;
  int wpos[4], rpos[4];
};

__device__ __forceinline__ LaneMap lane_map() {
  LaneMap L;
  L.lane = threadIdx.x & 63;  // lane within the wave (a workgroup may hold several)
  L.q4 = L.lane >> 4;
  L.c = L.lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = 4 * s + L.q4;                      // token written by this lane
    const int f = 4 * (t & 3) + (t >> 2);            // pi^-1(t)
    L.wpos[s] = t * 16 + (L.c ^ f);
  }
  const int rtok = (L.c >> 2) + 4 * (L.c & 3);       // pi(c): token read by this lane
#pragma unroll
  for (int j = 0; j < 4; ++j) L.rpos[j] = rtok * 16 + ((4 * j + L.q4) ^ L.c);
  return L;
}

template <int NG>
__device__ __forceinline__ void acc_init(Acc<NG>& acc) {
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    acc.m[G] = -INFINITY;
    acc.l[G] = 0.f;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) acc.o[G][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Running-max slack (log2 units): the running max m is raised only when a
// block's max exceeds it by more than this, so most blocks skip the rescale
// of the accumulators.  Probabilities 2^(s - m) then stay below 2^8, well
// inside fp32 and the hi + lo bf16 split.  The result is the same softmax:
// o and l are both relative to whatever m is current.
constexpr float kRescaleSlack = 8.0f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (round to nearest even), packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Scores and V operands of one block, kept until its pair is complete.
// The score in log2 units is s2 * kscale: bf16 blocks keep the raw product
// q . k and kscale = softmax_scale * log2(e), which folds the scaling into
// the exponent's fused multiply-add (and into one product of the block's
// max), so it needs kscale > 0; fp8 blocks, whose scale can have any sign,
// are scaled as they come out of the MFMA and carry kscale = 1.
template <int NG>
struct Half {
  float s2[NG][4];  // scores of tokens q + 4i for this lane's column
  u32x4 vb[4];      // V: token 4s + q, dims 8c .. 8c + 7 (bf16 pairs; fp8
                    // blocks keep the 8 codes in .x, .y)
  float kscale;     // log2-unit score = s2 * kscale
  float vscale;     // fp8 V scale of the block (1 for bf16)
};

// QK of one block of 16 positions.  `valid` counts the block's positions
// that hold cached entries (<= 0 for a padding step); V rows at or past it
// are zeroed.  A score of this lane's column of group G counts only for
// tokens <= lim[G] (block-relative); `full` (uniform) says that every
// column sees all 16 tokens, so no score needs a mask.  Masked scores are
// -inf.
template <int KV, int NG>
__device__ __forceinline__ void qk_block(float scale_log2, const LaneMap& L, u32x4* lds_k,
                                         const bf16x8 (&qop)[NG][4], const Raw<KV>& kr,
                                         const Raw<KV>& vr, int valid, bool full,
                                         const int (&lim)[NG], Half<NG>& out) {
  // ---- K: widen, transpose through LDS, QK on the matrix cores
#pragma unroll
  for (int s = 0; s < 4; ++s) lds_k[L.wpos[s]] = as_bf16x8<KV>(kr, s);
  lds_wave_sync();
  bf16x8 ka[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ka[j] = __builtin_bit_cast(bf16x8, lds_k[L.rpos[j]]);

  float kscale = scale_log2;
  out.kscale = scale_log2;
  out.vscale = 1.0f;
  if constexpr (KV == DT_FP8) {
    kscale *= kr.scale;
    out.kscale = 1.0f;
    out.vscale = vr.scale;
  }
  // ---- V operands: token q + 4i, dim 8c + n  (zero the invalid rows)
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (KV == DT_BF16) {
      out.vb[s] = vr.w[s];
    } else {
      // the 8 codes, widened with the PV operands
      out.vb[s] = __builtin_shufflevector(vr.w[s], u32x2{0u, 0u}, 0, 1, 2, 3);
    }
  }
  if (valid < kBS) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (4 * s + L.q4 >= valid) out.vb[s] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qop[G][j], sc, 0, 0, 0);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) out.s2[G][ii] = (KV == DT_FP8) ? sc[ii] * kscale : sc[ii];
    if (!full) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (L.q4 + 4 * ii > lim[G]) out.s2[G][ii] = -INFINITY;
    }
  }
  // the K tile in LDS is rewritten by the next block: keep its reads first
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Maximum without the quieting of signalling NaNs that fmaxf costs on this
// target (one extra instruction per operand): gfx950's v_maximum3_f32.  A
// NaN operand gives NaN; the scores it is used on are finite or -inf.
__device__ __forceinline__ float fmax_fast(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the quarters of one
// column), in registers: permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second, permlane32_swap the
// upper 32 lanes of the first with the lower 32 of the second, so with both
// operands equal to x each lane ends up with its partner's value in one of
// the two results.
__device__ __forceinline__ float colmax4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmax_fast(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmax_fast(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Online softmax and PV over a pair of blocks (32 positions) with K = 32
// products: MFMA k-index 8q + i is token q + 4i of block a for i < 4 and
// token q + 4(i - 4) of block b for i >= 4, so each lane builds both
// operands from what it holds.
// Two V values of dim 8c + n, tokens 4s + q and 4(s + 1) + q, as a bf16
// pair (low half: the first token) for n = 2m and n = 2m + 1 from the
// stored words w0 (token 4s + q) and w1 (token 4(s + 1) + q).  bf16 words
// hold dims 2k, 2k + 1 in word k: one byte permute per result.  fp8 words
// hold dims 4k .. 4k + 3 in word k: one permute pairs the two tokens' codes
// of two dims, and each half of it widens to one result.
// fp8 words c0 (token t0) and c1 (token t1) holding dims d .. d + 3: bytes
// (t0 d, t1 d, t0 d + 1, t1 d + 1) and (t0 d + 2, t1 d + 2, t0 d + 3, t1 d + 3)
// widen to the bf16 pairs of dims d, d + 1 (lo) and d + 2, d + 3 (hi).
__device__ __forceinline__ void fp8_pairs(uint32_t c0, uint32_t c1, u32x2& lo, u32x2& hi) {
  lo = fp8x4_to_bf16x4(__builtin_amdgcn_perm(c1, c0, 0x05010400u));
  hi = fp8x4_to_bf16x4(__builtin_amdgcn_perm(c1, c0, 0x07030602u));
}

template <int KV>
__device__ __forceinline__ void v_pairs(const u32x4& w0, const u32x4& w1, u32x2 (&out)[4]) {
  if constexpr (KV == DT_BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[k].x = __builtin_amdgcn_perm(w1[k], w0[k], 0x05040100u);  // dim 2k
      out[k].y = __builtin_amdgcn_perm(w1[k], w0[k], 0x07060302u);  // dim 2k + 1
    }
  } else {
    fp8_pairs(w0.x, w1.x, out[0], out[1]);  // dims 0 .. 3 of the lane's 8
    fp8_pairs(w0.y, w1.y, out[2], out[3]);  // dims 4 .. 7
  }
}

template <int KV, int NG>
__device__ __forceinline__ void softmax_pv_pair(const Half<NG>& a, const Half<NG>& b,
                                                Acc<NG>& acc) {
  // V operands for the 8 dim groups: A row c = dim 8c + n; pairs (tokens
  // q, q + 4) and (q + 8, q + 12) of each block
  u32x2 pa01[4], pa23[4], pb01[4], pb23[4];
  v_pairs<KV>(a.vb[0], a.vb[1], pa01);
  v_pairs<KV>(a.vb[2], a.vb[3], pa23);
  v_pairs<KV>(b.vb[0], b.vb[1], pb01);
  v_pairs<KV>(b.vb[2], b.vb[3], pb23);
  u32x4 va[8];
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) {
    const int k = nn >> 1;
    const bool odd = nn & 1;
    va[nn].x = odd ? pa01[k].y : pa01[k].x;
    va[nn].y = odd ? pa23[k].y : pa23[k].x;
    va[nn].z = odd ? pb01[k].y : pb01[k].x;
    va[nn].w = odd ? pb23[k].y : pb23[k].x;
  }
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const float mxa =
        fmax_fast(fmax_fast(a.s2[G][0], a.s2[G][1]), fmax_fast(a.s2[G][2], a.s2[G][3]));
    const float mxb =
        fmax_fast(fmax_fast(b.s2[G][0], b.s2[G][1]), fmax_fast(b.s2[G][2], b.s2[G][3]));
    // raise the running max only when needed (uniform branch over the wave;
    // the first real block always takes it since m starts at -inf).  A
    // column's max exceeds its running max by more than the slack exactly
    // when one of its four lanes' values does, so the column max -- a
    // reduction across lanes -- is only taken inside the branch, off the
    // per-block chain.
    const float ml = fmax_fast(mxa * a.kscale, mxb * b.kscale);
    if (__any(ml > acc.m[G] + kRescaleSlack)) {
      const float mx = colmax4(ml);
      const float m_new = fmaxf(acc.m[G], mx);
      const float alpha = __builtin_amdgcn_exp2f(acc.m[G] - m_new);
      acc.l[G] *= alpha;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) acc.o[G][nn] *= alpha;
      acc.m[G] = m_new;
    }
    float pr[8];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      // 0 if masked
      pr[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(a.s2[G][ii], a.kscale, -acc.m[G]));
      pr[4 + ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(b.s2[G][ii], b.kscale, -acc.m[G]));
    }
    acc.l[G] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // probabilities (times the fp8 V scale) as hi + lo bf16 pairs
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      pr[ii] *= a.vscale;
      pr[4 + ii] *= b.vscale;
    }
    u32x4 hi, lo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t h = pack_bf16x2(pr[2 * k], pr[2 * k + 1]);
      hi[k] = h;
      lo[k] = pack_bf16x2(pr[2 * k] - __uint_as_float(h << 16),
                          pr[2 * k + 1] - __uint_as_float(h & 0xffff0000u));
    }
    const bf16x8 ph = __builtin_bit_cast(bf16x8, hi);
    const bf16x8 pl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const bf16x8 v8 = __builtin_bit_cast(bf16x8, va[nn]);
      acc.o[G][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, ph, acc.o[G][nn], 0, 0, 0);
      acc.o[G][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pl, acc.o[G][nn], 0, 0, 0);
    }
  }
}

// Blocks [jb, je) of KV head h of one request (table row `row`, cached
// positions < n) folded into `acc`; with FUSED, `nr` is the new row to
// append and substitute into its block after the load.  Column (lane c of group G) sees the
// positions <= pcol[G]; p_first (uniform) is the smallest of them.  Decode
// passes n - 1 for all.  Table entries are read 64 at a time, one per lane.
// Within each group of up to 64 blocks, loads run DEPTH blocks ahead of the
// block being processed.  The step count is padded to a multiple of
// DEPTH + 1 so that every unrolled step issues and processes
// unconditionally: a load past the group's last block re-reads that block
// (an L2 hit), and a padding step sees no valid position.  The number of
// loads in flight -- and every wait count -- is then the same on every path.
// DEPTH + 1 is even, so steps come in pairs: the even step keeps its
// scores and V operands, the odd step completes the pair's softmax and PV.
template <int KV, int NG, int DEPTH, bool NT = true, bool FUSED = false>
__device__ __forceinline__ void run_blocks(const DecodeArgs& a, const LaneMap& L, u32x4* lds_k,
                                           const bf16x8 (&qop)[NG][4], Acc<NG>& acc,
                                           const int32_t* row, int n, int h, int jb, int je,
                                           int p_first, const int (&pcol)[NG],
                                           const NewRow* nr = nullptr) {
  constexpr int kElem = (KV == DT_BF16) ? 2 : 1;
  const size_t head_bytes = static_cast<size_t>(kBS) * kD * kElem;
  const size_t blk_bytes = head_bytes * a.H_KV;
  const char* kbase = static_cast<const char*>(a.k_cache) + h * head_bytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + h * head_bytes;
  const int end_pos = min(n, je * kBS);

  for (int g0 = jb; g0 < je; g0 += 64) {
    const int nblk = min(64, je - g0);
    int my_blk = 0;
    if (L.lane < nblk) my_blk = min(max(row[g0 + L.lane], 0), a.num_blocks - 1);

    Raw<KV> kbuf[DEPTH + 1], vbuf[DEPTH + 1];
    auto issue = [&](Raw<KV>& kr, Raw<KV>& vr, int i) {
      const int p = __builtin_amdgcn_readlane(my_blk, min(i, nblk - 1));
      load_raw<KV, NT>(kr, kbase + p * blk_bytes, L.lane);
      load_raw<KV, NT>(vr, vbase + p * blk_bytes, L.lane);
      if constexpr (KV == DT_FP8) {
        kr.scale = a.k_scale[static_cast<size_t>(p) * a.H_KV + h];
        vr.scale = a.v_scale[static_cast<size_t>(p) * a.H_KV + h];
      }
      // keep the scheduler from sinking these loads below the block being
      // processed (that would shrink the distance they run ahead)
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert((DEPTH + 1) % 2 == 0, "blocks are processed in pairs");
    const int nsteps = (nblk + DEPTH) / (DEPTH + 1) * (DEPTH + 1);
    Half<NG> half[2];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(kbuf[d], vbuf[d], d);
    for (int i0 = 0; i0 < nsteps; i0 += DEPTH + 1) {
#pragma unroll
      for (int u = 0; u <= DEPTH; ++u) {
        const int i = i0 + u;
        issue(kbuf[(u + DEPTH) % (DEPTH + 1)], vbuf[(u + DEPTH) % (DEPTH + 1)], i + DEPTH);
        const int t0 = (g0 + i) * kBS;
        const int valid = (i < nblk) ? end_pos - t0 : 0;
        const bool full = valid >= kBS && t0 + kBS - 1 <= p_first;
        int lim[NG];
#pragma unroll
        for (int G = 0; G < NG; ++G) lim[G] = min(pcol[G] - t0, valid - 1);
        if constexpr (FUSED) {
          static_assert(KV == DT_BF16, "the fused append stores bf16 rows as they come");
          if (g0 + i == nr->blk) {  // uniform: the block that holds the new row
            if (L.q4 == (nr->slot & 3)) {
              *nr->k_dst = nr->k;
              *nr->v_dst = nr->v;
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                if (s == (nr->slot >> 2)) {
                  kbuf[u].w[s] = nr->k;
                  vbuf[u].w[s] = nr->v;
                }
              }
            }
          }
        }
        // even steps keep their scores; odd steps complete the pair
        qk_block<KV, NG>(a.scale_log2, L, lds_k, qop, kbuf[u], vbuf[u], valid, full, lim,
                         half[u & 1]);
        if (u & 1) softmax_pv_pair<KV, NG>(half[0], half[1], acc);
      }
    }
  }
}

}  // namespace pkv
