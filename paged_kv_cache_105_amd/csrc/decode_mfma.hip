// Paged decode attention on the gfx950 matrix cores, for d_h = 128 and
// 16-slot blocks, bf16 or fp8 (E4M3) caches and bf16 queries.
//
// Page 1 "KV cache: Generation state, latency, and allocation", section 21.1:
// the g = H_Q / H_KV query heads of a group read the same KV head but keep
// separate scores; section 21.5: attention reads each position through the
// block table.  One wave (one workgroup) per (partition, KV head, request):
// each K/V block of the KV head is loaded once and used by all g query heads
// of the group, which makes the per-block work two small dense products:
//
//   S[token][head] = K_blk[16 x 128] . Q^T[128 x 16]      (4 x MFMA 16x16x32)
//   O^T[dim][head] += V_blk^T[128 x 16] . P^T[16 x 16]    (8 x 2 x MFMA 16x16x16)
//
// (head groups of 16; g <= 16 uses one group, g = 32 two).
//
// Lane l = 16 q + c (q = l / 16, c = l % 16).  Layouts:
//   * A coalesced 1 KiB load s (s = 0..3) of a bf16 block gives lane l the
//     8 dims 8c..8c+7 of token 4s + q.  fp8 blocks use 512 B loads with the
//     same token/dim assignment (8 codes per lane), widened to bf16.
//   * QK uses row r of the MFMA A operand for token pi(r) = r/4 + 4(r%4)
//     and reads K through LDS (16 B per lane, XOR-swizzled by chunk so that
//     both the row-major writes and the per-row reads are conflict free).
//     Its result then gives lane l the scores of tokens q + 4i (i = 0..3)
//     for head c -- exactly the B operand layout of the PV product with the
//     same token permutation, so P never moves between lanes.
//   * PV step n (n = 0..7) uses A-operand row c for dim 8c + n and k-index
//     4q + i for token q + 4i: lane l already holds V[q + 4i][8c + n] from
//     load s = i, so V needs one byte-permute per pair of values and no LDS.
//   * The accumulator of step n gives lane l head c, dims 32q + 8i + n: every
//     lane owns one head's running max and sum, and rescales its own
//     accumulators.
// Probabilities enter the bf16 MFMA as a hi + lo pair of bf16 values, so
// the weights keep ~16 significant bits; the running max moves only when a
// block exceeds it by more than 2^8, which spares most rescales.  Invalid positions (>= n, only in
// the request's last block) get probability 0 and their V rows are zeroed
// before the product, so garbage or NaN in unused slots is never mixed in.

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

// The cache is streamed: each tile is read once per decode step, so the
// loads carry the non-temporal hint and do not displace other data from the
// L2 and last-level caches (measured: +10-12% gather bandwidth on MI355X).
template <int KV>
__device__ __forceinline__ void load_raw(Raw<KV>& r, const char* base, int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (KV == DT_BF16) {
      r.w[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + s * 1024 + lane * 16));
    } else {
      r.w[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + s * 512 + lane * 8));
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
  L.lane = threadIdx.x;
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

// B operand of QK for the query heads of KV head h of request b:
// lane l holds Q[head 16G + c][dims 32j + 8q .. +7] (zero for heads >= g).
template <int NG>
__device__ __forceinline__ void load_q(const DecodeArgs& a, const LaneMap& L, int b, int h,
                                       bf16x8 (&qop)[NG][4]) {
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const int head = 16 * G + L.c;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(b) * a.H_Q + h * a.g + head) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < a.g) v = *reinterpret_cast<const u32x4*>(qrow + 32 * j + 8 * L.q4);
      qop[G][j] = __builtin_bit_cast(bf16x8, v);
    }
  }
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

// One block of 16 positions: QK, online softmax, PV.  `valid` counts the
// block's positions that belong to the request (<= 0 for a padding step,
// which leaves the state unchanged).
template <int KV, int NG>
__device__ __forceinline__ void process_block(const DecodeArgs& a, const LaneMap& L,
                                              u32x4* lds_k, const bf16x8 (&qop)[NG][4],
                                              Acc<NG>& acc, const Raw<KV>& kr,
                                              const Raw<KV>& vr, int valid) {
  // ---- K: widen, transpose through LDS, QK on the matrix cores
#pragma unroll
  for (int s = 0; s < 4; ++s) lds_k[L.wpos[s]] = as_bf16x8<KV>(kr, s);
  lds_wave_sync();
  bf16x8 ka[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ka[j] = __builtin_bit_cast(bf16x8, lds_k[L.rpos[j]]);

  float kscale = a.scale_log2;
  float vscale = 1.0f;
  if constexpr (KV == DT_FP8) {
    kscale *= kr.scale;
    vscale = vr.scale;
  }
  const bool full = valid >= kBS;  // uniform: only a request's last block is partial

  // ---- V operands: token q + 4i, dim 8c + n  (zero the invalid rows)
  u32x4 vb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) vb[s] = as_bf16x8<KV>(vr, s);
  if (!full) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (4 * s + L.q4 >= valid) vb[s] = u32x4{0u, 0u, 0u, 0u};
  }

#pragma unroll
  for (int G = 0; G < NG; ++G) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qop[G][j], sc, 0, 0, 0);

    // online softmax for head 16G + c over tokens q + 4i
    float s2[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) s2[ii] = sc[ii] * kscale;
    if (!full) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (L.q4 + 4 * ii >= valid) s2[ii] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // raise the running max only when needed (uniform branch over the wave;
    // the first real block always takes it since m starts at -inf)
    if (__any(mx > acc.m[G] + kRescaleSlack)) {
      const float m_new = fmaxf(acc.m[G], mx);
      const float alpha = __builtin_amdgcn_exp2f(acc.m[G] - m_new);
      acc.l[G] *= alpha;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) acc.o[G][nn] *= alpha;
      acc.m[G] = m_new;
    }
    float pr[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) pr[ii] = __builtin_amdgcn_exp2f(s2[ii] - acc.m[G]);  // 0 if invalid
    acc.l[G] += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    // probabilities (times the V scale) as hi + lo bf16 pairs
    if constexpr (KV == DT_FP8) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) pr[ii] *= vscale;
    }
    const uint32_t h01 = pack_bf16x2(pr[0], pr[1]), h23 = pack_bf16x2(pr[2], pr[3]);
    const uint32_t l01 = pack_bf16x2(pr[0] - __uint_as_float(h01 << 16),
                                     pr[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = pack_bf16x2(pr[2] - __uint_as_float(h23 << 16),
                                     pr[3] - __uint_as_float(h23 & 0xffff0000u));
    const i16x4 ph = __builtin_bit_cast(i16x4, u32x2{h01, h23});
    const i16x4 pl = __builtin_bit_cast(i16x4, u32x2{l01, l23});

#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
      const int k = nn >> 1;
      u32x2 av;
      av.x = __builtin_amdgcn_perm(vb[1][k], vb[0][k], sel);
      av.y = __builtin_amdgcn_perm(vb[3][k], vb[2][k], sel);
      const i16x4 va = __builtin_bit_cast(i16x4, av);
      acc.o[G][nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, acc.o[G][nn], 0, 0, 0);
      acc.o[G][nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, acc.o[G][nn], 0, 0, 0);
    }
  }
  // the K tile in LDS is rewritten by the next block: keep its reads first
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Blocks [jb, je) of KV head h of request b (n positions, table row `row`)
// folded into `acc`.  Table entries are read 64 at a time, one per lane.
// Within each group of up to 64 blocks, loads run DEPTH blocks ahead of the
// block being processed.  The step count is padded to a multiple of
// DEPTH + 1 so that every unrolled step issues and processes
// unconditionally: a load past the group's last block re-reads that block
// (an L2 hit), and a padding step sees no valid position.  The number of
// loads in flight -- and every wait count -- is then the same on every path.
template <int KV, int NG, int DEPTH>
__device__ __forceinline__ void run_blocks(const DecodeArgs& a, const LaneMap& L, u32x4* lds_k,
                                           const bf16x8 (&qop)[NG][4], Acc<NG>& acc,
                                           const int32_t* row, int n, int h, int jb, int je) {
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
      load_raw<KV>(kr, kbase + p * blk_bytes, L.lane);
      load_raw<KV>(vr, vbase + p * blk_bytes, L.lane);
      if constexpr (KV == DT_FP8) {
        kr.scale = a.k_scale[static_cast<size_t>(p) * a.H_KV + h];
        vr.scale = a.v_scale[static_cast<size_t>(p) * a.H_KV + h];
      }
      // keep the scheduler from sinking these loads below the block being
      // processed (that would shrink the distance they run ahead)
      __builtin_amdgcn_sched_barrier(0);
    };
    const int nsteps = (nblk + DEPTH) / (DEPTH + 1) * (DEPTH + 1);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(kbuf[d], vbuf[d], d);
    for (int i0 = 0; i0 < nsteps; i0 += DEPTH + 1) {
#pragma unroll
      for (int u = 0; u <= DEPTH; ++u) {
        const int i = i0 + u;
        issue(kbuf[(u + DEPTH) % (DEPTH + 1)], vbuf[(u + DEPTH) % (DEPTH + 1)], i + DEPTH);
        const int valid = (i < nblk) ? end_pos - (g0 + i) * kBS : 0;
        process_block<KV, NG>(a, L, lds_k, qop, acc, kbuf[u], vbuf[u], valid);
      }
    }
  }
}

// Write the state: normalised output when `final_out` is set, else the
// unnormalised partial (o, then (m, l) per head) with the given per-head
// strides.  Lane l holds head 16G + c, dims 32q + 8i + n.
template <int NG>
__device__ __forceinline__ void write_state(const Acc<NG>& acc, const LaneMap& L, int g,
                                            float* final_out, float* part_o, size_t o_stride,
                                            float* part_ml, size_t ml_stride) {
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float l_tot = acc.l[G] + __shfl_xor(acc.l[G], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int head = 16 * G + L.c;
    if (head >= g) continue;
    float* dst;
    float mul = 1.0f;
    if (final_out) {
      dst = final_out + static_cast<size_t>(head) * kD;
      mul = 1.0f / l_tot;
    } else {
      dst = part_o + head * o_stride;
      if (L.q4 == 0) {
        part_ml[head * ml_stride] = acc.m[G];
        part_ml[head * ml_stride + 1] = l_tot;
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      f32x4 w0 = {acc.o[G][0][ii], acc.o[G][1][ii], acc.o[G][2][ii], acc.o[G][3][ii]};
      f32x4 w1 = {acc.o[G][4][ii], acc.o[G][5][ii], acc.o[G][6][ii], acc.o[G][7][ii]};
      if (final_out) {
        w0 = w0 * mul;
        w1 = w1 * mul;
      }
      *reinterpret_cast<f32x4*>(dst + 32 * L.q4 + 8 * ii) = w0;
      *reinterpret_cast<f32x4*>(dst + 32 * L.q4 + 8 * ii + 4) = w1;
    }
  }
}

// Partition mode: one wave per (partition, KV head, request).
template <int KV, int NG, int DEPTH>
__global__ __launch_bounds__(64, 2) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ u32x4 lds_k[kBS * 16];  // 16 token rows x 16 chunks of 16 B
  const LaneMap L = lane_map();
  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int PT = a.partition_tokens;
  if (part == 0 && h == 0 && b == 0 && L.lane == 0 && a.ws) {
    WsHeader* hd = reinterpret_cast<WsHeader*>(a.ws);
    hd->mode = kWsPartition;
    hd->waves = 0;
    hd->B = a.B;
    hd->g = a.g;
  }
  const int n_raw = a.context_lens[b];
  const int n = min(n_raw, a.max_blocks_per_seq * kBS);
  const int t0 = part * PT;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + PT);
  const int nparts = min((n_raw + PT - 1) / PT, a.max_parts);

  bf16x8 qop[NG][4];
  load_q<NG>(a, L, b, h, qop);
  Acc<NG> acc;
  acc_init<NG>(acc);
  const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  run_blocks<KV, NG, DEPTH>(a, L, lds_k, qop, acc, row, t1, h, t0 / kBS,
                            (t1 + kBS - 1) / kBS);

  const size_t hq0 = static_cast<size_t>(b) * a.H_Q + static_cast<size_t>(h) * a.g;
  if (nparts == 1) {
    write_state<NG>(acc, L, a.g, a.out + hq0 * kD, nullptr, 0, nullptr, 0);
  } else {
    const PartitionLayout PL = partition_layout(a.B, a.H_Q, a.max_parts, kD);
    float* o = reinterpret_cast<float*>(a.ws + PL.o);
    float* ml = reinterpret_cast<float*>(a.ws + PL.ml);
    const size_t slot = hq0 * a.max_parts + part;
    write_state<NG>(acc, L, a.g, nullptr, o + slot * kD, static_cast<size_t>(a.max_parts) * kD,
                    ml + 2 * slot, static_cast<size_t>(a.max_parts) * 2);
  }
}

// Flat mode: the W = gridDim.x waves share the blocks of all (request, KV
// head) sequences equally.  Sequence (b, h) holds nb_b = ceil(n_b / 16)
// blocks and starts at H_KV * P_b + h * nb_b, P_b = sum of nb over requests
// before b; T = H_KV * P_B blocks in all, cut into C = min(W, T) chunks.
// Wave w < C takes [floor(w T / C), floor((w + 1) T / C)) and walks the
// sequences it overlaps: a sequence inside the chunk is written final, a cut
// one as a partial in slot 0 (the chunk's first sequence) or slot 1 (its
// last).
template <int KV, int NG, int DEPTH>
__global__ __launch_bounds__(64, 2) void decode_mfma_flat_kernel(DecodeArgs a) {
  __shared__ u32x4 lds_k[kBS * 16];
  extern __shared__ int32_t prefix[];  // [B + 1]
  const LaneMap L = lane_map();
  const int w = blockIdx.x, W = gridDim.x;
  const int B = a.B, HKV = a.H_KV;
  const int cap = a.max_blocks_per_seq;

  // block prefix over requests (n clamped to the table row; n < 1 -> 0 blocks)
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + L.lane;
    int nb = 0;
    if (b < B) nb = min(max(a.context_lens[b], 0), cap * kBS);
    nb = (nb + kBS - 1) / kBS;
    int x = nb;  // inclusive scan across the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (L.lane >= off) x += y;
    }
    if (b < B) prefix[b + 1] = carry + x;
    carry += __shfl(x, 63, 64);
  }
  if (L.lane == 0) prefix[0] = 0;
  lds_wave_sync();
  const long long T = static_cast<long long>(HKV) * prefix[B];
  // chunks of at least one block each: with more waves than blocks the
  // surplus waves stay idle (an empty chunk would leave a hole in the
  // sequence of pieces the combine walks)
  const int C = static_cast<int>(T < W ? T : W);
  const FlatLayout FL = flat_layout(B, W, a.g, kD);
  if (w == 0) {
    if (L.lane == 0) {
      WsHeader* hd = reinterpret_cast<WsHeader*>(a.ws);
      hd->mode = kWsFlat;
      hd->waves = W;
      hd->B = B;
      hd->g = a.g;
      hd->chunks = C;
    }
    int32_t* wp = reinterpret_cast<int32_t*>(a.ws + FL.prefix);
    for (int i = L.lane; i <= B; i += 64) wp[i] = prefix[i];
  }
  if (w >= C) return;
  const long long lo = flat_chunk_lo(w, T, C);
  const long long hi = flat_chunk_lo(w + 1, T, C);

  // request holding block lo: the last b with H_KV * P_b <= lo
  int b = 0;
  {
    int l0 = 0, l1 = B - 1;
    while (l0 < l1) {
      const int mid = (l0 + l1 + 1) >> 1;
      if (static_cast<long long>(HKV) * prefix[mid] <= lo) l0 = mid; else l1 = mid - 1;
    }
    b = l0;
  }
  int nb = prefix[b + 1] - prefix[b];
  int h = static_cast<int>((lo - static_cast<long long>(HKV) * prefix[b]) / nb);
  float* part_o = reinterpret_cast<float*>(a.ws + FL.o);
  float* part_ml = reinterpret_cast<float*>(a.ws + FL.ml);

  long long cur = lo;
  int slot = 0;
  while (cur < hi) {
    const long long S = static_cast<long long>(HKV) * prefix[b] + static_cast<long long>(h) * nb;
    const long long E = S + nb;
    const long long pe = E < hi ? E : hi;
    const int n = min(a.context_lens[b], a.max_blocks_per_seq * kBS);
    bf16x8 qop[NG][4];
    load_q<NG>(a, L, b, h, qop);
    Acc<NG> acc;
    acc_init<NG>(acc);
    const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
    run_blocks<KV, NG, DEPTH>(a, L, lds_k, qop, acc, row, n, h, static_cast<int>(cur - S),
                              static_cast<int>(pe - S));
    const size_t hq0 = static_cast<size_t>(b) * a.H_Q + static_cast<size_t>(h) * a.g;
    if (S >= lo && E <= hi) {
      write_state<NG>(acc, L, a.g, a.out + hq0 * kD, nullptr, 0, nullptr, 0);
    } else {
      const size_t base = (static_cast<size_t>(w) * 2 + slot) * a.g;
      write_state<NG>(acc, L, a.g, nullptr, part_o + base * kD, kD, part_ml + base * 2, 2);
    }
    slot = 1;
    cur = pe;
    // next sequence with at least one block
    if (++h == HKV) {
      h = 0;
      do {
        ++b;
      } while (b < B && prefix[b + 1] == prefix[b]);
      if (b >= B) break;
      nb = prefix[b + 1] - prefix[b];
    }
  }
}

bool mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size, int g) {
  return q_dtype == DT_BF16 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && d_h == kD &&
         block_size == kBS && g >= 1 && g <= 32;
}

namespace {
template <int KV, int NG, int DEPTH>
const void* mfma_kernel_ptr(bool flat) {
  return flat ? reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, DEPTH>)
              : reinterpret_cast<const void*>(&decode_mfma_kernel<KV, NG, DEPTH>);
}

const void* pick_kernel(int kv_dtype, int g, int depth, bool flat) {
  const bool two = g > 16;
#define PKV_PICK(KV, NG)                                   \
  switch (depth) {                                         \
    case 2: return mfma_kernel_ptr<KV, NG, 2>(flat);       \
    case 3: return mfma_kernel_ptr<KV, NG, 3>(flat);       \
    default: return mfma_kernel_ptr<KV, NG, 1>(flat);      \
  }
  if (kv_dtype == DT_BF16) {
    if (two) { PKV_PICK(DT_BF16, 2) } else { PKV_PICK(DT_BF16, 1) }
  } else {
    if (two) { PKV_PICK(DT_FP8, 2) } else { PKV_PICK(DT_FP8, 1) }
  }
#undef PKV_PICK
}
}  // namespace

// Grid size of the flat kernel: never more waves than fit on the device at
// once.  bf16 blocks (8 KiB of K and V per KV head) stream best with one wave
// per SIMD -- longer chunks amortise each wave's start (lengths, table, first
// block) and fewer streams contend for HBM; fp8 blocks carry half the bytes
// for the same matrix and softmax work, so they need every resident wave to
// keep the memory busy.  (Measured on MI355X: bf16 W = 1024 vs 3072 is
// 58 vs 65 us on the 8B-style batch; fp8 is best at full occupancy.)
int mfma_flat_waves(int kv_dtype, int g, int depth, int B) {
  const void* k = pick_kernel(kv_dtype, g, depth, true);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64,
                                                   sizeof(int32_t) * (B + 1)) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 256 * 4;
  }
  const int simds_per_cu = 4;
  if (kv_dtype == DT_BF16) per_cu = per_cu < simds_per_cu ? per_cu : simds_per_cu;
  return cus * per_cu;
}

hipError_t launch_decode_mfma(int kv_dtype, int depth, bool flat, int waves, const DecodeArgs& a,
                              hipStream_t stream) {
  const void* k = pick_kernel(kv_dtype, a.g, depth, flat);
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  if (flat) {
    return hipLaunchKernel(k, dim3(waves), dim3(64), args, sizeof(int32_t) * (a.B + 1), stream);
  }
  return hipLaunchKernel(k, dim3(a.max_parts, a.H_KV, a.B), dim3(64), args, 0, stream);
}

}  // namespace pkv
