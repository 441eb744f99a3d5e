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
// the weights keep ~16 significant bits.  Invalid positions (>= n, only in
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

// 4 E4M3 codes -> 4 bf16 values (two packed dwords), exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r.x = (__float_as_uint(e4m3_to_f32(w & 0xffu)) >> 16) |
        (__float_as_uint(e4m3_to_f32((w >> 8) & 0xffu)) & 0xffff0000u);
  r.y = (__float_as_uint(e4m3_to_f32((w >> 16) & 0xffu)) >> 16) |
        (__float_as_uint(e4m3_to_f32(w >> 24)) & 0xffff0000u);
  return r;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  // round to nearest even on the dropped 16 bits (inputs here are finite)
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
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

template <int KV>
__device__ __forceinline__ void load_raw(Raw<KV>& r, const char* base, int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (KV == DT_BF16) {
      r.w[s] = *reinterpret_cast<const u32x4*>(base + s * 1024 + lane * 16);
    } else {
      r.w[s] = *reinterpret_cast<const u32x2*>(base + s * 512 + lane * 8);
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

template <int KV, int NG, int DEPTH>
__global__ __launch_bounds__(64) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ u32x4 lds_k[kBS * 16];  // 16 token rows x 16 chunks of 16 B
  const int lane = threadIdx.x;
  const int q4 = lane >> 4, c = lane & 15;
  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int PT = a.partition_tokens;
  const int n_raw = a.context_lens[b];
  const int n = min(n_raw, a.max_blocks_per_seq * kBS);
  const int t0 = part * PT;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + PT);
  const int nblk = (t1 - t0 + kBS - 1) / kBS;
  const int j0 = t0 / kBS;
  const int nparts = min((n_raw + PT - 1) / PT, a.max_parts);
  const int g = a.g;

  // physical ids of this partition's blocks: lane i holds entry j0 + i
  int my_blk = 0;
  if (lane < nblk) {
    my_blk = a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + j0 + lane];
    my_blk = min(max(my_blk, 0), a.num_blocks - 1);
  }

  // B operand of QK: lane l holds Q[head 16G + c][dims 32j + 8q .. +7]
  bf16x8 qop[NG][4];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const int head = 16 * G + c;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(b) * a.H_Q + h * g + head) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < g) v = *reinterpret_cast<const u32x4*>(qrow + 32 * j + 8 * q4);
      qop[G][j] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[NG][8];
  float m_run[NG], l_run[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    m_run[G] = -INFINITY;
    l_run[G] = 0.f;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) o[G][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  constexpr int kElem = (KV == DT_BF16) ? 2 : 1;
  const size_t head_bytes = static_cast<size_t>(kBS) * kD * kElem;
  const size_t blk_bytes = head_bytes * a.H_KV;
  const char* kbase = static_cast<const char*>(a.k_cache) + h * head_bytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + h * head_bytes;

  // LDS addressing for the K transpose (chunk positions in units of 16 B)
  int wpos[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = 4 * s + q4;                       // token written by this lane
    const int f = 4 * (t & 3) + (t >> 2);           // pi^-1(t)
    wpos[s] = t * 16 + (c ^ f);
  }
  const int rtok = (c >> 2) + 4 * (c & 3);          // pi(c): token read by this lane
  int rpos[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rpos[j] = rtok * 16 + ((4 * j + q4) ^ c);

  // Loads run DEPTH blocks ahead of the block being processed.  The step
  // count is padded to a multiple of DEPTH + 1 so that every unrolled step
  // issues and processes unconditionally: a load past the partition's last
  // block re-reads that block (an L2 hit), and a padded step sees no valid
  // position, which leaves the running max, sum and output unchanged
  // (alpha = 1, p = 0, V rows zeroed).  The number of loads in flight -- and
  // every wait count -- is then the same on every path.
  const int nsteps = (nblk + DEPTH) / (DEPTH + 1) * (DEPTH + 1);
  Raw<KV> kbuf[DEPTH + 1], vbuf[DEPTH + 1];
  auto issue = [&](Raw<KV>& kr, Raw<KV>& vr, int i) {
    const int p = __builtin_amdgcn_readlane(my_blk, min(i, nblk - 1));
    load_raw<KV>(kr, kbase + p * blk_bytes, lane);
    load_raw<KV>(vr, vbase + p * blk_bytes, lane);
    if constexpr (KV == DT_FP8) {
      kr.scale = a.k_scale[static_cast<size_t>(p) * a.H_KV + h];
      vr.scale = a.v_scale[static_cast<size_t>(p) * a.H_KV + h];
    }
    // keep the scheduler from sinking these loads below the block being
    // processed (that would shrink the distance they run ahead)
    __builtin_amdgcn_sched_barrier(0);
  };

  auto process = [&](const Raw<KV>& kr, const Raw<KV>& vr, int i) {
    const int valid = t1 - (t0 + i * kBS);  // valid positions in this block (<= 0: padding)

    // ---- K: widen, transpose through LDS, QK on the matrix cores
#pragma unroll
    for (int s = 0; s < 4; ++s) lds_k[wpos[s]] = as_bf16x8<KV>(kr, s);
    lds_wave_sync();
    bf16x8 ka[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ka[j] = __builtin_bit_cast(bf16x8, lds_k[rpos[j]]);

    float kscale = a.scale_log2;
    float vscale = 1.0f;
    if constexpr (KV == DT_FP8) {
      kscale *= kr.scale;
      vscale = vr.scale;
    }

    // ---- V operands: token q + 4i, dim 8c + n  (zero the invalid rows)
    u32x4 vb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      vb[s] = as_bf16x8<KV>(vr, s);
      if (4 * s + q4 >= valid) vb[s] = u32x4{0u, 0u, 0u, 0u};
    }

#pragma unroll
    for (int G = 0; G < NG; ++G) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qop[G][j], sc, 0, 0, 0);

      // online softmax for head 16G + c over tokens q + 4i
      float s2[4];
      float mx = -INFINITY;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        s2[ii] = (q4 + 4 * ii < valid) ? sc[ii] * kscale : -INFINITY;
        mx = fmaxf(mx, s2[ii]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[G], mx);
      const float alpha = exp2f(m_run[G] - m_new);
      float pr[4], psum = 0.f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        pr[ii] = exp2f(s2[ii] - m_new);  // 0 for invalid positions
        psum += pr[ii];
      }
      l_run[G] = l_run[G] * alpha + psum;
      m_run[G] = m_new;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) o[G][nn] *= alpha;

      // probabilities (times the V scale) as hi + lo bf16 pairs
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float pv = pr[ii] * vscale;
        hi[ii] = f32_to_bf16_rne(pv);
        lo[ii] = f32_to_bf16_rne(pv - __uint_as_float(hi[ii] << 16));
      }
      const i16x4 ph = __builtin_bit_cast(i16x4, u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)});
      const i16x4 pl = __builtin_bit_cast(i16x4, u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)});

#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
        const int k = nn >> 1;
        u32x2 av;
        av.x = __builtin_amdgcn_perm(vb[1][k], vb[0][k], sel);
        av.y = __builtin_amdgcn_perm(vb[3][k], vb[2][k], sel);
        const i16x4 va = __builtin_bit_cast(i16x4, av);
        o[G][nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, o[G][nn], 0, 0, 0);
        o[G][nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, o[G][nn], 0, 0, 0);
      }
    }
    // the K tile in LDS is rewritten by the next block: keep its reads first
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(kbuf[d], vbuf[d], d);
  for (int i0 = 0; i0 < nsteps; i0 += DEPTH + 1) {
#pragma unroll
    for (int u = 0; u <= DEPTH; ++u) {
      issue(kbuf[(u + DEPTH) % (DEPTH + 1)], vbuf[(u + DEPTH) % (DEPTH + 1)], i0 + u + DEPTH);
      process(kbuf[u], vbuf[u], i0 + u);
    }
  }

  // ---- write: lane holds head 16G + c, dims 32q + 8i + n
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float l_tot = l_run[G] + __shfl_xor(l_run[G], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int head = 16 * G + c;
    if (head >= g) continue;
    const size_t hq = static_cast<size_t>(b) * a.H_Q + h * g + head;
    float* dst;
    float mul = 1.0f;
    if (nparts == 1) {
      dst = a.out + hq * kD;
      mul = 1.0f / l_tot;
    } else {
      const size_t slot = hq * a.max_parts + part;
      dst = a.ws.o + slot * kD;
      if (q4 == 0) {
        a.ws.ml[2 * slot] = m_run[G];
        a.ws.ml[2 * slot + 1] = l_tot;
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      f32x4 w0 = {o[G][0][ii], o[G][1][ii], o[G][2][ii], o[G][3][ii]};
      f32x4 w1 = {o[G][4][ii], o[G][5][ii], o[G][6][ii], o[G][7][ii]};
      if (nparts == 1) {
        w0 = w0 * mul;
        w1 = w1 * mul;
      }
      *reinterpret_cast<f32x4*>(dst + 32 * q4 + 8 * ii) = w0;
      *reinterpret_cast<f32x4*>(dst + 32 * q4 + 8 * ii + 4) = w1;
    }
  }
}

bool mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size, int g,
                   int partition_tokens) {
  return q_dtype == DT_BF16 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && d_h == kD &&
         block_size == kBS && g >= 1 && g <= 32 && partition_tokens % kBS == 0 &&
         partition_tokens <= 64 * kBS;
}

hipError_t launch_decode_mfma(int kv_dtype, int depth, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_parts, a.H_KV, a.B), block(64);
  const bool two = a.g > 16;
#define PKV_MF(KV, NG, D) \
  hipLaunchKernelGGL((decode_mfma_kernel<KV, NG, D>), grid, block, 0, stream, a)
#define PKV_MF_D(KV, NG)              \
  switch (depth) {                    \
    case 1: PKV_MF(KV, NG, 1); break; \
    case 3: PKV_MF(KV, NG, 3); break; \
    default: PKV_MF(KV, NG, 2); break; \
  }
  if (kv_dtype == DT_BF16) {
    if (two) { PKV_MF_D(DT_BF16, 2) } else { PKV_MF_D(DT_BF16, 1) }
  } else if (kv_dtype == DT_FP8) {
    if (two) { PKV_MF_D(DT_FP8, 2) } else { PKV_MF_D(DT_FP8, 1) }
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_MF_D
#undef PKV_MF
  return hipGetLastError();
}

}  // namespace pkv
