// Paged decode attention on the gfx950 matrix cores, for d_h = 128 and
// 16-slot blocks, bf16 or fp8 (E4M3) caches and bf16 queries.
//
// Page 1 "KV cache: Generation state, latency, and allocation", section 21.1:
// the g = H_Q / H_KV query heads of a group read the same KV head but keep
// separate scores; section 21.5: attention reads each position through the
// block table.  A wave works on one KV head of one request at a time: each
// K/V block of the KV head is loaded once and used by all g query heads of
// the group, which makes the per-block work two small dense products:
//
//   S[token][head] = K_blk[16 x 128] . Q^T[128 x 16]       (4 x MFMA 16x16x32)
//   O^T[dim][head] += V_pair^T[128 x 32] . P^T[32 x 16]    (8 x 2 x MFMA 16x16x32
//                                                            per pair of blocks)
//
// (head groups of 16; g <= 16 uses one group, g = 32 two).  The per-block
// step, its operand layouts and its masking are in mfma_tiles.h; a decode
// column is a query head, and every column sees all n positions.  Two
// kernels: the partition kernel (one wave per (partition, KV head,
// request)) and the flat kernel (the balanced split below), which is the
// one the library picks for batches up to 8192 requests.

#include <cstdlib>
#include <type_traits>

#include "cascade_prefix.h"
#include "mfma_tiles.h"

namespace pkv {

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

// The append fused into the attention launch (pkv_decode_step, bf16
// caches): the wave whose blocks [jb, je) of sequence (b, h) include the
// request's last position t = n - 1 loads the new K and V rows when it
// starts the sequence; run_blocks stores them into their slot -- a bit
// copy, the stored form of pkv_kv_append -- and uses them in place of the
// slot's old contents when it reaches that block, so the attention reads
// the new row without waiting for its own store.  Like pkv_kv_append it
// does nothing for a request whose length or block id is out of range.
__device__ __forceinline__ NewRow load_new_row(const DecodeArgs& a, const LaneMap& L, int b,
                                               int h, const int32_t* row, int jb, int je) {
  NewRow nr;
  nr.blk = -1;
  nr.slot = 0;
  const int n = a.context_lens[b];
  if (n < 1 || n > a.max_blocks_per_seq * kBS) return nr;
  const int jn = (n - 1) / kBS;
  if (jn < jb || jn >= je) return nr;
  const int p = row[jn];
  if (p < 0 || p >= a.num_blocks) return nr;
  nr.blk = jn;
  nr.slot = (n - 1) % kBS;
  const size_t src = (static_cast<size_t>(b) * a.H_KV + h) * kD + 8 * L.c;
  nr.k = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k_new) + src);
  nr.v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.v_new) + src);
  const size_t dst = ((static_cast<size_t>(p) * a.H_KV + h) * kBS + nr.slot) * kD + 8 * L.c;
  nr.k_dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(const_cast<void*>(a.k_cache)) + dst);
  nr.v_dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(const_cast<void*>(a.v_cache)) + dst);
  return nr;
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
template <int KV, int NG, int DEPTH, bool FUSED>
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
  int pcol[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) pcol[G] = t1 - 1;
  NewRow nr;
  if constexpr (FUSED) nr = load_new_row(a, L, b, h, row, t0 / kBS, (t1 + kBS - 1) / kBS);
  run_blocks<KV, NG, DEPTH, true, FUSED>(a, L, lds_k, qop, acc, row, t1, h, t0 / kBS,
                                         (t1 + kBS - 1) / kBS, t1 - 1, pcol, &nr);

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

// Flat mode: the W = gridDim.x workgroups share the blocks of all (request,
// KV head) sequences equally.  Sequence (b, h) holds nb_b = ceil(n_b / 16)
// blocks and starts at H_KV * P_b + h * nb_b, P_b = sum of nb over requests
// before b; T = H_KV * P_B blocks in all, cut into C = min(W, T) chunks.
// Workgroup w < C takes [floor(w T / C), floor((w + 1) T / C)) (its waves
// split it, see below) and walks the sequences it overlaps: a sequence
// inside the chunk is written final, a cut one as a partial in slot 0 (the
// chunk's first sequence) or slot 1 (its last).
//
// The walk is one stream of loads over the whole chunk.  It moves in groups
// of up to 64 blocks of one sequence (one table entry per lane); when a group
// starts, the next group's table entries (and, for a new sequence, its
// length) are requested, and the last two steps of a group already load the
// next group's first two blocks, so neither a table window nor a change of
// sequence lets the loads run dry.

typedef const __attribute__((address_space(4))) int32_t* const_i32p;

// The fused append, split for the streaming walk.  When the wave starts a
// sequence it works out whether the request's newest position falls in its
// blocks (from the raw length alone: nothing is appended for a length out of
// range, or when the wave's blocks [jb, je) miss the row's block) and loads
// the row's K and V, early.  Nothing else is read then: when the walk reaches
// that block, the block's id is in the table window it walks with (a row is
// appended only if that id is inside the pool, the rule of pkv_kv_append),
// so the store and the substitution into the loaded tile happen there.
//
// bf16 caches: lane (q, c) holds dims 8c .. 8c + 7 of both rows, the part of
// the slot's row it loads from the tile when q == slot % 4.
struct NewRowBf16 {
  int blk;   // the row's block within the sequence, -1: none in this wave
  int slot;
  u32x4 k, v;
};
// fp8 caches: the row arrives in bf16 and is stored as the E4M3 codes of
// fp32(x) / scale with the scale its block already has -- the stored form of
// pkv_kv_append (page 2 "KV Cache Explained", "What changes when you use FP8
// KV": one byte per element plus scales).  The 256 values of the row (K,
// then V) are spread over the wave, 4 per lane: lane j < 32 holds K dims
// 4j .. 4j + 3, lane 32 + j the same dims of V.  The block's two scales come
// with its tile.
struct NewRowFp8 {
  int blk;
  int slot;
  u32x2 x;   // this lane's 4 bf16 values
};
template <int KV>
using NewRowOf = std::conditional_t<KV == DT_FP8, NewRowFp8, NewRowBf16>;

template <class NR>
__device__ __forceinline__ void new_row_place(const DecodeArgs& a, int n_raw, int jb, int je,
                                              NR& nr) {
  nr.blk = -1;
  nr.slot = 0;
  if (n_raw < 1 || n_raw > a.max_blocks_per_seq * kBS) return;
  const int jn = (n_raw - 1) / kBS;
  if (jn < jb || jn >= je) return;
  nr.blk = jn;
  nr.slot = (n_raw - 1) % kBS;
}
__device__ __forceinline__ void new_row_load(const DecodeArgs& a, const LaneMap& L, int b, int h,
                                             NewRowBf16& nr) {
  const size_t src = (static_cast<size_t>(b) * a.H_KV + h) * kD + 8 * L.c;
  nr.k = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k_new) + src);
  nr.v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.v_new) + src);
}
__device__ __forceinline__ void new_row_load(const DecodeArgs& a, const LaneMap& L, int b, int h,
                                             NewRowFp8& nr) {
  const size_t src = (static_cast<size_t>(b) * a.H_KV + h) * kD + 4 * (L.lane & 31);
  const void* row = L.lane < 32 ? a.k_new : a.v_new;
  nr.x = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(row) + src);
}

// 4 bf16 values (dims 2k, 2k + 1 in word k) -> their E4M3 codes of
// fp32(x) / s, byte j = the j-th value: the same division (IEEE, correctly
// rounded) and encoder as pkv_kv_append, so the stored bytes are the same.
__device__ __forceinline__ uint32_t encode4(const u32x2& x, float s) {
  const uint32_t c0 = f32_to_e4m3(bf16_lo(x.x) / s), c1 = f32_to_e4m3(bf16_hi(x.x) / s);
  const uint32_t c2 = f32_to_e4m3(bf16_lo(x.y) / s), c3 = f32_to_e4m3(bf16_hi(x.y) / s);
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Where the walk is: sequence (b, h) with nb blocks (after any skipped
// shared ones) starting at flat index S, and the group of nblk <= 64 of its
// blocks starting at flat index x; nblk == 0 past the end of the chunk.
// Every field is the same in all lanes.
struct Cursor {
  long long S, x;
  int b, h, nb, nblk;
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The group after c inside [.., hi): the next blocks of the same sequence,
// else the first group of the next sequence that has blocks.
__device__ __forceinline__ Cursor next_group(Cursor c, long long hi, const int32_t* prefix,
                                             int B, int HKV) {
  const long long E = c.S + c.nb;
  const long long seg_end = E < hi ? E : hi;
  const long long nx = c.x + c.nblk;
  if (nx < seg_end) {
    c.x = nx;
    c.nblk = static_cast<int>(seg_end - nx < 64 ? seg_end - nx : 64);
    return c;
  }
  if (E >= hi) {
    c.nblk = 0;
    return c;
  }
  if (++c.h == HKV) {
    c.h = 0;
    do {
      ++c.b;
    } while (c.b < B && prefix[c.b + 1] == prefix[c.b]);
    if (c.b >= B) {  // cannot happen while E < hi <= T; keeps prefix[] in bounds
      c.nblk = 0;
      return c;
    }
    c.nb = uniform(prefix[c.b + 1] - prefix[c.b]);
  }
  c.S = E;
  c.x = E;
  const long long e2 = E + c.nb < hi ? E + c.nb : hi;
  c.nblk = static_cast<int>(e2 - E < 64 ? e2 - E : 64);
  return c;
}

// Table entries of a group, one per lane (lanes past the group read nothing);
// ids are clamped where they are used, so nothing waits for them here.
__device__ __forceinline__ int load_window(const DecodeArgs& a, const Cursor& c, int skip,
                                           int lane) {
  int v = 0;
  if (lane < c.nblk)
    v = a.block_table[static_cast<size_t>(c.b) * a.max_blocks_per_seq +
                      static_cast<int>(c.x - c.S) + skip + lane];
  return v;
}

// HW waves per workgroup share its chunk [lo, hi): wave k walks
// [q_k, q_(k+1)), q_k = lo + min(k ceil((hi - lo) / HW), hi - lo), so only
// the last waves of a short chunk can have nothing to do.  The waves read
// different blocks, so a SIMD interleaves independent walks, while the
// chunks -- and so the partial results and the combine -- stay those of one
// walk per chunk: a sequence cut inside the chunk is merged through LDS at
// the end.  The lowest wave that covers it (its walk ends in it) keeps it
// in registers; each later wave covering it leaves its piece in its own LDS
// slot; after one barrier the first wave merges the run of pieces by the
// log-sum-exp rule and writes the sequence as one walk over the chunk would
// have.
template <int KV, int NG, bool FUSED, bool CASCADE, int HW = 1>
__global__ __launch_bounds__(64 * HW, 2) void decode_mfma_flat_kernel(DecodeArgs a) {
  static_assert(HW == 1 || ((HW == 2 || HW == 4 || HW == 8) && !CASCADE),
                "split chunks: two or four waves, no cascade");
  __shared__ u32x4 lds_k_all[HW][kBS * 16];
  // the pieces waves 1 .. HW - 1 leave for the merge: [wave - 1][group][o
  // values, m, l][lane]
  constexpr int kSlot = NG * 34 * 64;
  __shared__ float piece_lds[HW > 1 ? (HW - 1) * kSlot : 1];
  extern __shared__ int32_t prefix[];  // [B + 1]
  const LaneMap L = lane_map();
  const int hw = HW > 1 ? uniform(static_cast<int>(threadIdx.x >> 6)) : 0;
  u32x4* lds_k = lds_k_all[hw];
  int w = blockIdx.x, W = gridDim.x;
  if constexpr (CASCADE) {
    // the first prefix_waves workgroups score the whole batch against the
    // shared blocks; the rest walk the private blocks
    if (w < a.prefix_waves) {
      prefix_wave<KV>(a, L, lds_k, w);
      return;
    }
    w -= a.prefix_waves;
    W -= a.prefix_waves;
  }
  const int B = a.B, HKV = a.H_KV;
  const int cap = a.max_blocks_per_seq;

  // block prefix over requests (n clamped to the table row; n < 1 -> 0
  // blocks); a cascade's phase B counts only the blocks after the shared ones
  const int skip = a.cascade ? a.shared_blocks : 0;
  int carry = 0;
  int x = 0;  // lane l ends with prefix[b0 + l + 1] of the last 64 requests
  // one slice of 64 requests: n = their lengths (lane l: request b0 + l)
  auto scan_slice = [&](int b0, int n) {
    const int b = b0 + L.lane;
    int nb = b < B ? min(max(n, 0), cap * kBS) : 0;
    nb = max((nb + kBS - 1) / kBS - skip, 0);
    x = nb;  // inclusive scan across the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (L.lane >= off) x += y;
    }
    x += carry;
    if (hw == 0 && b < B) prefix[b + 1] = x;  // every wave holds the same x
    carry = __builtin_amdgcn_readlane(x, 63);
  };
  constexpr int kSlices = 4;
  if (B <= 64 * kSlices) {
    // the lengths of up to 256 requests load together, so the walk waits
    // for one round trip to memory rather than one per slice
    int n[kSlices];
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
      const int b = s * 64 + L.lane;
      n[s] = b < B ? a.context_lens[b] : 0;
    }
#pragma unroll
    for (int s = 0; s < kSlices; ++s)
      if (s * 64 < B) scan_slice(s * 64, n[s]);
  } else {
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + L.lane;
      scan_slice(b0, b < B ? a.context_lens[b] : 0);
    }
  }
  if (hw == 0 && L.lane == 0) prefix[0] = 0;
  if constexpr (HW > 1) {
    __syncthreads();  // the prefix wave 0 wrote
  } else {
    lds_wave_sync();
  }
  const long long T = static_cast<long long>(HKV) * carry;
  // chunks of at least one block each: with more waves than blocks the
  // surplus waves stay idle (an empty chunk would leave a hole in the
  // sequence of pieces the combine walks)
  const int C = static_cast<int>(T < W ? T : W);
  const FlatLayout FL = flat_layout(B, W, a.g, kD);
  if (w == 0 && hw == 0) {
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
  // this wave's chunk [floor(w T / C), floor((w + 1) T / C)): in 32 bits
  // (floor(w T / C) = w floor(T / C) + floor(w (T mod C) / C)) whenever the
  // operands allow, which avoids the long 64-bit division sequences
  const bool small = T < (1LL << 31) && C <= 46340;
  long long lo, hi;
  if (small) {
    const int Ti = static_cast<int>(T), q = Ti / C, r = Ti % C;
    lo = w * q + (w * r) / C;
    hi = (w + 1) * q + ((w + 1) * r) / C;
  } else {
    lo = flat_chunk_lo(w, T, C);
    hi = flat_chunk_lo(w + 1, T, C);
  }
  // this wave's part of the chunk: [wlo, whi) = [q_hw, q_(hw + 1))
  long long wlo = lo, whi = hi, part = hi - lo;
  if constexpr (HW > 1) {
    part = (hi - lo + HW - 1) / HW;
    wlo = lo + min(hw * part, hi - lo);
    whi = lo + min((hw + 1) * part, hi - lo);
  }
  float* part_o = reinterpret_cast<float*>(a.ws + FL.o);
  float* part_ml = reinterpret_cast<float*>(a.ws + FL.ml);
  // a sequence cut inside the chunk, held in this wave's registers until
  // the merge
  bool held = false;
  int held_b = 0, held_h = 0;
  long long held_S = 0, held_E = 0;
  Acc<NG> acc;

  if (wlo < whi) {
  // the sequence holding block wlo: request = the last b with H_KV * P_b <= wlo
  Cursor cur;
  {
    int pb, pb1;
    if (B <= 64) {
      // the prefix is still in the lanes (lane l: P_(l+1)): the requests
      // with H_KV * P_(b) <= wlo, b >= 1, are lanes 0 .. count - 1
      const bool le = L.lane < B && static_cast<long long>(HKV) * x <= wlo;
      const int count = __builtin_popcountll(__ballot(le));
      cur.b = min(count, B - 1);
      pb = cur.b == 0 ? 0 : __builtin_amdgcn_readlane(x, cur.b - 1);
      pb1 = __builtin_amdgcn_readlane(x, cur.b);
    } else {
      int l0 = 0, l1 = B - 1;
      while (l0 < l1) {
        const int m2 = (l0 + l1 + 1) >> 1;
        if (static_cast<long long>(HKV) * prefix[m2] <= wlo) l0 = m2; else l1 = m2 - 1;
      }
      cur.b = uniform(l0);
      pb = uniform(prefix[cur.b]);
      pb1 = uniform(prefix[cur.b + 1]);
    }
    cur.nb = pb1 - pb;
    cur.h = small ? (static_cast<int>(wlo) - HKV * pb) / cur.nb
                  : static_cast<int>((wlo - static_cast<long long>(HKV) * pb) / cur.nb);
    cur.S = static_cast<long long>(HKV) * pb + static_cast<long long>(cur.h) * cur.nb;
    cur.x = wlo;
    const long long e = cur.S + cur.nb < whi ? cur.S + cur.nb : whi;
    cur.nblk = static_cast<int>(e - wlo < 64 ? e - wlo : 64);
  }
  constexpr int kElem = (KV == DT_BF16) ? 2 : 1;
  const size_t head_bytes = static_cast<size_t>(kBS) * kD * kElem;
  Raw<KV> kbuf[2], vbuf[2];
  // load block id p (clamped into the pool) of KV head hh.  Steps that only
  // keep the load count even -- the padding step of a group with an odd
  // number of blocks, and the loads past the end of the walk -- load the
  // tile of block 0, KV head 0 instead of re-reading a block: the stream's
  // loads bypass the caches, so a re-read goes back to HBM, while the one
  // tile every wave uses that way stays cached (the data is never used: a
  // padding step masks every position).
  auto issue = [&](Raw<KV>& kr, Raw<KV>& vr, int p, int hh) {
    p = min(max(p, 0), a.num_blocks - 1);
    const size_t off = (static_cast<size_t>(p) * HKV + hh) * head_bytes;
    load_raw<KV, true>(kr, static_cast<const char*>(a.k_cache) + off, L.lane);
    load_raw<KV, true>(vr, static_cast<const char*>(a.v_cache) + off, L.lane);
    if constexpr (KV == DT_FP8) {
      kr.scale = a.k_scale[static_cast<size_t>(p) * HKV + hh];
      vr.scale = a.v_scale[static_cast<size_t>(p) * HKV + hh];
    }
    // keep the scheduler from sinking these loads below the block being
    // processed (that would shrink the distance they run ahead)
    __builtin_amdgcn_sched_barrier(0);
  };

  // context lengths and the first two table entries of each group are read
  // through the scalar cache (uniform indices; neither changes during the
  // launch), so their waits never hold up the vector loads of the stream
  const_i32p lens = (const_i32p)(a.context_lens);
  const_i32p table = (const_i32p)(a.block_table);
  auto seg_bounds = [&](const Cursor& c, int& jb, int& je) {
    const long long s0 = c.S > wlo ? c.S : wlo;
    const long long s1 = c.S + c.nb < whi ? c.S + c.nb : whi;
    jb = static_cast<int>(s0 - c.S) + skip;
    je = static_cast<int>(s1 - c.S) + skip;
  };
  int win0 = load_window(a, cur, skip, L.lane);
  const int n_raw0 = lens[cur.b];
  int n0 = min(n_raw0, cap * kBS);
  bf16x8 qop[NG][4];
  load_q<NG>(a, L, cur.b, cur.h, qop);
  NewRowOf<KV> nr;
  if constexpr (FUSED) {
    int jb, je;
    seg_bounds(cur, jb, je);
    new_row_place(a, n_raw0, jb, je, nr);
    if (nr.blk >= 0) new_row_load(a, L, cur.b, cur.h, nr);
  }
  issue(kbuf[0], vbuf[0], __builtin_amdgcn_readlane(win0, 0), cur.h);
  issue(kbuf[1], vbuf[1], cur.nblk > 1 ? __builtin_amdgcn_readlane(win0, 1) : 0,
        cur.nblk > 1 ? cur.h : 0);
  acc_init<NG>(acc);

  // One group: blocks [c.x, c.x + c.nblk) of sequence (c.b, c.h) with n
  // cached positions and table entries `win`; the loads of its first two
  // steps are already on the way.  Each step processes its block and then
  // loads the block two steps ahead: a later block of this group (the last
  // one again for a padding step), or one of the next group's first two.
  // Requests the next group's table entries into win_nxt and its sequence
  // length into n_nxt, and returns that group in nxt (nblk == 0: the chunk
  // is done).  The walk calls it with two window registers in turn, so a
  // window still on its way is never copied (a copy would wait for every
  // load in flight).
  auto group = [&](const Cursor& c, int n, int win, Cursor& nxt, int& win_nxt, int& n_nxt) {
    nxt = next_group(c, whi, prefix, B, HKV);
    const bool more = nxt.nblk > 0;
    const bool new_seq = more && nxt.x == nxt.S;
    win_nxt = load_window(a, nxt, skip, L.lane);
    int p_nxt0 = 0, p_nxt1 = 0;
    if (more) {
      const size_t e = static_cast<size_t>(nxt.b) * cap + static_cast<int>(nxt.x - nxt.S) + skip;
      p_nxt0 = table[e];
      p_nxt1 = nxt.nblk > 1 ? table[e + 1] : 0;  // 0: the padding tile
    }
    const int n_raw_nxt = new_seq ? lens[nxt.b] : n;
    n_nxt = min(n_raw_nxt, cap * kBS);
    const int jb = static_cast<int>(c.x - c.S) + skip;
    __builtin_assume(c.nblk >= 1);  // a group has at least one block
    const int nsteps = (c.nblk + 1) & ~1;
    int lim[NG];
    Half<NG> half[2];
    // One pair of steps.  The pairs before a group's last are full blocks of
    // the sequence (its last block, the only partial one and the one that
    // holds the newest position, can only end a group), so only the last
    // pair masks, substitutes the new row and sends the next sequence's
    // queries: the steady-state body has none of those branches.
    auto pair = [&](int i0, auto last_pair) {
      constexpr bool LAST = decltype(last_pair)::value;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u;
        const int t0 = (jb + i) * kBS;
        const int valid = !LAST ? kBS : i < c.nblk ? n - t0 : 0;
#pragma unroll
        for (int G = 0; G < NG; ++G) lim[G] = valid - 1;
        if constexpr (FUSED && LAST) {
          if (jb + i == nr.blk) {  // uniform: the block that holds the new row
            // its id, from the window the walk loads it with (and, for fp8,
            // its scales, loaded with the tile)
            const int p = i < c.nblk ? __builtin_amdgcn_readlane(win, i) : -1;
            if (p >= 0 && p < a.num_blocks) {
              const size_t row0 = ((static_cast<size_t>(p) * HKV + c.h) * kBS + nr.slot) * kD;
              if constexpr (KV == DT_FP8) {
                const uint32_t code =
                    encode4(nr.x, L.lane < 32 ? kbuf[u].scale : vbuf[u].scale);
                void* pool = const_cast<void*>(L.lane < 32 ? a.k_cache : a.v_cache);
                *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(pool) + row0 +
                                             4 * (L.lane & 31)) = code;
                // lane (q, c) holds dims 8c .. 8c + 7: the codes of lanes 2c, 2c + 1
                const u32x2 kw = {static_cast<uint32_t>(__shfl(code, 2 * L.c, 64)),
                                  static_cast<uint32_t>(__shfl(code, 2 * L.c + 1, 64))};
                const u32x2 vw = {static_cast<uint32_t>(__shfl(code, 32 + 2 * L.c, 64)),
                                  static_cast<uint32_t>(__shfl(code, 33 + 2 * L.c, 64))};
                if (L.q4 == (nr.slot & 3)) {
#pragma unroll
                  for (int s = 0; s < 4; ++s) {
                    if (s == (nr.slot >> 2)) {
                      kbuf[u].w[s] = kw;
                      vbuf[u].w[s] = vw;
                    }
                  }
                }
              } else if (L.q4 == (nr.slot & 3)) {
                const size_t d = row0 + 8 * L.c;
                *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(const_cast<void*>(a.k_cache)) + d) =
                    nr.k;
                *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(const_cast<void*>(a.v_cache)) + d) =
                    nr.v;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                  if (s == (nr.slot >> 2)) {
                    kbuf[u].w[s] = nr.k;
                    vbuf[u].w[s] = nr.v;
                  }
                }
              }
            }
          }
        }
        // even steps keep their scores; odd steps complete the pair
        qk_block<KV, NG>(a.scale_log2, L, lds_k, qop, kbuf[u], vbuf[u], valid, valid >= kBS,
                         lim, half[u]);
        if (u == 1) softmax_pv_pair<KV, NG>(half[0], half[1], acc);
        if (LAST && u == 1 && new_seq) {
          // the group's last QK is done: the next sequence's Q (and new
          // row) go out between its first two blocks, so every wait for
          // them is one the first block needs anyway
          load_q<NG>(a, L, nxt.b, nxt.h, qop);
          if constexpr (FUSED) {
            // this sequence's row is in place (its block came earlier in
            // the group): place the next one, and load it only where it is
            // this wave's to append
            int jb2, je2;
            seg_bounds(nxt, jb2, je2);
            new_row_place(a, n_raw_nxt, jb2, je2, nr);
            if (nr.blk >= 0) new_row_load(a, L, nxt.b, nxt.h, nr);
          }
        }
        // the load of step i + 2, into the buffer this step has used
        const int j = i + 2;
        int p, hh = c.h;
        if (j < c.nblk) {
          p = __builtin_amdgcn_readlane(win, j);
        } else if (j < nsteps) {
          p = hh = 0;  // the padding step
        } else if (more) {
          p = j == nsteps ? p_nxt0 : p_nxt1;
          hh = j == nsteps || nxt.nblk > 1 ? nxt.h : 0;
        } else {
          p = hh = 0;  // past the end of the walk
        }
        issue(kbuf[u], vbuf[u], p, hh);
      }
    };
    int i0 = 0;
    for (; i0 + 2 < nsteps; i0 += 2) pair(i0, std::false_type{});
    pair(i0, std::true_type{});
    if (!more || new_seq) {
      // the sequence's part in this wave's range is done; what is written
      // follows the workgroup's chunk [lo, hi)
      const long long S = c.S, E = c.S + c.nb;
      const size_t hq0 = static_cast<size_t>(c.b) * a.H_Q + static_cast<size_t>(c.h) * a.g;
      if (HW > 1 && hw > 0 && S < wlo) {
        // cut at this wave's start: its piece goes to the wave's LDS slot
#pragma unroll
        for (int G = 0; G < NG; ++G) {
          float* pg = piece_lds + (hw - 1) * kSlot + G * 34 * 64 + L.lane;
#pragma unroll
          for (int nn = 0; nn < 8; ++nn)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) pg[(4 * nn + ii) * 64] = acc.o[G][nn][ii];
          pg[32 * 64] = acc.m[G];
          pg[33 * 64] = acc.l[G];
        }
      } else if (HW > 1 && E > whi && whi < hi) {
        // it continues into the next wave's part: keep it for the merge (the
        // walk ends here)
        held = true;
        held_b = c.b;
        held_h = c.h;
        held_S = S;
        held_E = E;
      } else if (S >= lo && E <= hi && a.cascade) {
        // whole sequence of a cascade: a piece, merged with the prefix pieces
        const CascadeLayout CL = cascade_layout(B, a.H_Q, W, a.g, kD, a.prefix_splits);
        write_state<NG>(acc, L, a.g, nullptr,
                        reinterpret_cast<float*>(a.ws + CL.seq_o) + hq0 * kD, kD,
                        reinterpret_cast<float*>(a.ws + CL.seq_ml) + hq0 * 2, 2);
      } else if (S >= lo && E <= hi) {
        write_state<NG>(acc, L, a.g, a.out + hq0 * kD, nullptr, 0, nullptr, 0);
      } else {
        // slot 0: the chunk's first sequence (it holds block lo); slot 1: its last
        const int slot = S <= lo ? 0 : 1;
        const size_t base = (static_cast<size_t>(w) * 2 + slot) * a.g;
        write_state<NG>(acc, L, a.g, nullptr, part_o + base * kD, kD, part_ml + base * 2, 2);
      }
      if (new_seq) acc_init<NG>(acc);
    }
    return more;
  };

  Cursor cur1;
  int win1, n1;
  while (group(cur, n0, win0, cur1, win1, n1) && group(cur1, n1, win1, cur, win0, n0)) {
  }
  }  // wlo < whi

  if constexpr (HW > 1) {
    __syncthreads();  // the later waves' pieces are in LDS
    if (held) {
      // merge the pieces of the following waves that cover the sequence: all
      // use the same lane layout, and a lane's (m, l) belong to its own
      // column and dims
      for (int j = hw + 1; j < HW; ++j) {
        const long long qj = lo + min(j * part, hi - lo);
        const long long qj1 = lo + min((j + 1) * part, hi - lo);
        if (qj >= qj1 || held_E <= qj) break;  // wave j has nothing of it
#pragma unroll
        for (int G = 0; G < NG; ++G) {
          const float* pg = piece_lds + (j - 1) * kSlot + G * 34 * 64 + L.lane;
          const float m1 = pg[32 * 64], l1 = pg[33 * 64];
          const float mn = fmaxf(acc.m[G], m1);
          const float f0 = acc.m[G] == mn ? 1.0f : __builtin_amdgcn_exp2f(acc.m[G] - mn);
          const float f1 = m1 == mn ? 1.0f : __builtin_amdgcn_exp2f(m1 - mn);
          acc.l[G] = acc.l[G] * f0 + l1 * f1;
#pragma unroll
          for (int nn = 0; nn < 8; ++nn)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              acc.o[G][nn][ii] = acc.o[G][nn][ii] * f0 + pg[(4 * nn + ii) * 64] * f1;
          acc.m[G] = mn;
        }
      }
      const size_t hq0 = static_cast<size_t>(held_b) * a.H_Q + static_cast<size_t>(held_h) * a.g;
      if (held_S >= lo && held_E <= hi) {
        write_state<NG>(acc, L, a.g, a.out + hq0 * kD, nullptr, 0, nullptr, 0);
      } else {
        const int slot = held_S <= lo ? 0 : 1;
        const size_t base = (static_cast<size_t>(w) * 2 + slot) * a.g;
        write_state<NG>(acc, L, a.g, nullptr, part_o + base * kD, kD, part_ml + base * 2, 2);
      }
    }
  }
}

// The fused append keeps the new row in registers for the whole walk.  With
// bf16 caches and one head group that fits (the bf16 kernel runs one wave
// per SIMD anyway), in every launch shape.  fp8 rows are encoded when the
// walk reaches their block, 4 values per lane; that pays where the walks are
// long and latency bound, the flat walk with two head groups per wave (fp8
// MQA: one sequence per request, 32 query heads on it), without a cascade.
// Measured on MI355X, step us with the append fused / launched first: fp8
// MQA 45.0-45.6 / 47.0-47.6; fp8 GQA (one head group, four waves per chunk)
// 170.0-171.2 / 169.1-170.6, no gain (again 165.9-167.5 / 165.5-166.3 once
// the split chunks ran three waves per SIMD: its fused kernel needs 171
// registers, two waves; held to 168 registers for three, with 4 spilled,
// 171.1-172.5 / 164.9); fp8 MHA would lose a wave per SIMD the same way
// (171 instead of 155 registers: two waves instead of three).
bool mfma_fuses_append(int kv_dtype, int g, bool flat, bool cascade) {
  if (kv_dtype == DT_BF16) return g <= 16;
  return kv_dtype == DT_FP8 && g > 16 && flat && !cascade;
}

bool mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size, int g) {
  return q_dtype == DT_BF16 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && d_h == kD &&
         block_size == kBS && g >= 1 && g <= 32;
}

namespace {
// Loads run one block ahead of the block being processed (measured best;
// blocks are processed in pairs, so the distance must be odd).
constexpr int kDepth = 1;

struct KernelPick {
  const void* fn;
  int waves_per_group;  // waves of one workgroup (64 lanes each)
};

// Waves per chunk of the flat grid (no cascade).  fp8 tiles carry half the
// bytes for the same per-block chain of dependent products, so with several
// query heads per KV head the walks are latency bound and more walks per
// SIMD pay, best as four waves on each of half as many chunks (fewer cut
// sequences), and with two head groups per wave (g > 16) as eight waves on
// a quarter as many, whose 32-head pieces then shrink the combine's work;
// with one query head per KV head there is little work per block and one
// wave per chunk at full occupancy streams best; bf16 walks stream best one
// per SIMD.  Measured on MI355X, kernel us with 1 / 2 / 4 waves per chunk:
// fp8 MQA 40.6 / 37.0 / 34.4, fp8 GQA 159.8 / 152.9 / 152.6, fp8 MHA 568.6
// (full occupancy) / - / 582.2, 8B-style bf16 batch 54.5 / 55.6 / 55.4, 32K
// bf16 161.5 / 164.0 / 162.5; step us with 4 / 8 waves per chunk: fp8 MQA
// 46.6-47.0 / 45.7-45.9 (the same kernel time), fp8 GQA 166.5-167.8 /
// 168.7-169.1.  PKV_FLAT_SPLIT (1, 2, 4 or 8; 8 only for fp8 caches with
// two head groups) overrides it, for tuning measurements.
int flat_split(int kv_dtype, int g) {
  static const int forced = [] {
    const char* e = std::getenv("PKV_FLAT_SPLIT");
    const int v = e ? std::atoi(e) : 0;
    return (v == 1 || v == 2 || v == 4 || v == 8) ? v : 0;
  }();
  if (forced) return forced == 8 && !(kv_dtype == DT_FP8 && g > 16) ? 4 : forced;
  return kv_dtype == DT_FP8 && g >= 4 ? (g > 16 ? 8 : 4) : 1;
}

template <int KV, int NG, bool FUSED = false>
KernelPick mfma_kernel_ptr(bool flat, bool cascade, int split) {
  if constexpr (KV == DT_FP8 && FUSED) {
    // the flat walk without a cascade only (mfma_fuses_append)
    (void)flat;
    (void)cascade;
    switch (split) {
      case 2:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, true, false, 2>), 2};
      case 4:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, true, false, 4>), 4};
      case 8:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, true, false, 8>), 8};
      default:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, true, false, 1>), 1};
    }
  } else {
    if (!flat)
      return {reinterpret_cast<const void*>(&decode_mfma_kernel<KV, NG, kDepth, FUSED>), 1};
    if (cascade)
      return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, FUSED, true>), 1};
    switch (split) {
      case 2:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, FUSED, false, 2>),
                2};
      case 4:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, FUSED, false, 4>),
                4};
      case 8:  // fp8 caches with two head groups only (flat_split)
        if constexpr (KV == DT_FP8 && NG == 2)
          return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, FUSED, false, 8>),
                  8};
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, FUSED, false, 4>),
                4};
      default:
        return {reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, FUSED, false, 1>),
                1};
    }
  }
}

// fused: the append runs inside the launch (see mfma_fuses_append);
// cascade: the flat grid also does the prefix work
KernelPick pick_kernel(int kv_dtype, int g, bool flat, bool fused, bool cascade) {
  const bool two = g > 16;
  const int split = flat_split(kv_dtype, g);
  if (kv_dtype == DT_BF16) {
    if (fused && !two) return mfma_kernel_ptr<DT_BF16, 1, true>(flat, cascade, split);
    return two ? mfma_kernel_ptr<DT_BF16, 2>(flat, cascade, split)
               : mfma_kernel_ptr<DT_BF16, 1>(flat, cascade, split);
  }
  if (fused && two && flat && !cascade) return mfma_kernel_ptr<DT_FP8, 2, true>(flat, cascade, split);
  return two ? mfma_kernel_ptr<DT_FP8, 2>(flat, cascade, split)
             : mfma_kernel_ptr<DT_FP8, 1>(flat, cascade, split);
}
}  // namespace

// Grid size of the flat kernel: never more waves than fit on the device at
// once.  bf16 blocks (8 KiB of K and V per KV head) stream best with two
// waves per CU -- longer chunks amortise each wave's start (lengths, table,
// first block) and fewer streams contend for HBM; fp8 blocks carry half the bytes
// for the same matrix and softmax work, so with one head group they need
// every resident wave to keep the memory busy.  With two head groups (g > 16)
// every cut sequence writes 32 heads of partials (16.6 KiB per piece), so
// fewer, longer chunks win there too.  (Measured on MI355X: bf16 W = 1024 vs
// 3072 is 58 vs 65 us on the 8B-style batch; fp8 with one group is best at
// full occupancy; fp8 MQA, W = 512 / 1024 / 1536 / 2048 / 3072: 53.1 / 40.6 /
// 41.1 / 44.0 / 54.6 us.)
int mfma_flat_waves(int kv_dtype, int g, int B, bool cascade) {
  // the occupancy of the variant with the fused append where one exists
  // (the step launches it; it needs at least the registers of the other)
  const KernelPick k =
      pick_kernel(kv_dtype, g, true, mfma_fuses_append(kv_dtype, g, true, cascade), cascade);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.fn, 64 * k.waves_per_group,
                                                   sizeof(int32_t) * (B + 1)) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 256 * 4;
  }
  // per_cu counts workgroups (chunks) of waves_per_group waves.  Waves per
  // CU: two for bf16; one per SIMD for two head groups with one wave per
  // chunk; what the occupancy allows for the other fp8 walks (split chunks
  // with two head groups: two per SIMD; with one: three; one wave per chunk:
  // three).
  // Measured on MI355X, fp8 GQA (four waves per chunk) with 512 / 640 / 768
  // chunks: kernel 152.8-153.2 / 166.7 (uneven: some CUs hold three, some
  // two) / 151.3-151.4 us, step 167.1-167.3 / 181.3-181.6 / 164.5-165.9 us;
  // on another box, 512 vs 768: kernel 151.6-152.3 vs 151.4-152.0 us, step
  // 165.0-165.7 vs 164.6-165.2 us.
  //
  // bf16 walks read best with two waves per CU, half the SIMDs: fewer,
  // longer streams (and half as many cut sequences); a cascade keeps one
  // wave per SIMD, since its prefix workgroups are bound by their score and
  // P.V products (shared-prefix batch, kernel us with W = 512 / 640 / 768 /
  // 896 / 1024 / 1152 / 1280: 50.8 / 49.6 / 48.9 / 50.6 / 48.8-48.9 / 53.5 /
  // 51.2).  Measured on MI355X,
  // kernel us with W = 256 / 320 / 384 / 448 / 512 / 576 / 640 / 704 / 768
  // / 832 / 896 / 960 / 1024 / 1152 waves: 8B-style batch 80.4 / 67.9 /
  // 59.0 / 53.6 / 51.2-51.5 / 53.9 / 53.7 / 53.0 / 52.3-52.6 / 56.4 / 54.2
  // / 53.1 / 53.5-53.8 / 58.3, 32K batch 251.9 / 210.7 / 182.0 / 163.9 /
  // 155.3-155.5 / 166.6 / 162.6 / 162.0 / 161.1-162.8 / 172.6 / 165.8 /
  // 163.8 / 160.9-162.3 / 176.1 (grids that do not divide evenly over the
  // CUs are slower).
  const int simds_per_cu = 4;
  int cap_per_cu = 0;  // 0: the occupancy
  if (kv_dtype == DT_BF16)
    cap_per_cu = cascade ? simds_per_cu : 2;
  else if (g > 16 && k.waves_per_group == 1)
    cap_per_cu = simds_per_cu;
  if (cap_per_cu > 0) {
    const int cap = cap_per_cu / k.waves_per_group;
    per_cu = per_cu < cap ? per_cu : cap;
  }
  return cus * (per_cu > 0 ? per_cu : 1);
}

hipError_t launch_decode_mfma(int kv_dtype, bool flat, int waves, const DecodeArgs& a,
                              hipStream_t stream) {
  const bool cascade = a.cascade != 0;
  const KernelPick k = pick_kernel(kv_dtype, a.g, flat, a.k_new != nullptr, cascade);
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  if (flat) {
    // `waves` chunks, one workgroup each
    const int grid = waves + (cascade ? a.prefix_waves : 0);
    return hipLaunchKernel(k.fn, dim3(grid), dim3(64 * k.waves_per_group), args,
                           sizeof(int32_t) * (a.B + 1), stream);
  }
  return hipLaunchKernel(k.fn, dim3(a.max_parts, a.H_KV, a.B), dim3(64), args, 0, stream);
}

}  // namespace pkv
