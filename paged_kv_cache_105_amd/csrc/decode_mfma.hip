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
// (head groups of 16; g <= 16 uses one group, g = 32 two).  The per-block
// step, its operand layouts and its masking are in mfma_tiles.h; a decode
// column is a query head, and every column sees all n positions.

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

// Flat mode: the W = gridDim.x waves share the blocks of all (request, KV
// head) sequences equally.  Sequence (b, h) holds nb_b = ceil(n_b / 16)
// blocks and starts at H_KV * P_b + h * nb_b, P_b = sum of nb over requests
// before b; T = H_KV * P_B blocks in all, cut into C = min(W, T) chunks.
// Wave w < C takes [floor(w T / C), floor((w + 1) T / C)) and walks the
// sequences it overlaps: a sequence inside the chunk is written final, a cut
// one as a partial in slot 0 (the chunk's first sequence) or slot 1 (its
// last).
template <int KV, int NG, int DEPTH, bool FUSED, bool CASCADE>
__global__ __launch_bounds__(64, 2) void decode_mfma_flat_kernel(DecodeArgs a) {
  __shared__ u32x4 lds_k[kBS * 16];
  extern __shared__ int32_t prefix[];  // [B + 1]
  const LaneMap L = lane_map();
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
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + L.lane;
    int nb = 0;
    if (b < B) nb = min(max(a.context_lens[b], 0), cap * kBS);
    nb = max((nb + kBS - 1) / kBS - skip, 0);
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
    int pcol[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) pcol[G] = n - 1;
    const int jb = static_cast<int>(cur - S) + skip, je = static_cast<int>(pe - S) + skip;
    NewRow nr;
    if constexpr (FUSED) nr = load_new_row(a, L, b, h, row, jb, je);
    run_blocks<KV, NG, DEPTH, true, FUSED>(a, L, lds_k, qop, acc, row, n, h, jb, je, n - 1, pcol,
                                           &nr);
    const size_t hq0 = static_cast<size_t>(b) * a.H_Q + static_cast<size_t>(h) * a.g;
    if (S >= lo && E <= hi && a.cascade) {
      // whole sequence of a cascade: a piece, merged with the prefix pieces
      const CascadeLayout CL = cascade_layout(B, a.H_Q, W, a.g, kD, a.prefix_splits);
      write_state<NG>(acc, L, a.g, nullptr, reinterpret_cast<float*>(a.ws + CL.seq_o) + hq0 * kD,
                      kD, reinterpret_cast<float*>(a.ws + CL.seq_ml) + hq0 * 2, 2);
    } else if (S >= lo && E <= hi) {
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

// The fused append keeps the new row in registers for the whole walk: with
// bf16 caches and one head group that fits (the bf16 kernel runs one wave
// per SIMD anyway); fp8 would lose a wave per SIMD and two head groups
// would spill, so those cases launch the append kernel first.
bool mfma_fuses_append(int kv_dtype, int g) { return kv_dtype == DT_BF16 && g <= 16; }

bool mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size, int g) {
  return q_dtype == DT_BF16 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && d_h == kD &&
         block_size == kBS && g >= 1 && g <= 32;
}

namespace {
// Loads run one block ahead of the block being processed (measured best;
// blocks are processed in pairs, so the distance must be odd).
constexpr int kDepth = 1;

template <int KV, int NG, bool FUSED = false>
const void* mfma_kernel_ptr(bool flat, bool cascade) {
  if (!flat) return reinterpret_cast<const void*>(&decode_mfma_kernel<KV, NG, kDepth, FUSED>);
  return cascade
             ? reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, kDepth, FUSED, true>)
             : reinterpret_cast<const void*>(&decode_mfma_flat_kernel<KV, NG, kDepth, FUSED, false>);
}

// fused: the append runs inside the launch (bf16 caches, one head group;
// see mfma_fuses_append); cascade: the flat grid also does the prefix work
const void* pick_kernel(int kv_dtype, int g, bool flat, bool fused, bool cascade) {
  const bool two = g > 16;
  if (kv_dtype == DT_BF16) {
    if (fused && !two) return mfma_kernel_ptr<DT_BF16, 1, true>(flat, cascade);
    return two ? mfma_kernel_ptr<DT_BF16, 2>(flat, cascade)
               : mfma_kernel_ptr<DT_BF16, 1>(flat, cascade);
  }
  return two ? mfma_kernel_ptr<DT_FP8, 2>(flat, cascade) : mfma_kernel_ptr<DT_FP8, 1>(flat, cascade);
}
}  // namespace

// Grid size of the flat kernel: never more waves than fit on the device at
// once.  bf16 blocks (8 KiB of K and V per KV head) stream best with one wave
// per SIMD -- longer chunks amortise each wave's start (lengths, table, first
// block) and fewer streams contend for HBM; fp8 blocks carry half the bytes
// for the same matrix and softmax work, so they need every resident wave to
// keep the memory busy.  (Measured on MI355X: bf16 W = 1024 vs 3072 is
// 58 vs 65 us on the 8B-style batch; fp8 is best at full occupancy.)
int mfma_flat_waves(int kv_dtype, int g, int B, bool cascade) {
  const void* k = pick_kernel(kv_dtype, g, true, cascade && mfma_fuses_append(kv_dtype, g),
                              cascade);
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

hipError_t launch_decode_mfma(int kv_dtype, bool flat, int waves, const DecodeArgs& a,
                              hipStream_t stream) {
  const bool cascade = a.cascade != 0;
  const void* k = pick_kernel(kv_dtype, a.g, flat, a.k_new != nullptr, cascade);
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  if (flat) {
    const int grid = waves + (cascade ? a.prefix_waves : 0);
    return hipLaunchKernel(k, dim3(grid), dim3(64), args, sizeof(int32_t) * (a.B + 1), stream);
  }
  return hipLaunchKernel(k, dim3(a.max_parts, a.H_KV, a.B), dim3(64), args, 0, stream);
}

}  // namespace pkv
