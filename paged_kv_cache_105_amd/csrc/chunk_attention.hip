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
// Three kernels:
//   * chunk_mfma_wg_kernel (bf16 queries and caches, d_h 128, 16-slot
//     blocks): one workgroup of four waves per (tile of 128 columns, KV
//     head, request), a column being one (new token, query head of the
//     group) pair, columns ordered token-major.  The workgroup walks blocks
//     0 .. (its last position) / 16, loading each pair of blocks once into
//     LDS for all four waves; each column masks the positions after its own.
//     No split: every wave writes final outputs.
//   * chunk_mfma_kernel (the same for fp8 caches): one wave per tile of 32
//     columns, each wave loading its own tiles and using the shared MFMA step
//     (mfma_tiles.h).
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
// One-wave MFMA kernel (fp8 caches)
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
// Workgroup MFMA kernel (bf16 caches): four waves share every K/V tile
// ---------------------------------------------------------------------------
//
// One workgroup of four waves per (tile of 128 columns, KV head, request);
// wave w holds columns 32w .. 32w + 31 of the tile (two groups of 16), with
// the score and softmax steps of the one-wave kernel.  The four waves load
// each pair of blocks together (each thread 16 bytes of each block's K and
// V), once for all 128 columns, into one of two LDS stages: the loads of
// pair p + 2 go out after pair p's products and are stored after pair p + 1's,
// so they have a whole step to arrive.  K is stored in the transposed layout
// the score products read; V row-major with its 32-byte column groups
// XOR-swizzled by row, and read as the P.V operand with gfx950's transposing
// LDS read (ds_read_b64_tr_b16): lane 16q + 4e + j reads the 4 dims
// 16n + 4j .. + 3 of token q + 4e, and the transpose hands lane 16q + c the
// dim 16n + c of tokens q, q + 4, q + 8, q + 12 -- the operand of P.V step
// n, whose accumulator then holds dims 16n + 4q .. 16n + 4q + 3 of column c.
// So V needs no byte permutes.  Positions past the cached ones are stored as
// zeros.
constexpr int kWgWaves = 4;
constexpr int kWgCols = 16 * 2 * kWgWaves;  // columns per workgroup
typedef short i16x4v __attribute__((ext_vector_type(4)));

// LDS byte offset of (token t, 32-byte column group k) of a V tile
__device__ __forceinline__ int v_tile_off(int t, int k) { return (t * 8 + (k ^ (t & 7))) * 32; }

// 16 bytes at byte `off` (< 4096) of the head tile at `tile` (a uniform
// address): a raw buffer load (descriptor word 3 = 0x00020000: 32-bit data
// format, no swizzle), so the tile's base stays in scalar registers
__device__ __forceinline__ u32x4 load_tile16(const char* tile, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile), 0, kBS * kD * 2, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  const i16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4v*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__global__ __launch_bounds__(64 * kWgWaves, 2) void chunk_mfma_wg_kernel(DecodeArgs a) {
  constexpr int NG = 2;
  // [stage][block of the pair]: K in the score layout, V row-major swizzled
  __shared__ u32x4 k_lds[2][2][kBS * 16];
  __shared__ __align__(16) char v_lds[2][2][kBS * kD * 2];
  const LaneMap L = lane_map();
  const int wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int item = xcd_block(blockIdx.x, gridDim.x);
  const int tile = item % a.chunk_tiles;
  const int h = (item / a.chunk_tiles) % a.H_KV, b = item / a.chunk_tiles / a.H_KV;
  int qs0, n_new, ctx;
  if (!chunk_bounds(a, b, qs0, n_new, ctx)) return;  // uniform over the workgroup
  const int g = a.g, cols = n_new * g, c0w = tile * kWgCols;
  if (c0w >= cols) return;                            // uniform over the workgroup
  const int first = ctx - n_new;
  // this wave's columns (a wave past the chunk still loads and waits)
  const int c0 = c0w + 32 * wave;
  const bool active = c0 < cols;
  const int c_last = min(c0 + 32, cols) - 1;
  const int p_first = first + min(c0, cols - 1) / g, p_last = first + c_last / g;
  const int p_last_wg = first + (min(c0w + kWgCols, cols) - 1) / g;
  const int nblk = p_last_wg / kBS + 1;               // the workgroup's blocks
  const int nblk_w = active ? p_last / kBS + 1 : 0;   // the blocks this wave scores

  bf16x8 qop[NG][4];
  int pcol[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const int col = c0 + 16 * G + L.c;
    pcol[G] = first + min(col, c_last) / g;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(qs0 + min(col, cols - 1) / g) * a.H_Q + h * g +
                            min(col, cols - 1) % g) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col < cols) v = *reinterpret_cast<const u32x4*>(qrow + 32 * j + 8 * L.q4);
      qop[G][j] = __builtin_bit_cast(bf16x8, v);
    }
  }
  Acc<NG> acc;
  acc_init<NG>(acc);

  // loading: thread tid moves 16 bytes (token tid / 16, dims 8 (tid % 16) ..)
  // of K and of V of both blocks of a pair
  const int lt = tid >> 4, lc = tid & 15;
  const int k_wr = lt * 16 + (lc ^ (4 * (lt & 3) + (lt >> 2)));
  const int v_wr = v_tile_off(lt, lc >> 1) + (lc & 1) * 16;
  const size_t head_bytes = static_cast<size_t>(kBS) * kD * 2;
  const size_t blk_bytes = head_bytes * a.H_KV;
  const char* kbase = static_cast<const char*>(a.k_cache) + h * head_bytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + h * head_bytes;
  const uint32_t lane_off = static_cast<uint32_t>(tid) * 16u;
  const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  int win0 = 0;
  int tab = L.lane < nblk ? min(max(row[L.lane], 0), a.num_blocks - 1) : 0;
  auto block_of = [&](int i) {
    if (i - win0 >= 64) {  // uniform, at most once per 64 blocks
      win0 += 64;
      tab = L.lane + win0 < nblk ? min(max(row[L.lane + win0], 0), a.num_blocks - 1) : 0;
    }
    return i < nblk ? __builtin_amdgcn_readlane(tab, i - win0) : 0;
  };
  u32x4 rk[2], rv[2];
  // block addresses are uniform: one scalar base per block, the thread's
  // 16-byte offset in a vector register
  auto load_pair = [&](int p) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const size_t off = static_cast<size_t>(block_of(2 * p + e)) * blk_bytes;
      rk[e] = load_tile16(kbase + off, lane_off);
      rv[e] = load_tile16(vbase + off, lane_off);
    }
  };
  auto store_pair = [&](int p, int st) {
    if ((2 * p + 2) * kBS > ctx) {  // uniform: the pair has uncached positions
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (lt >= ctx - (2 * p + e) * kBS) rk[e] = rv[e] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      k_lds[st][e][k_wr] = rk[e];
      *reinterpret_cast<u32x4*>(&v_lds[st][e][v_wr]) = rv[e];
    }
  };

  // score one block of the pair from the shared K tile
  auto score = [&](const u32x4* kt, int i, float (&s2)[NG][4]) {
    const int t0 = i * kBS;
    const int valid = i < nblk ? min(ctx - t0, kBS) : 0;
    const bool full = valid >= kBS && t0 + kBS - 1 <= p_first;
    bf16x8 ka[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ka[j] = __builtin_bit_cast(bf16x8, kt[L.rpos[j]]);
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qop[G][j], sc, 0, 0, 0);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) s2[G][ii] = sc[ii];
      if (!full) {
        const int lim = min(pcol[G] - t0, valid - 1);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if (L.q4 + 4 * ii > lim) s2[G][ii] = -INFINITY;
      }
    }
  };

  const float kscale = a.scale_log2;
  const int npairs = (nblk + 1) >> 1;
  // tr-read addresses: lane 16q + 4e + j reads token q + 4e, dims 16n + 4j
  const int tr_tok = L.q4 + 4 * ((L.lane & 15) >> 2);
  const int tr_j = L.lane & 3;

  // pair p + 1 is stored after pair p's products (the stage it overwrites
  // held pair p - 1, which every wave finished before the barrier), and pair
  // p + 2 is loaded right after: each pair's loads have a whole step to land
  load_pair(0);
  store_pair(0, 0);
  if (npairs > 1) load_pair(1);
  for (int p = 0; p < npairs; ++p) {
    const int st = p & 1;
    __syncthreads();  // stage st holds pair p; stage st ^ 1 is no longer read
    if (2 * p < nblk_w) {  // uniform per wave: the pair has positions this wave sees
      float sa[NG][4], sb[NG][4];
      score(k_lds[st][0], 2 * p, sa);
      score(k_lds[st][1], 2 * p + 1, sb);
      bf16x8 ph[NG], pl[NG];
#pragma unroll
      for (int G = 0; G < NG; ++G) {
        const float mxa = fmax_fast(fmax_fast(sa[G][0], sa[G][1]), fmax_fast(sa[G][2], sa[G][3]));
        const float mxb = fmax_fast(fmax_fast(sb[G][0], sb[G][1]), fmax_fast(sb[G][2], sb[G][3]));
        // the column max only where the running max moves (see softmax_pv_pair)
        const float ml = fmax_fast(mxa, mxb) * kscale;
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
          pr[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[G][ii], kscale, -acc.m[G]));
          pr[4 + ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[G][ii], kscale, -acc.m[G]));
        }
        acc.l[G] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        u32x4 hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t hh = pack_bf16x2(pr[2 * k], pr[2 * k + 1]);
          hi[k] = hh;
          lo[k] = pack_bf16x2(pr[2 * k] - __uint_as_float(hh << 16),
                              pr[2 * k + 1] - __uint_as_float(hh & 0xffff0000u));
        }
        ph[G] = __builtin_bit_cast(bf16x8, hi);
        pl[G] = __builtin_bit_cast(bf16x8, lo);
      }
      const char* va = v_lds[st][0];
      const char* vb = v_lds[st][1];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int off = v_tile_off(tr_tok, n) + 8 * tr_j;
        const u32x2 x = lds_read_tr16(va + off), y = lds_read_tr16(vb + off);
        const bf16x8 v8 = __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, y.x, y.y});
#pragma unroll
        for (int G = 0; G < NG; ++G) {
          acc.o[G][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, ph[G], acc.o[G][n], 0, 0, 0);
          acc.o[G][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pl[G], acc.o[G][n], 0, 0, 0);
        }
      }
    }
    if (p + 1 < npairs) {
      store_pair(p + 1, st ^ 1);
      if (p + 2 < npairs) load_pair(p + 2);
    }
  }

  // normalised outputs: lane l holds column 16G + c, dims 16n + 4q .. + 3
  if (!active) return;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float l_tot = acc.l[G] + __shfl_xor(acc.l[G], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int col = c0 + 16 * G + L.c;
    if (col >= cols) continue;
    float* dst = a.out + (static_cast<size_t>(qs0 + col / g) * a.H_Q + h * g + col % g) * kD;
    const float mul = 1.0f / l_tot;
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<f32x4*>(dst + 16 * n + 4 * L.q4) = acc.o[G][n] * mul;
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
  if (kv_dtype == DT_BF16) {
    const long long wtiles = (cols + kWgCols - 1) / kWgCols;
    const long long witems = wtiles * a.H_KV * a.B;
    if (witems > 0x7fffffffLL) return hipErrorInvalidValue;
    ta.chunk_tiles = static_cast<int32_t>(wtiles);
    hipLaunchKernelGGL(chunk_mfma_wg_kernel, dim3(static_cast<unsigned>(witems)),
                       dim3(64 * kWgWaves), 0, stream, ta);
  } else
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
