// Device-side helpers shared by the HIP kernels of the library (gfx950).
//
// Scalar formats of the cache (page 2 "KV Cache Explained", section "What
// changes when you use FP8 KV": one byte per element plus scales):
//   bf16 -- upper 16 bits of an IEEE float32;
//   fp8  -- OCP E4M3 ("E4M3FN"): sign, 4 exponent bits with bias 7, 3
//           mantissa bits, subnormals m * 2^-9, no infinities, S.1111.111 is
//           NaN, largest finite magnitude 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// E4M3 code -> float32, exact (every E4M3 value is a float32).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t mag = code & 0x7fu;
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t e = mag >> 3, m = mag & 7u;
  float v;
  if (mag == 0x7fu) {
    v = __uint_as_float(0x7fc00000u);                       // NaN
  } else if (e == 0) {
    v = static_cast<float>(m) * 0.001953125f;               // m * 2^-9, exact
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));    // rebias 7 -> 127
  }
  return __uint_as_float(__float_as_uint(v) | sign);
}

// float32 -> E4M3 code: round to nearest, ties to even mantissa, saturate
// to +-448, NaN -> NaN code with the input's sign.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  if (a != a) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {
    // subnormal range (and the bottom of the first normal binade): step 2^-9.
    // a * 512 is exact; rint rounds half to even.  A result of 8 is the code
    // of 2^-6, which is where the normal codes continue.
    return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  }
  // normal: keep 3 of the 23 mantissa bits with round-half-even on the
  // dropped 20 bits; a carry moves into the exponent field as it should.
  const uint32_t ab = bits & 0x7fffffffu;
  const uint32_t r = (ab + 0x7ffffu + ((ab >> 20) & 1u)) >> 20;  // (exp127 << 3) | m
  uint32_t code = r - (120u << 3);
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// Scalar loads of one stored element as float32.
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t idx) {
  if constexpr (DT == DT_F32) {
    return static_cast<const float*>(base)[idx];
  } else if constexpr (DT == DT_BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  } else {
    return e4m3_to_f32(static_cast<const uint8_t*>(base)[idx]);
  }
}

// Workspace of the attention call.  It starts with a 256-byte header the
// partition kernels write and the combine kernel reads, so the combine knows
// which of the two partial layouts it has to merge:
//
//   partition layout (kWsPartition): one partial per (request, query head,
//     partition of partition_tokens positions):
//       o [B][H_Q][max_parts][d_h]   unnormalised sum_t 2^(s2_t - m) V_t
//       ml[B][H_Q][max_parts][2]     (m, l): m = max_t s2_t, l = sum_t 2^(s2_t - m)
//   flat layout (kWsFlat): the blocks of all (request, KV head) sequences,
//     concatenated request-major, are cut into C = min(W, T) equal chunks of
//     at least one block, one per wave (waves w >= C idle);
//     a wave writes at most two partials (slot 0: its first sequence, slot 1:
//     its last one) for the sequences its chunk cuts, each for all g heads:
//       prefix[B + 1]                blocks of requests 0..b-1 (int32)
//       ml[W][2][g][2], o[W][2][g][d_h]
// where s2_t = softmax_scale * log2(e) * q . k_t (log2 units).
constexpr int kWsPartition = 1;
constexpr int kWsFlat = 2;
constexpr size_t kWsHeader = 256;
constexpr size_t kWsAlign = 256;

struct WsHeader {
  int32_t mode;
  int32_t waves;   // flat layout: grid size W (sizes the partial arrays)
  int32_t B;
  int32_t g;
  int32_t chunks;  // flat layout: chunks actually used, min(W, T) (T = total blocks)
};

__host__ __device__ inline size_t ws_align(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct PartitionLayout {
  size_t o, ml, total;  // byte offsets from the workspace start, total size
};
__host__ __device__ inline PartitionLayout partition_layout(int B, int H_Q, int parts, int d_h) {
  PartitionLayout L;
  L.o = kWsHeader;
  L.ml = L.o + ws_align(sizeof(float) * static_cast<size_t>(B) * H_Q * parts * d_h);
  L.total = L.ml + ws_align(sizeof(float) * static_cast<size_t>(B) * H_Q * parts * 2);
  return L;
}

struct FlatLayout {
  size_t prefix, ml, o, total;
};
__host__ __device__ inline FlatLayout flat_layout(int B, int W, int g, int d_h) {
  FlatLayout L;
  L.prefix = kWsHeader;
  L.ml = L.prefix + ws_align(sizeof(int32_t) * (static_cast<size_t>(B) + 1));
  L.o = L.ml + ws_align(sizeof(float) * static_cast<size_t>(W) * 2 * g * 2);
  L.total = L.o + ws_align(sizeof(float) * static_cast<size_t>(W) * 2 * g * d_h);
  return L;
}

// Cascade over a shared prefix (the first `shared` blocks of every request's
// table are the same blocks): after the flat layout, which phase B (the
// private blocks) uses as usual,
//   seq_ml[B*H_Q][2], seq_o[B*H_Q][d_h]   phase B's pieces of the (request,
//                                          head) sequences no wave cut
//   pre_ml[S][B*H_Q][2], pre_o[S][B*H_Q][d_h]
//                                          phase A's pieces: split s of the
//                                          shared blocks, every query head
// all unnormalised (m, l, o) in log2 units like the other pieces.
struct CascadeLayout {
  size_t seq_ml, seq_o, pre_ml, pre_o, total;
};
__host__ __device__ inline CascadeLayout cascade_layout(int B, int H_Q, int W, int g, int d_h,
                                                        int S) {
  const FlatLayout F = flat_layout(B, W, g, d_h);
  const size_t rows = static_cast<size_t>(B) * H_Q;
  CascadeLayout C;
  C.seq_ml = F.total;
  C.seq_o = C.seq_ml + ws_align(sizeof(float) * rows * 2);
  C.pre_ml = C.seq_o + ws_align(sizeof(float) * rows * d_h);
  C.pre_o = C.pre_ml + ws_align(sizeof(float) * S * rows * 2);
  C.total = C.pre_o + ws_align(sizeof(float) * S * rows * d_h);
  return C;
}

// The chunk [floor(w T / C), floor((w + 1) T / C)) holding block x (C <= T,
// so no chunk is empty).
__host__ __device__ inline int flat_wave_of(long long x, long long T, int W) {
  return static_cast<int>(((x + 1) * W - 1) / T);
}
__host__ __device__ inline long long flat_chunk_lo(int w, long long T, int W) {
  return static_cast<long long>(w) * T / W;
}

struct DecodeArgs {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  char* ws;  // workspace base (header first)
  int32_t max_blocks_per_seq;
  int32_t B, H_Q, H_KV, g, d_h, block_size, num_blocks;
  int32_t partition_tokens, max_parts;
  float scale_log2;  // softmax_scale * log2(e)
  // chunk attention only: [B + 1] prefix sum of each request's new tokens
  // (query rows), nullptr for a decode step (one query row per request), and
  // the number of query rows
  const int32_t* query_start;
  int32_t total_q;
  // decode step with the append fused in: [B][H_KV][d_h] new K and V in the
  // query dtype, nullptr when the caller appended them already
  const void* k_new;
  const void* v_new;
  // cascade over a shared prefix: the number of shared leading blocks
  // (phase B skips them, phase A reads only them) and phase A's split count;
  // cascade == 0 for a plain decode
  int32_t cascade;
  int32_t shared_blocks;
  int32_t prefix_splits;
  int32_t waves_for_layout;  // W of the flat layout the cascade regions follow
  int32_t prefix_waves;      // leading workgroups of the flat grid that do prefix work
  int32_t prefix_end;        // positions the prefix work reads: min(shared, max context)
  int32_t chunk_tiles;       // chunk kernel: column tiles per (request, KV head)
};

// Workgroups are dispatched to the 8 XCDs of the device round robin (id i
// runs on XCD i mod 8), and each XCD has its own L2.  xcd_block gives
// workgroup i the logical item that puts a contiguous eighth of the logical
// order on each XCD, so items that read the same data -- the column tiles of
// one request and KV head -- share an L2.  Any device is correct with it;
// only where work lands changes.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int i, int n) {
  const int x = i % kXcds, j = i / kXcds;
  const int q = n / kXcds, r = n % kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// Request of query row r: the last b with query_start[b] <= r (binary
// search; query_start is non-decreasing).  Used by the chunk kernels.
__device__ __forceinline__ int request_of_row(const int32_t* query_start, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (query_start[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace pkv
