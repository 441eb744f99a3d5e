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

// Partial results of one (request, query head, partition), shared by the
// partition kernels and the combine kernel:
//   ws_o [B][H_Q][max_parts][d_h]  unnormalised sum_t 2^(s2_t - m) V_t
//   ws_ml[B][H_Q][max_parts][2]    (m, l) with m = max_t s2_t and
//                                  l = sum_t 2^(s2_t - m),
// where s2_t = softmax_scale * log2(e) * q . k_t (log2 units).
struct Workspace {
  float* o;
  float* ml;
};

__host__ __device__ inline size_t ws_o_floats(int B, int H_Q, int parts, int d_h) {
  return static_cast<size_t>(B) * H_Q * parts * d_h;
}
__host__ __device__ inline size_t ws_ml_floats(int B, int H_Q, int parts) {
  return static_cast<size_t>(B) * H_Q * parts * 2;
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
  Workspace ws;
  int32_t max_blocks_per_seq;
  int32_t B, H_Q, H_KV, g, d_h, block_size, num_blocks;
  int32_t partition_tokens, max_parts;
  float scale_log2;  // softmax_scale * log2(e)
};

}  // namespace pkv
