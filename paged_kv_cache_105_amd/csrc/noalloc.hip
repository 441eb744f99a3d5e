// pkv_decode_step_noalloc: the decode step with its workspace in a static
// device array, for callers that cannot allocate device memory (code under
// stream capture, tight serving loops, hosts that forbid allocation).
//
// The array lives in this file at file scope, so every GPU the library runs
// on holds its own copy for as long as the process runs.  Host code never
// passes the array's name to a kernel (on the host it only stands for the
// symbol); the device address of the current device's copy is looked up
// once per device with hipGetSymbolAddress and kept, and that address is
// what the decode step receives as its workspace.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "pkv.h"

namespace {

// Upper bound of the step's workspace: the partial results of the split
// (e.g. 2.1 MB for 32 requests of 32 query heads on 8 KV heads, 8.5 MB for
// 128 requests of 32 query heads sharing one KV head).  Shapes that need
// more are refused.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_decode_step_noalloc(const void* k_new, const void* v_new, float* out, const void* q,
                            int q_dtype, void* k_cache, void* v_cache, int kv_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, int32_t B,
                            int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                            int32_t num_blocks, float softmax_scale, int32_t partition_tokens,
                            pkv_stream_t stream) {
  // refuse shapes whose workspace exceeds the array before touching the
  // device (a host-only plan)
  size_t need = 0;
  int st = pkv_decode_plan(B, H_Q, H_KV, d_h, block_size, max_context_len, partition_tokens,
                           q_dtype, kv_dtype, nullptr, nullptr, &need);
  if (st != PKV_OK) return st;
  if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  // pkv_decode_step checks the plan again with the variant it reads and
  // refuses (before any launch) a workspace that is too small
  return pkv_decode_step(k_new, v_new, out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale,
                         v_scale, block_table, max_blocks_per_seq, context_lens,
                         max_context_len, B, H_Q, H_KV, d_h, block_size, num_blocks,
                         softmax_scale, partition_tokens, ws, kScratchBytes, stream);
}

}  // extern "C"
