// C ABI entry points for the device path: argument checks on the host, the
// partition plan, and the kernel launches.  See include/pkv.h for the
// contract of each function.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>

#include "pkv.h"
#include "pkv_device.h"

namespace pkv {
hipError_t launch_kv_append(int in_dtype, int kv_dtype, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const float* k_scale,
                            const float* v_scale, const int32_t* block_table,
                            int max_blocks_per_seq, const int32_t* context_lens,
                            const int32_t* query_start, int B, int rows, int H_KV, int d_h,
                            int block_size, int num_blocks, hipStream_t stream);
hipError_t launch_swap(bool to_host, void* k_cache, void* v_cache, float* k_scale,
                       float* v_scale, const int32_t* blocks, int n, size_t blk_bytes,
                       size_t rec_bytes, int H_KV, int num_blocks, void* records,
                       hipStream_t stream);
bool chunk_mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size);
hipError_t launch_chunk_mfma(int kv_dtype, int max_q_len, const DecodeArgs& a,
                             hipStream_t stream);
hipError_t launch_chunk_generic(int q_dtype, int kv_dtype, const DecodeArgs& a,
                                hipStream_t stream);
hipError_t launch_decode_generic(int q_dtype, int kv_dtype, const DecodeArgs& a,
                                 hipStream_t stream);
size_t generic_lds_bytes(int g, int d_h, int partition_tokens);
bool mfma_supports(int q_dtype, int kv_dtype, int d_h, int block_size, int g);
bool mfma_fuses_append(int kv_dtype, int g, bool flat, bool cascade);
int mfma_flat_waves(int kv_dtype, int g, int B, bool cascade);
hipError_t launch_decode_mfma(int kv_dtype, bool flat, int waves, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int n_pairs, size_t block_bytes, int H_KV,
                              int num_blocks, hipStream_t stream);
hipError_t launch_combine(float* out, const int32_t* context_lens, const void* ws,
                          size_t ws_bytes, int B, int H_Q, int H_KV, int d_h, int partition_tokens,
                          int max_parts, int prefix_splits, hipStream_t stream);
}  // namespace pkv

namespace {

std::atomic<int> g_variant{PKV_VARIANT_AUTO};  // read and set from any thread

constexpr int kMaxDh = 256;
constexpr int kMaxGenericPartition = 256;
constexpr size_t kMaxGenericLds = 64 * 1024;

bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_BF16 || d == PKV_FP8_E4M3; }

// Default partition length: enough workgroups to cover the chip several
// times over, but no shorter than 4 blocks and no longer than 256 positions
// (the longest partition both kernels take).
int default_partition(int B, int H_KV, int block_size, int max_context_len) {
  const long long target_groups = 4LL * 256;  // 256 compute units
  const long long heads = static_cast<long long>(B) * H_KV;
  int pt = 256;
  while (pt > 4 * block_size && pt > block_size &&
         heads * ((max_context_len + pt - 1) / pt) < target_groups)
    pt /= 2;
  pt = std::max(block_size, pt / block_size * block_size);
  return pt;
}

int resolve_partition(int B, int H_KV, int block_size, int max_context_len, int requested) {
  if (requested > 0) return requested;
  return default_partition(B, H_KV, block_size, max_context_len);
}

// Largest batch the flat kernel takes: its per-request block prefix lives in
// LDS (4 bytes per request).
constexpr int kMaxFlatBatch = 8192;
constexpr int kMfmaMaxPartition = 64 * 16;

enum Kernel { K_GENERIC = 0, K_MFMA_PARTITION = 1, K_MFMA_FLAT = 2 };

struct Plan {
  Kernel kernel;
  int partition_tokens;
  int max_parts;
  int waves;      // flat kernel grid
  size_t total;   // workspace bytes (0: none needed)
};

int flat_waves_cached(int kv_dtype, int g, int B, bool cascade = false) {
  // the occupancy query depends on the kernel instance and its LDS size
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = -1;
  }
  const auto key = std::make_tuple(dev, kv_dtype, g, cascade ? 1 : 0, B);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int w = pkv::mfma_flat_waves(kv_dtype, g, B, cascade);
  // PKV_FLAT_WAVES overrides the grid size of the balanced split, for tuning
  // measurements (more waves than fit at once only adds a second round)
  if (const char* e = std::getenv("PKV_FLAT_WAVES")) {
    const int v = std::atoi(e);
    if (v >= 1 && v <= (1 << 20)) w = v;
  }
  cache[key] = w;
  return w;
}

// The variant is read once by each entry point (current_variant) and passed
// down, so every decision of one call -- plan, kernel, combine -- sees the
// same value even while another thread changes the setting.
int current_variant() { return g_variant.load(std::memory_order_relaxed); }

int make_plan(int variant, int B, int H_Q, int H_KV, int d_h, int block_size,
              int max_context_len, int partition_tokens, int q_dtype, int kv_dtype, Plan* plan) {
  if (B < 1 || H_Q < 1 || H_KV < 1 || H_Q % H_KV || d_h < 1 || d_h > kMaxDh || block_size < 1 ||
      max_context_len < 1 || partition_tokens < 0 || !valid_dtype(q_dtype) ||
      !valid_dtype(kv_dtype))
    return PKV_ERR_INVALID_ARG;
  if (B > 65535 || H_KV > 65535 || H_Q > 65535) return PKV_ERR_INVALID_ARG;
  const int g = H_Q / H_KV;
  const int pt = resolve_partition(B, H_KV, block_size, max_context_len, partition_tokens);
  if (pt % block_size) return PKV_ERR_INVALID_ARG;
  plan->partition_tokens = pt;
  plan->max_parts = (max_context_len + pt - 1) / pt;
  if (plan->max_parts > 65535) return PKV_ERR_INVALID_ARG;  // grid.x of the launch
  plan->waves = 0;

  const bool mfma_ok = pkv::mfma_supports(q_dtype, kv_dtype, d_h, block_size, g);
  switch (variant) {
    case PKV_VARIANT_GENERIC:
      plan->kernel = K_GENERIC;
      break;
    case PKV_VARIANT_MFMA:
      if (!mfma_ok || B > kMaxFlatBatch) return PKV_ERR_UNSUPPORTED;
      plan->kernel = K_MFMA_FLAT;
      break;
    case PKV_VARIANT_MFMA_PARTITION:
      if (!mfma_ok) return PKV_ERR_UNSUPPORTED;
      plan->kernel = K_MFMA_PARTITION;
      break;
    default:
      plan->kernel = !mfma_ok ? K_GENERIC : (B <= kMaxFlatBatch ? K_MFMA_FLAT : K_MFMA_PARTITION);
  }
  if (plan->kernel == K_GENERIC &&
      (pt > kMaxGenericPartition || pkv::generic_lds_bytes(g, d_h, pt) > kMaxGenericLds))
    return PKV_ERR_UNSUPPORTED;
  if (plan->kernel == K_MFMA_PARTITION && pt > kMfmaMaxPartition) return PKV_ERR_UNSUPPORTED;

  if (plan->kernel == K_MFMA_FLAT) {
    plan->waves = flat_waves_cached(kv_dtype, g, B);
    plan->total = pkv::flat_layout(B, plan->waves, g, d_h).total;
  } else if (plan->max_parts == 1) {
    plan->total = 0;
  } else {
    plan->total = pkv::partition_layout(B, H_Q, plan->max_parts, d_h).total;
  }
  return PKV_OK;
}

int check_attention_args(const float* out, const void* q, int q_dtype, const void* k_cache,
                         const void* v_cache, int kv_dtype, const float* k_scale,
                         const float* v_scale, const int32_t* block_table,
                         int max_blocks_per_seq, const int32_t* context_lens,
                         int max_context_len, int B, int H_Q, int H_KV, int d_h, int block_size,
                         int num_blocks, float softmax_scale) {
  if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype) || q_dtype == PKV_FP8_E4M3)
    return PKV_ERR_INVALID_ARG;
  if (B < 1 || H_Q < 1 || H_KV < 1 || H_Q % H_KV || d_h < 1 || d_h > kMaxDh || block_size < 1 ||
      num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 1)
    return PKV_ERR_INVALID_ARG;
  // positions are int32: a table row may span at most INT32_MAX of them
  if (static_cast<long long>(max_blocks_per_seq) * block_size > INT32_MAX)
    return PKV_ERR_INVALID_ARG;
  if (static_cast<long long>(max_context_len) >
      static_cast<long long>(max_blocks_per_seq) * block_size)
    return PKV_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return PKV_ERR_INVALID_ARG;
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  const bool pair_ok = (q_dtype == PKV_F32 && kv_dtype == PKV_F32) ||
                       (q_dtype == PKV_BF16 && kv_dtype == PKV_BF16) ||
                       (q_dtype == PKV_BF16 && kv_dtype == PKV_FP8_E4M3);
  if (!pair_ok) return PKV_ERR_UNSUPPORTED;
  // 16-byte row alignment is assumed by the vector loads of the MFMA kernel
  const uintptr_t align_mask = 15;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out)) &
      align_mask)
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PKV_ERR_BAD_BLOCK: return "bad block";
    case PKV_ERR_SHARED_BLOCK: return "shared block";
    case PKV_ERR_HIP: return "HIP error";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

int pkv_abi_version(void) { return 2; }

int pkv_set_decode_variant(int variant) {
  if (variant == PKV_VARIANT_AUTO || variant == PKV_VARIANT_GENERIC ||
      variant == PKV_VARIANT_MFMA || variant == PKV_VARIANT_MFMA_PARTITION)
    return g_variant.exchange(variant, std::memory_order_relaxed);
  return g_variant.load(std::memory_order_relaxed);
}

}  // extern "C"

namespace {

int check_append_args(const void* k_new, const void* v_new, int in_dtype, void* k_cache,
                      void* v_cache, int kv_dtype, const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t B, int32_t H_KV, int32_t d_h,
                      int32_t block_size, int32_t num_blocks) {
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype) || !valid_dtype(kv_dtype) || in_dtype == PKV_FP8_E4M3)
    return PKV_ERR_INVALID_ARG;
  if (B < 1 || H_KV < 1 || d_h < 1 || d_h > kMaxDh || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return PKV_ERR_INVALID_ARG;
  if (static_cast<long long>(max_blocks_per_seq) * block_size > INT32_MAX)
    return PKV_ERR_INVALID_ARG;  // positions are int32
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  const bool pair_ok = (in_dtype == kv_dtype) || kv_dtype == PKV_FP8_E4M3;
  if (!pair_ok) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_kv_append(const void* k_new, const void* v_new, int in_dtype, void* k_cache,
                  void* v_cache, int kv_dtype, const float* k_scale, const float* v_scale,
                  const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t B, int32_t H_KV, int32_t d_h,
                  int32_t block_size, int32_t num_blocks, pkv_stream_t stream) {
  const int st = check_append_args(k_new, v_new, in_dtype, k_cache, v_cache, kv_dtype, k_scale,
                                   v_scale, block_table, max_blocks_per_seq, context_lens, B,
                                   H_KV, d_h, block_size, num_blocks);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_kv_append(in_dtype, kv_dtype, k_new, v_new, k_cache, v_cache,
                                          k_scale, v_scale, block_table, max_blocks_per_seq,
                                          context_lens, nullptr, B, B, H_KV, d_h, block_size,
                                          num_blocks, static_cast<hipStream_t>(stream)));
}

int pkv_kv_append_chunk(const void* k_new, const void* v_new, int in_dtype, void* k_cache,
                        void* v_cache, int kv_dtype, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, const int32_t* query_start, int32_t B,
                        int32_t total_tokens, int32_t H_KV, int32_t d_h, int32_t block_size,
                        int32_t num_blocks, pkv_stream_t stream) {
  const int st = check_append_args(k_new, v_new, in_dtype, k_cache, v_cache, kv_dtype, k_scale,
                                   v_scale, block_table, max_blocks_per_seq, context_lens, B,
                                   H_KV, d_h, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (!query_start || total_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (total_tokens == 0) return PKV_OK;
  return hip_status(pkv::launch_kv_append(in_dtype, kv_dtype, k_new, v_new, k_cache, v_cache,
                                          k_scale, v_scale, block_table, max_blocks_per_seq,
                                          context_lens, query_start, B, total_tokens, H_KV, d_h,
                                          block_size, num_blocks,
                                          static_cast<hipStream_t>(stream)));
}

int pkv_paged_chunk_attention(float* out, const void* q, int q_dtype, const void* k_cache,
                              const void* v_cache, int kv_dtype, const float* k_scale,
                              const float* v_scale, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              const int32_t* query_start, int32_t B, int32_t total_q,
                              int32_t max_q_len, int32_t max_context_len, int32_t H_Q,
                              int32_t H_KV, int32_t d_h, int32_t block_size, int32_t num_blocks,
                              float softmax_scale, pkv_stream_t stream) {
  int st = check_attention_args(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                block_table, max_blocks_per_seq, context_lens, max_context_len,
                                B, H_Q, H_KV, d_h, block_size, num_blocks, softmax_scale);
  if (st != PKV_OK) return st;
  if (!query_start || total_q < 0 || max_q_len < 1 || max_q_len > max_context_len ||
      B > 65535 || H_Q > 65535)
    return PKV_ERR_INVALID_ARG;
  if (total_q == 0) return PKV_OK;

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.B = B;
  a.H_Q = H_Q;
  a.H_KV = H_KV;
  a.g = H_Q / H_KV;
  a.d_h = d_h;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.scale_log2 = softmax_scale * pkv::kLog2e;
  a.query_start = query_start;
  a.total_q = total_q;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool mfma = current_variant() != PKV_VARIANT_GENERIC &&
                    pkv::chunk_mfma_supports(q_dtype, kv_dtype, d_h, block_size);
  return hip_status(mfma ? pkv::launch_chunk_mfma(kv_dtype, max_q_len, a, s)
                         : pkv::launch_chunk_generic(q_dtype, kv_dtype, a, s));
}

int pkv_copy_blocks(void* k_cache, void* v_cache, int kv_dtype, float* k_scale, float* v_scale,
                    const int32_t* pairs, int32_t n_pairs, int32_t H_KV, int32_t d_h,
                    int32_t block_size, int32_t num_blocks, pkv_stream_t stream) {
  if (!k_cache || !v_cache || !pairs || n_pairs < 0 || !valid_dtype(kv_dtype) || H_KV < 1 ||
      d_h < 1 || d_h > kMaxDh || block_size < 1 || num_blocks < 1)
    return PKV_ERR_INVALID_ARG;
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (n_pairs == 0) return PKV_OK;
  if (n_pairs > 2147483647 / 2) return PKV_ERR_INVALID_ARG;
  const size_t elem = kv_dtype == PKV_F32 ? 4 : (kv_dtype == PKV_BF16 ? 2 : 1);
  const size_t block_bytes = static_cast<size_t>(H_KV) * block_size * d_h * elem;
  return hip_status(pkv::launch_copy_blocks(
      k_cache, v_cache, kv_dtype == PKV_FP8_E4M3 ? k_scale : nullptr,
      kv_dtype == PKV_FP8_E4M3 ? v_scale : nullptr, pairs, n_pairs, block_bytes, H_KV,
      num_blocks, static_cast<hipStream_t>(stream)));
}

int pkv_decode_plan(int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                    int32_t max_context_len, int32_t partition_tokens, int q_dtype, int kv_dtype,
                    int32_t* partition_tokens_out, int32_t* max_partitions_out,
                    size_t* workspace_bytes) {
  Plan plan;
  const int st = make_plan(current_variant(), B, H_Q, H_KV, d_h, block_size, max_context_len,
                           partition_tokens, q_dtype, kv_dtype, &plan);
  if (st != PKV_OK) return st;
  if (partition_tokens_out) *partition_tokens_out = plan.partition_tokens;
  if (max_partitions_out) *max_partitions_out = plan.max_parts;
  if (workspace_bytes) *workspace_bytes = plan.total;
  return PKV_OK;
}

int pkv_decode_workspace_size(int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h,
                              int32_t block_size, int32_t max_context_len,
                              int32_t partition_tokens, int q_dtype, int kv_dtype,
                              size_t* workspace_bytes) {
  if (!workspace_bytes) return PKV_ERR_INVALID_ARG;
  // the largest workspace any kernel variant needs for these shapes, so the
  // size holds whatever the process-wide variant is when the call runs
  size_t most = 0;
  bool any = false;
  for (const int v : {PKV_VARIANT_AUTO, PKV_VARIANT_GENERIC, PKV_VARIANT_MFMA,
                      PKV_VARIANT_MFMA_PARTITION}) {
    Plan plan;
    const int st = make_plan(v, B, H_Q, H_KV, d_h, block_size, max_context_len,
                             partition_tokens, q_dtype, kv_dtype, &plan);
    if (st == PKV_ERR_UNSUPPORTED) continue;
    if (st != PKV_OK) return st;  // the shapes themselves are invalid
    most = std::max(most, plan.total);
    any = true;
  }
  if (!any) return PKV_ERR_UNSUPPORTED;
  *workspace_bytes = most;
  return PKV_OK;
}

}  // extern "C"

namespace {

// The partition launch; with k_new / v_new set (MFMA kernels only) the
// owning waves also append the new token (see pkv_decode_step).
int decode_launch(int variant, Plan* plan_out, const void* k_new, const void* v_new, float* out,
                  const void* q, int q_dtype,
                  const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                  const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_Q,
                  int32_t H_KV, int32_t d_h, int32_t block_size, int32_t num_blocks,
                  float softmax_scale, int32_t partition_tokens, void* workspace,
                  size_t workspace_bytes, pkv_stream_t stream) {
  int st = check_attention_args(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                block_table, max_blocks_per_seq, context_lens, max_context_len,
                                B, H_Q, H_KV, d_h, block_size, num_blocks, softmax_scale);
  if (st != PKV_OK) return st;
  Plan plan;
  st = make_plan(variant, B, H_Q, H_KV, d_h, block_size, max_context_len, partition_tokens,
                 q_dtype, kv_dtype, &plan);
  if (st != PKV_OK) return st;
  if (plan_out) *plan_out = plan;
  if (plan.total > 0 && (!workspace || workspace_bytes < plan.total)) return PKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return PKV_ERR_INVALID_ARG;
  // a workspace too small to hold the header is not used at all
  if (workspace_bytes < pkv::kWsHeader) workspace = nullptr;

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.ws = static_cast<char*>(workspace);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.B = B;
  a.H_Q = H_Q;
  a.H_KV = H_KV;
  a.g = H_Q / H_KV;
  a.d_h = d_h;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.partition_tokens = plan.partition_tokens;
  a.max_parts = plan.max_parts;
  a.scale_log2 = softmax_scale * pkv::kLog2e;
  a.k_new = k_new;
  a.v_new = v_new;
  if (k_new && (!pkv::mfma_fuses_append(kv_dtype, H_Q / H_KV, plan.kernel == K_MFMA_FLAT, false) ||
                (plan.kernel != K_MFMA_FLAT && plan.kernel != K_MFMA_PARTITION)))
    return PKV_ERR_UNSUPPORTED;

  hipError_t e;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (plan.kernel) {
    case K_MFMA_FLAT:
      e = pkv::launch_decode_mfma(kv_dtype, true, plan.waves, a, s);
      break;
    case K_MFMA_PARTITION:
      e = pkv::launch_decode_mfma(kv_dtype, false, 0, a, s);
      break;
    default:
      e = pkv::launch_decode_generic(q_dtype, kv_dtype, a, s);
  }
  return hip_status(e);
}


}  // namespace

extern "C" {

int pkv_decode_partitions(float* out, const void* q, int q_dtype, const void* k_cache,
                          const void* v_cache, int kv_dtype, const float* k_scale,
                          const float* v_scale, const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t max_context_len, int32_t B, int32_t H_Q, int32_t H_KV,
                          int32_t d_h, int32_t block_size, int32_t num_blocks,
                          float softmax_scale, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, pkv_stream_t stream) {
  return decode_launch(current_variant(), nullptr, nullptr, nullptr, out, q, q_dtype, k_cache,
                       v_cache, kv_dtype, k_scale, v_scale, block_table, max_blocks_per_seq,
                       context_lens, max_context_len, B, H_Q, H_KV, d_h, block_size, num_blocks,
                       softmax_scale, partition_tokens, workspace, workspace_bytes, stream);
}

int pkv_combine_partitions(float* out, const int32_t* context_lens, int32_t max_context_len,
                           int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h,
                           int32_t block_size, int32_t partition_tokens, const void* workspace,
                           size_t workspace_bytes, pkv_stream_t stream) {
  if (!out || !context_lens) return PKV_ERR_INVALID_ARG;
  if (B < 1 || H_Q < 1 || H_KV < 1 || H_Q % H_KV || d_h < 1 || d_h > kMaxDh || block_size < 1 ||
      max_context_len < 1 || partition_tokens < 0 || B > 65535 || H_Q > 65535)
    return PKV_ERR_INVALID_ARG;
  // without a workspace no partial can exist: the partition call wrote out
  if (!workspace || workspace_bytes < pkv::kWsHeader) return PKV_OK;
  // the combine reads and writes 16-byte vectors
  if ((reinterpret_cast<uintptr_t>(workspace) | reinterpret_cast<uintptr_t>(out)) & 15)
    return PKV_ERR_INVALID_ARG;
  const int pt = resolve_partition(B, H_KV, block_size, max_context_len, partition_tokens);
  if (pt % block_size) return PKV_ERR_INVALID_ARG;
  const int max_parts = (max_context_len + pt - 1) / pt;
  // the workspace header written by the partition call selects the layout
  return hip_status(pkv::launch_combine(out, context_lens, workspace, workspace_bytes, B, H_Q,
                                        H_KV, d_h, pt, max_parts, 0,
                                        static_cast<hipStream_t>(stream)));
}

int pkv_paged_decode_attention(float* out, const void* q, int q_dtype, const void* k_cache,
                               const void* v_cache, int kv_dtype, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, int32_t B, int32_t H_Q, int32_t H_KV,
                               int32_t d_h, int32_t block_size, int32_t num_blocks,
                               float softmax_scale, int32_t partition_tokens, void* workspace,
                               size_t workspace_bytes, pkv_stream_t stream) {
  Plan plan;
  const int st = decode_launch(current_variant(), &plan, nullptr, nullptr, out, q, q_dtype,
                               k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table,
                               max_blocks_per_seq, context_lens, max_context_len, B, H_Q, H_KV,
                               d_h, block_size, num_blocks, softmax_scale, partition_tokens,
                               workspace, workspace_bytes, stream);
  if (st != PKV_OK) return st;
  if (plan.total == 0) return PKV_OK;  // one partition per request: out is final
  return pkv_combine_partitions(out, context_lens, max_context_len, B, H_Q, H_KV, d_h,
                                block_size, partition_tokens, workspace, workspace_bytes,
                                stream);
}

int pkv_decode_step(const void* k_new, const void* v_new, float* out, const void* q, int q_dtype,
                    void* k_cache, void* v_cache, int kv_dtype, const float* k_scale,
                    const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_Q,
                    int32_t H_KV, int32_t d_h, int32_t block_size, int32_t num_blocks,
                    float softmax_scale, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, pkv_stream_t stream) {
  int st = check_attention_args(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                block_table, max_blocks_per_seq, context_lens, max_context_len,
                                B, H_Q, H_KV, d_h, block_size, num_blocks, softmax_scale);
  if (st != PKV_OK) return st;
  st = check_append_args(k_new, v_new, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                         block_table, max_blocks_per_seq, context_lens, B, H_KV, d_h,
                         block_size, num_blocks);
  if (st != PKV_OK) return st;
  const int variant = current_variant();
  Plan plan;
  st = make_plan(variant, B, H_Q, H_KV, d_h, block_size, max_context_len, partition_tokens,
                 q_dtype, kv_dtype, &plan);
  if (st != PKV_OK) return st;
  // every check before the first launch: a workspace the attention launch
  // would refuse must not leave the append done
  if (plan.total > 0 && (!workspace || workspace_bytes < plan.total)) return PKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return PKV_ERR_INVALID_ARG;
  const bool aligned =
      ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15) == 0;
  const bool fused = aligned &&
                     pkv::mfma_fuses_append(kv_dtype, H_Q / H_KV, plan.kernel == K_MFMA_FLAT, false) &&
                     (plan.kernel == K_MFMA_FLAT || plan.kernel == K_MFMA_PARTITION);
  if (!fused) {
    st = pkv_kv_append(k_new, v_new, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                       block_table, max_blocks_per_seq, context_lens, B, H_KV, d_h, block_size,
                       num_blocks, stream);
    if (st != PKV_OK) return st;
  }
  st = decode_launch(variant, nullptr, fused ? k_new : nullptr, fused ? v_new : nullptr, out, q,
                     q_dtype, k_cache,
                     v_cache, kv_dtype, k_scale, v_scale, block_table, max_blocks_per_seq,
                     context_lens, max_context_len, B, H_Q, H_KV, d_h, block_size, num_blocks,
                     softmax_scale, partition_tokens, workspace, workspace_bytes, stream);
  if (st != PKV_OK || plan.total == 0) return st;
  return pkv_combine_partitions(out, context_lens, max_context_len, B, H_Q, H_KV, d_h,
                                block_size, partition_tokens, workspace, workspace_bytes,
                                stream);
}

int pkv_swap_record_bytes(int kv_dtype, int32_t H_KV, int32_t d_h, int32_t block_size,
                          size_t* block_bytes, size_t* record_bytes) {
  if (!valid_dtype(kv_dtype) || H_KV < 1 || d_h < 1 || d_h > kMaxDh || block_size < 1 ||
      !record_bytes)
    return PKV_ERR_INVALID_ARG;
  const size_t elem = kv_dtype == PKV_F32 ? 4 : (kv_dtype == PKV_BF16 ? 2 : 1);
  const size_t blk = static_cast<size_t>(H_KV) * block_size * d_h * elem;
  const size_t rec = 2 * blk + (kv_dtype == PKV_FP8_E4M3 ? 2 * sizeof(float) * H_KV : 0);
  if (block_bytes) *block_bytes = blk;
  *record_bytes = (rec + 255) / 256 * 256;
  return PKV_OK;
}

}  // extern "C"

namespace {

// Device address of a record buffer: device memory as is, pinned host
// memory through its device mapping; anything else (pageable host memory)
// is refused.
int device_view(const void* p, void** out) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_INVALID_ARG;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = const_cast<void*>(p);
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return PKV_ERR_INVALID_ARG;
    }
    *out = d;
    return PKV_OK;
  }
  return PKV_ERR_INVALID_ARG;
}

int swap_common(bool to_host, void* k_cache, void* v_cache, int kv_dtype, float* k_scale,
                float* v_scale, const int32_t* blocks, int32_t n, int32_t H_KV, int32_t d_h,
                int32_t block_size, int32_t num_blocks, const void* records,
                pkv_stream_t stream) {
  if (!k_cache || !v_cache || !blocks || !records || n < 0 || num_blocks < 1)
    return PKV_ERR_INVALID_ARG;
  size_t blk = 0, rec = 0;
  int st = pkv_swap_record_bytes(kv_dtype, H_KV, d_h, block_size, &blk, &rec);
  if (st != PKV_OK) return st;
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  void* dev = nullptr;
  st = device_view(records, &dev);
  if (st != PKV_OK) return st;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  return hip_status(pkv::launch_swap(to_host, k_cache, v_cache, fp8 ? k_scale : nullptr,
                                     fp8 ? v_scale : nullptr, blocks, n, blk, rec, H_KV,
                                     num_blocks, dev, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pkv_swap_out(const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                 const float* v_scale, const int32_t* blocks, int32_t n, int32_t H_KV,
                 int32_t d_h, int32_t block_size, int32_t num_blocks, void* records,
                 pkv_stream_t stream) {
  return swap_common(true, const_cast<void*>(k_cache), const_cast<void*>(v_cache), kv_dtype,
                     const_cast<float*>(k_scale), const_cast<float*>(v_scale), blocks, n, H_KV,
                     d_h, block_size, num_blocks, records, stream);
}

int pkv_swap_in(void* k_cache, void* v_cache, int kv_dtype, float* k_scale, float* v_scale,
                const int32_t* blocks, int32_t n, int32_t H_KV, int32_t d_h, int32_t block_size,
                int32_t num_blocks, const void* records, pkv_stream_t stream) {
  return swap_common(false, k_cache, v_cache, kv_dtype, k_scale, v_scale, blocks, n, H_KV, d_h,
                     block_size, num_blocks, records, stream);
}

}  // extern "C"

namespace {

// Launch shape of a cascade.  The flat kernel's grid G (sized by occupancy:
// one workgroup per SIMD for bf16) is shared by the prefix workgroups and the
// private chunks, so every workgroup is resident from the start: on the
// shared-prefix batch (64 requests, 75 shared blocks) any grid beyond G cost
// 8-13% of the kernel time.  The shared blocks are split so that a prefix
// workgroup walks about as many blocks as a private chunk: the total work,
// tiles x shared blocks of prefix plus the private blocks, spread over G.
// The host knows only the longest context, so the private blocks are
// estimated as 3/4 of B x H_KV x (blocks of the longest context - shared
// blocks); the prefix takes at most half the grid.  Measured on that batch
// (kernel us, prefix splits / private chunks): 1 / 960: 68.8 (the prefix
// walks become the longest), 2 / 896: 48.8, 3 / 832: 50.1, 4 / 768: 50.6;
// 4 / 1024: 51.6.
struct CascadeShape {
  int splits;   // prefix splits (no empty split)
  int chunks;   // private chunks of the balanced split
};

CascadeShape cascade_shape(int grid, int B, int g, int H_KV, int shared_blocks, int block_size,
                           int max_context_len) {
  const long long tiles = (static_cast<long long>(B) * g + 31) / 32 * H_KV;
  const long long ctx_blocks = (static_cast<long long>(max_context_len) + block_size - 1) / block_size;
  const long long priv = static_cast<long long>(B) * H_KV *
                         std::max<long long>(ctx_blocks - shared_blocks, 0) * 3 / 4;
  const long long per_slot =
      std::max<long long>((tiles * shared_blocks + priv) / std::max(grid, 1), 1);
  long long want = (shared_blocks + per_slot - 1) / per_slot;
  // at most half the grid for the prefix, so the private chunks keep the
  // other half and the launch still fits the grid
  want = std::min<long long>(want, std::max<long long>(grid / 2 / tiles, 1));
  want = std::max<long long>(std::min<long long>(want, shared_blocks), 1);
  const int bps = static_cast<int>((shared_blocks + want - 1) / want);
  CascadeShape c;
  c.splits = (shared_blocks + bps - 1) / bps;
  const long long prefix_waves = c.splits * tiles;
  c.chunks = static_cast<int>(std::max<long long>(grid - prefix_waves, grid / 2));
  c.chunks = std::max(c.chunks, 1);
  return c;
}

int cascade_plan(int variant, int B, int H_Q, int H_KV, int d_h, int block_size,
                 int max_context_len, int shared_blocks, int q_dtype, int kv_dtype, Plan* plan,
                 int* splits, size_t* ws) {
  int st = make_plan(variant, B, H_Q, H_KV, d_h, block_size, max_context_len, 0, q_dtype,
                     kv_dtype, plan);
  if (st != PKV_OK) return st;
  if (plan->kernel != K_MFMA_FLAT) return PKV_ERR_UNSUPPORTED;
  if (shared_blocks < 1 || static_cast<long long>(shared_blocks) * block_size > max_context_len)
    return PKV_ERR_INVALID_ARG;
  // the cascade launches the flat kernel's cascade variant: size its grid
  // (and the layout) by that kernel's occupancy
  const CascadeShape c =
      cascade_shape(flat_waves_cached(kv_dtype, H_Q / H_KV, B, true), B, H_Q / H_KV, H_KV,
                    shared_blocks, block_size, max_context_len);
  plan->waves = c.chunks;
  *splits = c.splits;
  *ws = pkv::cascade_layout(B, H_Q, plan->waves, H_Q / H_KV, d_h, *splits).total;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_cascade_plan(int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                     int32_t max_context_len, int32_t shared_blocks, int q_dtype, int kv_dtype,
                     int32_t* splits_out, size_t* workspace_bytes) {
  Plan plan;
  int splits = 0;
  size_t ws = 0;
  const int st = cascade_plan(current_variant(), B, H_Q, H_KV, d_h, block_size,
                              max_context_len, shared_blocks, q_dtype, kv_dtype, &plan, &splits,
                              &ws);
  if (st != PKV_OK) return st;
  if (splits_out) *splits_out = splits;
  if (workspace_bytes) *workspace_bytes = ws;
  return PKV_OK;
}

}  // extern "C"

namespace {

// The cascade step; with_combine = false launches the attention kernel only
// (no append may be asked for then).
int cascade_step(const void* k_new, const void* v_new, float* out, const void* q, int q_dtype,
                 void* k_cache, void* v_cache, int kv_dtype, const float* k_scale,
                 const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_Q,
                 int32_t H_KV, int32_t d_h, int32_t block_size, int32_t num_blocks,
                 float softmax_scale, int32_t shared_blocks, void* workspace,
                 size_t workspace_bytes, pkv_stream_t stream, bool with_combine) {
  int st = check_attention_args(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                block_table, max_blocks_per_seq, context_lens, max_context_len,
                                B, H_Q, H_KV, d_h, block_size, num_blocks, softmax_scale);
  if (st != PKV_OK) return st;
  if (k_new || v_new) {
    st = check_append_args(k_new, v_new, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                           block_table, max_blocks_per_seq, context_lens, B, H_KV, d_h,
                           block_size, num_blocks);
    if (st != PKV_OK) return st;
  }
  Plan plan;
  int splits = 0;
  size_t ws = 0;
  st = cascade_plan(current_variant(), B, H_Q, H_KV, d_h, block_size, max_context_len,
                    shared_blocks, q_dtype, kv_dtype, &plan, &splits, &ws);
  if (st != PKV_OK) return st;
  if (!workspace || workspace_bytes < ws) return PKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return PKV_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused =
      k_new && ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15) == 0 &&
      pkv::mfma_fuses_append(kv_dtype, H_Q / H_KV, true, true);
  if (k_new && !fused) {
    st = pkv_kv_append(k_new, v_new, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                       block_table, max_blocks_per_seq, context_lens, B, H_KV, d_h, block_size,
                       num_blocks, stream);
    if (st != PKV_OK) return st;
  }
  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.ws = static_cast<char*>(workspace);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.B = B;
  a.H_Q = H_Q;
  a.H_KV = H_KV;
  a.g = H_Q / H_KV;
  a.d_h = d_h;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.partition_tokens = plan.partition_tokens;
  a.max_parts = plan.max_parts;
  a.scale_log2 = softmax_scale * pkv::kLog2e;
  a.cascade = 1;
  a.shared_blocks = shared_blocks;
  a.prefix_splits = splits;
  a.waves_for_layout = plan.waves;
  a.prefix_end = std::min(shared_blocks * block_size, max_context_len);
  a.prefix_waves = splits * H_KV * static_cast<int>((static_cast<long long>(B) * (H_Q / H_KV) + 31) / 32);
  if (fused) {
    a.k_new = k_new;
    a.v_new = v_new;
  }
  hipError_t e = pkv::launch_decode_mfma(kv_dtype, true, plan.waves, a, s);
  if (e != hipSuccess || !with_combine) return hip_status(e);
  return hip_status(pkv::launch_combine(out, context_lens, workspace, workspace_bytes, B, H_Q,
                                        H_KV, d_h, plan.partition_tokens, plan.max_parts, splits,
                                        s));
}

}  // namespace

extern "C" {

int pkv_decode_step_cascade(const void* k_new, const void* v_new, float* out, const void* q,
                            int q_dtype, void* k_cache, void* v_cache, int kv_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, int32_t B,
                            int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                            int32_t num_blocks, float softmax_scale, int32_t shared_blocks,
                            void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
  return cascade_step(k_new, v_new, out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                      block_table, max_blocks_per_seq, context_lens, max_context_len, B, H_Q,
                      H_KV, d_h, block_size, num_blocks, softmax_scale, shared_blocks, workspace,
                      workspace_bytes, stream, true);
}

int pkv_cascade_partitions(float* out, const void* q, int q_dtype, const void* k_cache,
                           const void* v_cache, int kv_dtype, const float* k_scale,
                           const float* v_scale, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t B, int32_t H_Q, int32_t H_KV,
                           int32_t d_h, int32_t block_size, int32_t num_blocks,
                           float softmax_scale, int32_t shared_blocks, void* workspace,
                           size_t workspace_bytes, pkv_stream_t stream) {
  return cascade_step(nullptr, nullptr, out, q, q_dtype, const_cast<void*>(k_cache),
                      const_cast<void*>(v_cache), kv_dtype, k_scale, v_scale, block_table,
                      max_blocks_per_seq, context_lens, max_context_len, B, H_Q, H_KV, d_h,
                      block_size, num_blocks, softmax_scale, shared_blocks, workspace,
                      workspace_bytes, stream, false);
}

}  // extern "C"
