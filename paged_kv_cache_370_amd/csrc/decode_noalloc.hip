// paged_attention_decode for callers that cannot allocate device memory:
// the decode workspace (work-queue counters and split partials) is a
// file-scope device array instead of a caller buffer.
//
// Each device the library runs on holds its own copy of `scratch` until the
// process ends.  Its address is looked up once per device (with that device
// current) and every kernel argument uses that address, never the array's
// host-side name.  All calls on one device share the array: calls that may
// overlap on one device race, and must be ordered by the caller (one stream,
// or events).
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace {

constexpr size_t kScratchBytes = PKV_DECODE_NOALLOC_MAX_WORKSPACE;
constexpr int kClearThreads = 256;  // 16 bytes each: 4 KiB per workgroup
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's scratch array, or nullptr.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

// Zeroes the leading counters (n_vec 16-byte vectors) with plain vector
// stores: a fill kernel rather than a memset node, so the call can be
// captured in a graph.
__global__ __launch_bounds__(kClearThreads) void clear_counters_kernel(uint4* head, size_t n_vec) {
  const size_t i = (size_t)blockIdx.x * kClearThreads + threadIdx.x;
  if (i < n_vec) head[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

size_t paged_attention_decode_noalloc_max_workspace(void) { return kScratchBytes; }

pkv_status_t paged_attention_decode_noalloc(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, int32_t q_dtype, int32_t cache_dtype, int32_t partition_size, void* stream) {
  const size_t need = paged_attention_decode_workspace_size(
      num_seqs, num_heads, num_kv_heads, head_size, block_size, max_context_len, q_dtype,
      cache_dtype, partition_size);
  // Invalid sizes or dtypes (need == 0) and empty batches: the plain entry
  // point reports them, or returns without a launch, and touches nothing.
  if (need == 0 || num_seqs == 0)
    return paged_attention_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                                  block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                  head_size, block_size, max_blocks_per_seq, max_context_len,
                                  scale, q_dtype, cache_dtype, partition_size, nullptr, 0,
                                  stream);
  if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  if (cache_dtype == PKV_FP8_E4M3 && (!key_scale || !value_scale)) return PKV_ERR_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  void* ws = scratch_ptr(dev);
  if (!ws) return PKV_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // a multiple of 256 bytes, within `need`
  const size_t zero = paged_attention_decode_workspace_counter_bytes(
      num_seqs, num_heads, num_kv_heads, head_size, block_size, max_context_len, q_dtype,
      cache_dtype, partition_size);
  const size_t n_vec = zero / 16;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((n_vec + kClearThreads - 1) / kClearThreads)),
                     dim3(kClearThreads), 0, s, reinterpret_cast<uint4*>(ws), n_vec);
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  return paged_attention_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                                block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                head_size, block_size, max_blocks_per_seq, max_context_len, scale,
                                q_dtype, cache_dtype, partition_size, ws, kScratchBytes, stream);
}

}  // extern "C"
