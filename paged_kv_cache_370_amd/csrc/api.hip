// C ABI of libpagedkv: host-side argument checks, partition choice, workspace
// layout and kernel dispatch.  Nothing here touches device memory; every
// check happens before the first launch.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pkv_internal.h"

using namespace pkv;

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kDefaultPartition = 512;

bool valid_d(int D) { return D == 64 || D == 128; }
bool valid_bs(int bs) { return bs == 8 || bs == 16 || bs == 32; }

bool decode_pair_ok(int q, int c) {
  return (q == PKV_F32 && c == PKV_F32) || (q == PKV_BF16 && c == PKV_BF16) ||
         (q == PKV_BF16 && c == PKV_FP8_E4M3);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Partition size in tokens, or -1.  A context that fits one partition is
// finished by the partition kernel itself.  The decode kernel takes its
// items longest first; the choice below follows what was measured on
// MI355X (bf16 7B-class batch, FP8 batch, shared-prefix batch):
//   * few (sequence, KV head) items (`items` < kWholeMinItems): contexts are
//     split into partitions of kDefaultPartition tokens (twice that for FP8
//     caches, the same K/V bytes per item), so long sequences spread over
//     many workgroups;
//   * kWholeMinItems .. kHalfMaxItems items (under two per workgroup):
//     whole contexts up to one item's table (kDecodeMaxTable blocks), so no
//     partials are left to merge (shared-prefix batch: 90 -> 82 us);
//   * more items: partitions of half the longest context (at least the
//     default, at most one item's table): the workgroups sharing a CU are
//     served at up to 3x different rates, and items that large would keep
//     the slowest ones busy past the others (7B-class: 204 us at 512, 202
//     at 1024, 205-210 whole; FP8: 177 us at 1024, 165 at 4096).
constexpr long long kWholeMinItems = 1024;
constexpr long long kHalfMaxItems = 1536;

int resolve_partition(int bs, int max_ctx, int requested, int cache_dtype, long long items = 0) {
  if (requested < 0) return -1;
  if (requested > 0) return requested % bs == 0 ? requested : -1;
  const int def = cache_dtype == PKV_FP8_E4M3 ? 2 * kDefaultPartition : kDefaultPartition;
  const int whole = std::max(bs, ((max_ctx + bs - 1) / bs) * bs);
  if (max_ctx <= def) return whole;
  const int cap = kDecodeMaxTable * bs;
  if (items >= kHalfMaxItems) {
    const int half = ((max_ctx + 1) / 2 + bs - 1) / bs * bs;
    return std::min(cap, std::max(def, half));
  }
  if (items >= kWholeMinItems) return std::min(whole, cap);
  return def;
}

// (sequence, KV head, 16-row chunk) items of a call whose contexts are not split.
long long context_items(int S, int H, int H_kv, int M = 1) {
  if (H_kv <= 0 || H % H_kv != 0) return 0;
  return (long long)S * H_kv * (((long long)M * (H / H_kv) + 15) / 16);
}

int num_partitions(int max_ctx, int P) {
  const int np = (max_ctx + P - 1) / P;
  return np < 1 ? 1 : np;
}

pkv_status_t check_decode_shape(int S, int H, int H_kv, int D, int bs, int max_ctx, int q,
                                int c) {
  if (S < 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0) return PKV_ERR_SHAPE;
  if (!valid_d(D) || !valid_bs(bs) || max_ctx < 0) return PKV_ERR_SHAPE;
  if (!decode_pair_ok(q, c)) return PKV_ERR_DTYPE;
  return PKV_OK;
}

// Workspace: a 4 KiB header of work-queue counters (10 counters, 256 bytes
// apart), then, when a context can span more than one partition, the
// partition arrival counters of one-token decode (one per sequence and row
// group, at most S x H) and the split partials (m, l, acc).  The counters
// are zero between calls: each call returns them to zero.
constexpr size_t kSchedBytes = 4096;

// Row groups per sequence (H_kv x 16-row chunks) never exceed H.
size_t arrival_bytes(int S, int H, int M) {
  return M == 1 ? align256((size_t)S * H * sizeof(int)) : 0;
}

// rows of partials: S sequences x M query tokens x H heads x partitions
size_t decode_workspace(int S, int H, int D, int max_ctx, int P, int M = 1) {
  const int np = num_partitions(max_ctx, P);
  if (np <= 1) return kSchedBytes;
  const size_t rows = (size_t)S * M * H * np;
  return kSchedBytes + arrival_bytes(S, H, M) + 2 * align256(rows * sizeof(float)) +
         align256(rows * D * sizeof(float));
}

struct DecodeSetup {
  pkv_status_t status;
  bool empty;  // no sequences: nothing to launch, pointers not inspected
  DecodeArgs a;
};

DecodeSetup setup_decode(void* out, const void* query, const void* key_cache,
                         const void* value_cache, const float* key_scale,
                         const float* value_scale, const int32_t* block_tables,
                         const int32_t* context_lens, int S, int H, int H_kv, int D, int bs,
                         int max_blocks, int max_ctx, float scale, int q, int c, int partition,
                         void* workspace, size_t workspace_bytes, void* stream,
                         bool need_inputs, int M = 1) {
  DecodeSetup r{};
  r.status = check_decode_shape(S, H, H_kv, D, bs, max_ctx, q, c);
  if (r.status != PKV_OK) return r;
  if (need_inputs && (max_blocks <= 0 || (long long)max_blocks * bs < max_ctx)) {
    r.status = PKV_ERR_SHAPE;
    return r;
  }
  const int P = resolve_partition(bs, max_ctx, partition, c, context_items(S, H, H_kv, M));
  if (P <= 0) {
    r.status = PKV_ERR_SHAPE;
    return r;
  }
  // Work items (KV head x 16-row chunk x sequence x partition) and reduce
  // rows index with 32-bit integers.
  const long long chunks = ((long long)M * (H / H_kv) + 15) / 16;
  if ((long long)H_kv * chunks * S * num_partitions(max_ctx, P) >= (1LL << 30) ||
      (long long)S * M * H * D >= (1LL << 31)) {
    r.status = PKV_ERR_SHAPE;
    return r;
  }
  if (S == 0) {
    r.empty = true;
    return r;
  }
  if (!out || !context_lens) {
    r.status = PKV_ERR_NULL;
    return r;
  }
  if (need_inputs) {
    if (!query || !key_cache || !value_cache || !block_tables) {
      r.status = PKV_ERR_NULL;
      return r;
    }
    if (c == PKV_FP8_E4M3 && (!key_scale || !value_scale)) {
      r.status = PKV_ERR_NULL;
      return r;
    }
  }
  const size_t need = decode_workspace(S, H, D, max_ctx, P, M);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0) {
    r.status = PKV_ERR_WORKSPACE;
    return r;
  }
  DecodeArgs& a = r.a;
  a.out = out; a.q = query; a.key_cache = key_cache; a.value_cache = value_cache;
  a.key_scale = key_scale; a.value_scale = value_scale;
  a.tables = block_tables; a.lens = context_lens;
  a.S = S; a.H = H; a.H_kv = H_kv; a.D = D; a.bs = bs; a.max_blocks = max_blocks;
  a.max_ctx = max_ctx; a.scale = scale; a.q_dtype = q; a.cache_dtype = c;
  a.P = P; a.NP = num_partitions(max_ctx, P); a.M = M;
  {
    char* ws = reinterpret_cast<char*>(workspace);
    a.sched = reinterpret_cast<int*>(ws);
    if (a.NP > 1) {
      const size_t rows = (size_t)S * M * H * a.NP;
      if (M == 1) a.arrivals = reinterpret_cast<int*>(ws + kSchedBytes);
      char* part = ws + kSchedBytes + arrival_bytes(S, H, M);
      a.ws_m = reinterpret_cast<float*>(part);
      a.ws_l = reinterpret_cast<float*>(part + align256(rows * sizeof(float)));
      a.ws_acc = reinterpret_cast<float*>(part + 2 * align256(rows * sizeof(float)));
    }
  }
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return r;
}

pkv_status_t hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

extern "C" {

const char* pkv_status_string(int32_t s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "unsupported or inconsistent size";
    case PKV_ERR_DTYPE: return "unsupported dtype combination";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t pkv_version(void) { return kVersion; }

size_t paged_kv_cache_write_workspace_size(int32_t num_tokens, int32_t num_kv_heads,
                                           int32_t num_blocks, int32_t cache_dtype) {
  (void)num_tokens;
  if (cache_dtype != PKV_FP8_E4M3 || num_blocks <= 0 || num_kv_heads <= 0) return 0;
  return kv_write_fp8_workspace(num_blocks, num_kv_heads);
}

pkv_status_t paged_kv_cache_write(const void* key, const void* value, void* key_cache,
                                  void* value_cache, float* key_scale, float* value_scale,
                                  const int32_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                  int32_t num_blocks, int32_t src_dtype, int32_t cache_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!valid_d(head_size) || !valid_bs(block_size)) return PKV_ERR_SHAPE;
  const bool copy = (src_dtype == cache_dtype) && (src_dtype == PKV_F32 || src_dtype == PKV_BF16);
  const bool fp8 = cache_dtype == PKV_FP8_E4M3 && (src_dtype == PKV_BF16 || src_dtype == PKV_F32);
  if (!copy && !fp8) return PKV_ERR_DTYPE;
  // Nothing is read or written for an empty batch, so its (possibly NULL)
  // pointers are not inspected.
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_NULL;
  if (fp8 && (!key_scale || !value_scale)) return PKV_ERR_NULL;
  if (fp8) {
    const size_t need = kv_write_fp8_workspace(num_blocks, num_kv_heads);
    if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return PKV_ERR_WORKSPACE;
  }
  WriteArgs a;
  a.key = key; a.value = value; a.key_cache = key_cache; a.value_cache = value_cache;
  a.key_scale = key_scale; a.value_scale = value_scale; a.slots = slot_mapping;
  a.T = num_tokens; a.H_kv = num_kv_heads; a.D = head_size; a.bs = block_size;
  a.num_blocks = num_blocks; a.src_dtype = src_dtype; a.cache_dtype = cache_dtype;
  a.workspace = workspace; a.stream = reinterpret_cast<hipStream_t>(stream);
  return hip_status(copy ? launch_kv_write_copy(a) : launch_kv_write_fp8(a));
}

pkv_status_t paged_kv_block_copy(const void* src_key_cache, const void* src_value_cache,
                                 const float* src_key_scale, const float* src_value_scale,
                                 void* dst_key_cache, void* dst_value_cache, float* dst_key_scale,
                                 float* dst_value_scale, const int32_t* block_pairs,
                                 int32_t num_pairs, int32_t num_kv_heads, int32_t head_size,
                                 int32_t block_size, int32_t cache_dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0) return PKV_ERR_SHAPE;
  if (!valid_d(head_size) || !valid_bs(block_size)) return PKV_ERR_SHAPE;
  if (cache_dtype != PKV_F32 && cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3)
    return PKV_ERR_DTYPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_pairs)
    return PKV_ERR_NULL;
  if (cache_dtype == PKV_FP8_E4M3 &&
      (!src_key_scale || !src_value_scale || !dst_key_scale || !dst_value_scale))
    return PKV_ERR_NULL;
  BlockCopyArgs a;
  a.src_k = src_key_cache; a.src_v = src_value_cache;
  a.dst_k = dst_key_cache; a.dst_v = dst_value_cache;
  a.src_ks = src_key_scale; a.src_vs = src_value_scale;
  a.dst_ks = dst_key_scale; a.dst_vs = dst_value_scale;
  a.pairs = block_pairs; a.n = num_pairs; a.H_kv = num_kv_heads; a.D = head_size;
  a.bs = block_size; a.cache_dtype = cache_dtype;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return hip_status(launch_kv_block_copy(a));
}

size_t paged_attention_decode_workspace_counter_bytes(int32_t num_seqs, int32_t num_heads,
                                                     int32_t num_kv_heads, int32_t head_size,
                                                     int32_t block_size, int32_t max_context_len,
                                                     int32_t q_dtype, int32_t cache_dtype,
                                                     int32_t partition_size) {
  if (check_decode_shape(num_seqs, num_heads, num_kv_heads, head_size, block_size,
                         max_context_len, q_dtype, cache_dtype) != PKV_OK)
    return 0;
  const int P = resolve_partition(block_size, max_context_len, partition_size, cache_dtype,
                                  context_items(num_seqs, num_heads, num_kv_heads));
  if (P <= 0) return 0;
  if (num_partitions(max_context_len, P) <= 1) return kSchedBytes;
  return kSchedBytes + arrival_bytes(num_seqs, num_heads, 1);
}

int32_t paged_attention_decode_partition_size(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_size,
                                              int32_t block_size, int32_t max_context_len,
                                              int32_t q_dtype, int32_t cache_dtype,
                                              int32_t partition_size) {
  if (check_decode_shape(num_seqs, num_heads, num_kv_heads, head_size, block_size,
                         max_context_len, q_dtype, cache_dtype) != PKV_OK)
    return -1;
  return resolve_partition(block_size, max_context_len, partition_size, cache_dtype,
                           context_items(num_seqs, num_heads, num_kv_heads));
}

size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                             int32_t num_kv_heads, int32_t head_size,
                                             int32_t block_size, int32_t max_context_len,
                                             int32_t q_dtype, int32_t cache_dtype,
                                             int32_t partition_size) {
  const int P = paged_attention_decode_partition_size(num_seqs, num_heads, num_kv_heads,
                                                      head_size, block_size, max_context_len,
                                                      q_dtype, cache_dtype, partition_size);
  if (P <= 0) return 0;
  return decode_workspace(num_seqs, num_heads, head_size, max_context_len, P);
}

pkv_status_t paged_attention_decode_partitions(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, int32_t q_dtype, int32_t cache_dtype, int32_t partition_size, void* workspace,
    size_t workspace_bytes, void* stream) {
  DecodeSetup s = setup_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                               block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                               head_size, block_size, max_blocks_per_seq, max_context_len, scale,
                               q_dtype, cache_dtype, partition_size, workspace, workspace_bytes,
                               stream, true);
  if (s.status != PKV_OK || s.empty) return s.status;
  return hip_status(decode_mfma_supported(s.a) ? launch_decode_mfma(s.a)
                                               : launch_decode_valu(s.a));
}

pkv_status_t paged_attention_decode_reduce(void* out, const int32_t* context_lens,
                                           int32_t num_seqs, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_size,
                                           int32_t block_size, int32_t max_context_len,
                                           int32_t q_dtype, int32_t cache_dtype,
                                           int32_t partition_size, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  DecodeSetup s = setup_decode(out, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                               block_size, 0, max_context_len, 1.0f, q_dtype, cache_dtype,
                               partition_size, workspace, workspace_bytes, stream, false);
  if (s.status != PKV_OK || s.empty || s.a.NP <= 1) return s.status;
  return hip_status(launch_decode_reduce(s.a));
}

pkv_status_t paged_attention_decode(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const float* key_scale,
                                    const float* value_scale, const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t max_context_len, float scale, int32_t q_dtype,
                                    int32_t cache_dtype, int32_t partition_size,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  DecodeSetup s = setup_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                               block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                               head_size, block_size, max_blocks_per_seq, max_context_len, scale,
                               q_dtype, cache_dtype, partition_size, workspace, workspace_bytes,
                               stream, true);
  if (s.status != PKV_OK || s.empty) return s.status;
  // Up to kFusedMaxPartitions partitions per context, the matrix-core
  // kernel merges the partials itself (the last partition of a row group
  // to arrive merges them): one launch.
  if (decode_mfma_supported(s.a) && s.a.NP > 1 && s.a.NP <= kFusedMaxPartitions &&
      s.a.arrivals) {
    s.a.fused = true;
    return hip_status(launch_decode_mfma(s.a));
  }
  pkv_status_t st = hip_status(decode_mfma_supported(s.a) ? launch_decode_mfma(s.a)
                                                          : launch_decode_valu(s.a));
  if (st != PKV_OK || s.a.NP <= 1) return st;
  return hip_status(launch_decode_reduce(s.a));
}

pkv_status_t paged_attention_decode_write(
    void* out, const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, const int32_t* slot_mapping, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale, int32_t q_dtype, int32_t cache_dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_blocks <= 0) return PKV_ERR_SHAPE;
  if (cache_dtype != PKV_BF16 && cache_dtype != PKV_F32) return PKV_ERR_DTYPE;  // copy writes
  DecodeSetup s = setup_decode(out, query, key_cache, value_cache, nullptr, nullptr,
                               block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                               head_size, block_size, max_blocks_per_seq, max_context_len, scale,
                               q_dtype, cache_dtype, partition_size, workspace, workspace_bytes,
                               stream, true);
  if (s.status != PKV_OK || s.empty) return s.status;
  if (!key || !value || !slot_mapping) return PKV_ERR_NULL;
  WriteArgs w;
  w.key = key; w.value = value; w.key_cache = key_cache; w.value_cache = value_cache;
  w.key_scale = nullptr; w.value_scale = nullptr; w.slots = slot_mapping;
  w.T = num_seqs; w.H_kv = num_kv_heads; w.D = head_size; w.bs = block_size;
  w.num_blocks = num_blocks; w.src_dtype = cache_dtype; w.cache_dtype = cache_dtype;
  w.workspace = nullptr; w.stream = s.a.stream;
  if (!decode_mfma_supported(s.a)) {
    // fp32 queries (vector-ALU kernel), or partitions past the matrix-core
    // kernel's table slice: the write, then the decode
    pkv_status_t st = hip_status(launch_kv_write_copy(w));
    if (st == PKV_OK) st = hip_status(launch_decode_valu(s.a));
    if (st != PKV_OK || s.a.NP <= 1) return st;
    return hip_status(launch_decode_reduce(s.a));
  }
  s.a.new_k = key;
  s.a.new_v = value;
  s.a.slots = slot_mapping;
  const long long pool = (long long)num_blocks * block_size;
  s.a.num_slots = pool > 0x7fffffffLL ? 0x7fffffff : (int)pool;
  if (s.a.NP > 1 && s.a.NP <= kFusedMaxPartitions && s.a.arrivals) {
    s.a.fused = true;
    return hip_status(launch_decode_mfma(s.a));
  }
  pkv_status_t st = hip_status(launch_decode_mfma(s.a));
  if (st != PKV_OK || s.a.NP <= 1) return st;
  return hip_status(launch_decode_reduce(s.a));
}

// Shared-prefix decode: the prefix's partials (ceil(prefix / P) slots) come
// before the suffix partitions' in every row; the prefix is cut into
// partitions of the same P tokens.  (Cutting it finer for more parallel
// items was measured slower.)
struct PrefixSplit {
  int P = -1, pre_slots = 0, suf_slots = 0;
};

static PrefixSplit prefix_split(int bs, int max_ctx, int prefix, int requested,
                                int cache_dtype) {
  PrefixSplit sp;
  if (prefix <= 0 || prefix % bs != 0 || prefix > max_ctx) return sp;
  sp.P = resolve_partition(bs, max_ctx - prefix > 0 ? max_ctx - prefix : bs, requested,
                           cache_dtype);
  if (sp.P <= 0) return sp;
  sp.pre_slots = (prefix + sp.P - 1) / sp.P;
  sp.suf_slots = num_partitions(max_ctx - prefix, sp.P);
  return sp;
}

static size_t shared_prefix_workspace(int S, int H, int D, const PrefixSplit& sp) {
  const size_t rows = (size_t)S * H * (sp.pre_slots + sp.suf_slots);
  return kSchedBytes + 2 * align256(rows * sizeof(float)) + align256(rows * D * sizeof(float));
}

// Which kernel serves a multi-token call, and its partition size.  Long
// chunks (at least kTileMinRows (token, head) rows per KV head) run on the
// tiled prefill kernel (an FP8 cache staged to bf16 first); short ones on
// the decode kernel's multi-token mode, whose 16-row tiles suit the
// HBM-bound case.  The tiled kernel's own partition choice keeps whole contexts in one
// partition unless the grid would leave CUs idle (two workgroups per CU on
// 256 CUs), in partitions of at least 512 keys.
constexpr int kTileMinRows = 64;
constexpr long long kTileFillWorkgroups = 512;

struct PrefillPlan {
  bool tiled;
  int P;  // partition size, or <= 0 for invalid arguments
};

static PrefillPlan prefill_plan(int S, int M, int H, int H_kv, int D, int bs, int max_ctx, int q,
                         int c, int requested) {
  PrefillPlan pl{false, -1};
  if (M <= 0 || check_decode_shape(S, H, H_kv, D, bs, max_ctx, q, c) != PKV_OK ||
      q != PKV_BF16)
    return pl;
  const long long rows = (long long)M * (H / H_kv);
  pl.tiled = rows >= kTileMinRows;
  if (!pl.tiled) {
    // Several tokens per sequence on the decode kernel: an item's partial
    // output is M * G rows wide, so with enough items to give every CU two
    // (S x KV heads x 16-row chunks >= 512) a context is not split at all
    // when its blocks fit one item: no partials and no merge (beams over
    // forked tables, 64 beams x 4 tokens over 2069 positions: 78 -> 50 us).
    const long long items = (long long)S * H_kv * ((rows + 15) / 16);
    const int whole = ((max_ctx + bs - 1) / bs) * bs;
    if (requested == 0 && items >= 512 && whole <= kDecodeMaxTable * bs) {
      pl.P = whole < bs ? bs : whole;
      return pl;
    }
    pl.P = resolve_partition(bs, max_ctx, requested, c);
    return pl;
  }
  if (requested != 0) {
    pl.P = requested > 0 && requested % bs == 0 && requested / bs + 1 <= kPrefillMaxTable
               ? requested
               : -1;
    return pl;
  }
  const int tile = prefill_tile_rows();
  const long long tiles = (long long)S * H_kv * ((rows + tile - 1) / tile);
  const int cap = (kPrefillMaxTable - 1) * bs / 64 * 64;  // keys one table slice holds
  long long np = (max_ctx + cap - 1) / cap;
  const long long fill = tiles > 0 ? (kTileFillWorkgroups + tiles - 1) / tiles : 1;
  const long long by_len = max_ctx / 512 > 1 ? max_ctx / 512 : 1;
  np = std::max(np, std::min(fill, by_len));
  if (np < 1) np = 1;
  const long long per = (max_ctx + np - 1) / np;
  pl.P = (int)std::max<long long>(64, (per + 63) / 64 * 64);
  return pl;
}

// The FP8 stage after the tiled kernel's workspace: the pool's table
// ([S][nb] int32), then the bf16 K and V pools of S * nb blocks each.  Pool
// block ids are 32-bit.
struct StageLayout {
  int nb = 0;
  size_t tab = 0, pool = 0;  // bytes of the table and of one pool
  size_t bytes() const { return tab + 2 * pool; }
};

static StageLayout stage_layout(int S, int H_kv, int D, int bs, int max_ctx) {
  StageLayout l;
  l.nb = (max_ctx + bs - 1) / bs;
  if ((long long)S * l.nb >= (1LL << 31)) {
    l.nb = -1;
    return l;
  }
  l.tab = align256((size_t)S * l.nb * sizeof(int32_t));
  l.pool = align256((size_t)S * l.nb * H_kv * bs * D * 2);
  return l;
}

pkv_status_t paged_attention_prefill(void* out, const void* query, const void* key_cache,
                                     const void* value_cache, const float* key_scale,
                                     const float* value_scale, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_query_tokens, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t q_dtype, int32_t cache_dtype,
                                     int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (num_query_tokens <= 0) return PKV_ERR_SHAPE;
  const pkv_status_t shape = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_size,
                                                block_size, max_context_len, q_dtype, cache_dtype);
  if (shape != PKV_OK) return shape;
  if (q_dtype != PKV_BF16) return PKV_ERR_DTYPE;  // the matrix-core kernels take bf16 queries
  const PrefillPlan plan = prefill_plan(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                        head_size, block_size, max_context_len, q_dtype,
                                        cache_dtype, partition_size);
  if (plan.P <= 0) return PKV_ERR_SHAPE;
  DecodeSetup s = setup_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                               block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                               head_size, block_size, max_blocks_per_seq, max_context_len, scale,
                               q_dtype, cache_dtype, plan.P, workspace, workspace_bytes, stream,
                               true, num_query_tokens);
  if (s.status != PKV_OK || s.empty) return s.status;
  pkv_status_t st;
  if (plan.tiled && cache_dtype == PKV_FP8_E4M3) {
    const StageLayout sl =
        stage_layout(num_seqs, num_kv_heads, head_size, block_size, max_context_len);
    if (sl.nb < 0) return PKV_ERR_SHAPE;
    const size_t base = decode_workspace(num_seqs, num_heads, head_size, max_context_len,
                                         plan.P, num_query_tokens);
    if (workspace_bytes < base + sl.bytes()) return PKV_ERR_WORKSPACE;
    char* ws = reinterpret_cast<char*>(workspace) + base;
    PrefillStage stage{ws + sl.tab, ws + sl.tab + sl.pool, reinterpret_cast<int32_t*>(ws),
                       sl.nb};
    DecodeArgs t = s.a;  // the tiled kernel's view: the bf16 pool and its table
    t.key_cache = stage.key_pool;
    t.value_cache = stage.value_pool;
    t.key_scale = t.value_scale = nullptr;
    t.tables = stage.tables;
    t.max_blocks = sl.nb;
    t.cache_dtype = PKV_BF16;
    if (!prefill_mfma_supported(t)) return PKV_ERR_SHAPE;
    st = hip_status(launch_prefill_stage_fp8(s.a, stage));
    if (st == PKV_OK) st = hip_status(launch_prefill_mfma(t));
  } else if (plan.tiled) {
    if (!prefill_mfma_supported(s.a)) return PKV_ERR_SHAPE;
    st = hip_status(launch_prefill_mfma(s.a));
  } else {
    if (!decode_mfma_supported(s.a)) return PKV_ERR_SHAPE;
    st = hip_status(launch_decode_mfma(s.a));
  }
  if (st != PKV_OK || s.a.NP <= 1) return st;
  return hip_status(launch_decode_reduce(s.a));
}

pkv_status_t paged_attention_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale, const int32_t* block_tables,
    const int32_t* context_lens, int32_t prefix_tokens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale, int32_t q_dtype, int32_t cache_dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (prefix_tokens == 0)
    return paged_attention_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                                  block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                  head_size, block_size, max_blocks_per_seq, max_context_len,
                                  scale, q_dtype, cache_dtype, partition_size, workspace,
                                  workspace_bytes, stream);
  const pkv_status_t shape = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_size,
                                                block_size, max_context_len, q_dtype, cache_dtype);
  if (shape != PKV_OK) return shape;
  if (q_dtype != PKV_BF16) return PKV_ERR_DTYPE;  // rows of many sequences: matrix cores
  const PrefixSplit sp =
      prefix_split(block_size, max_context_len, prefix_tokens, partition_size, cache_dtype);
  if (sp.P <= 0) return PKV_ERR_SHAPE;
  DecodeSetup s = setup_decode(out, query, key_cache, value_cache, key_scale, value_scale,
                               block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                               head_size, block_size, max_blocks_per_seq, max_context_len, scale,
                               q_dtype, cache_dtype, sp.P, workspace, SIZE_MAX, stream, true);
  if (s.status != PKV_OK || s.empty) return s.status;
  // The split's own workspace layout (setup_decode's size is a plain decode's).
  const size_t need = shared_prefix_workspace(num_seqs, num_heads, head_size, sp);
  if (workspace_bytes < need) return PKV_ERR_WORKSPACE;
  // Partials for every (sequence, head) row: pre_slots + suf_slots each.
  DecodeArgs base = s.a;
  {
    const size_t rows = (size_t)num_seqs * num_heads * (sp.pre_slots + sp.suf_slots);
    char* part = reinterpret_cast<char*>(workspace) + kSchedBytes;
    base.ws_m = reinterpret_cast<float*>(part);
    base.ws_l = reinterpret_cast<float*>(part + align256(rows * sizeof(float)));
    base.ws_acc = reinterpret_cast<float*>(part + 2 * align256(rows * sizeof(float)));
  }
  base.np_stride = sp.pre_slots + sp.suf_slots;
  base.force_partial = true;
  // 1. One launch: the prefix once per KV head for all sequences (items
  //    whose rows are the (sequence, head) pairs, keys the prefix blocks of
  //    the first table), then each sequence's positions after the prefix,
  //    as a decode of its own.
  DecodeArgs one = base;
  one.prefix_rows = prefix_tokens;
  one.prefix_slots = sp.pre_slots;
  one.len_off = prefix_tokens;  // the suffix items skip the prefix's table entries
  one.max_ctx = max_context_len - prefix_tokens;
  one.NP = sp.suf_slots;
  one.slot_off = sp.pre_slots;
  if (!decode_mfma_supported(one)) return PKV_ERR_SHAPE;
  pkv_status_t st = hip_status(launch_decode_mfma(one));
  if (st != PKV_OK) return st;
  // 2. Merge the prefix and suffix partials of every row.
  DecodeArgs red = base;
  red.NP = sp.pre_slots + sp.suf_slots;
  red.prefix_slots = sp.pre_slots;
  red.len_off = prefix_tokens;
  return hip_status(launch_decode_reduce(red));
}

size_t paged_attention_decode_shared_prefix_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, int32_t prefix_tokens, int32_t q_dtype,
    int32_t cache_dtype, int32_t partition_size) {
  if (prefix_tokens == 0)
    return paged_attention_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size,
                                                 block_size, max_context_len, q_dtype,
                                                 cache_dtype, partition_size);
  if (check_decode_shape(num_seqs, num_heads, num_kv_heads, head_size, block_size,
                         max_context_len, q_dtype, cache_dtype) != PKV_OK ||
      q_dtype != PKV_BF16)
    return 0;
  const PrefixSplit sp =
      prefix_split(block_size, max_context_len, prefix_tokens, partition_size, cache_dtype);
  if (sp.P <= 0) return 0;
  return shared_prefix_workspace(num_seqs, num_heads, head_size, sp);
}

size_t paged_attention_prefill_workspace_size(int32_t num_seqs, int32_t num_query_tokens,
                                              int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_size, int32_t block_size,
                                              int32_t max_context_len, int32_t q_dtype,
                                              int32_t cache_dtype, int32_t partition_size) {
  const PrefillPlan plan = prefill_plan(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                        head_size, block_size, max_context_len, q_dtype,
                                        cache_dtype, partition_size);
  if (plan.P <= 0) return 0;
  const size_t base =
      decode_workspace(num_seqs, num_heads, head_size, max_context_len, plan.P, num_query_tokens);
  if (!plan.tiled || cache_dtype != PKV_FP8_E4M3) return base;
  const StageLayout sl = stage_layout(num_seqs, num_kv_heads, head_size, block_size,
                                      max_context_len);
  return sl.nb < 0 ? 0 : base + sl.bytes();
}

}  // extern "C"
