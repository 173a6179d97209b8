// Host-side declarations shared by the translation units of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// Block-table entries one work item of the decode kernel may span (so a
// partition holds at most this many blocks).
constexpr int kDecodeMaxTable = 256;

// Most partitions per context whose partials the decode kernel merges
// itself (one batch of loads per merge); longer splits use the reduce kernel.
constexpr int kFusedMaxPartitions = 4;

struct WriteArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  float* key_scale;
  float* value_scale;
  const int32_t* slots;
  int T, H_kv, D, bs, num_blocks;
  int src_dtype, cache_dtype;
  void* workspace;
  hipStream_t stream;
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* key_cache;
  const void* value_cache;
  const float* key_scale;
  const float* value_scale;
  const int32_t* tables;
  const int32_t* lens;
  int S, H, H_kv, D, bs, max_blocks, max_ctx;
  int M = 1;  // query tokens per sequence: 1 for decode, the chunk for prefill;
              // q and out are [S][M][H][D]
  // Attention split at a prefix shared by every table (zero otherwise):
  int len_off = 0;        // the launch sees positions from len_off on (tables offset to match)
  int prefix_rows = 0;    // > 0: one launch over the prefix, rows = (sequence, head) pairs
  int slot_off = 0;       // partial slot of the launch's partition 0
  int np_stride = 0;      // partial slots per row (0: NP)
  bool force_partial = false;  // partials even for contexts within one partition
  int prefix_slots = 0;   // reduce: slots before the suffix partitions
  float scale;
  int q_dtype, cache_dtype;
  int P;   // partition size in tokens (multiple of bs)
  int NP;  // partitions per sequence the grid covers: ceil(max_ctx / P)
  int* sched;     // work-queue counters (4 KiB header of the workspace), zero
                  // between calls
  float* ws_m;    // [S][H][NP]  running max (base-2 units) per partition
  float* ws_l;    // [S][H][NP]  running sum per partition
  float* ws_acc;  // [S][H][NP][D]  unnormalised output per partition: fp32 for
                  // fp32 queries, bf16 (in the first half of the region) for
                  // bf16 queries, whose output is bf16 anyway
  int* arrivals;  // [S][H_kv x row groups] partition arrivals (split partials
                  // merged by the partition kernel), zero between calls
  bool fused = false;  // the partition kernel merges the partials: no reduce launch
  // A write fused into a one-token decode (matrix-core kernel, bf16 cache):
  // sequence s's new rows new_k/new_v[s][H_kv][D] go to slot slots[s].
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  const int32_t* slots = nullptr;
  int num_slots = 0;  // slots of the pool (num_blocks x bs): others are not written
  hipStream_t stream;
};

struct BlockCopyArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const float* src_ks;
  const float* src_vs;
  float* dst_ks;
  float* dst_vs;
  const int32_t* pairs;  // [n][2] (source block, destination block)
  int n, H_kv, D, bs, cache_dtype;
  hipStream_t stream;
};

hipError_t launch_kv_block_copy(const BlockCopyArgs& a);
hipError_t launch_kv_write_copy(const WriteArgs& a);
hipError_t launch_kv_write_fp8(const WriteArgs& a);
size_t kv_write_fp8_workspace(int num_blocks, int H_kv);

hipError_t launch_decode_valu(const DecodeArgs& a);
bool decode_mfma_supported(const DecodeArgs& a);
hipError_t launch_decode_mfma(const DecodeArgs& a);
hipError_t launch_decode_reduce(const DecodeArgs& a);

// Tiled multi-token kernel (long prefill chunks, bf16 cache, or an FP8 cache
// staged to bf16 first): a workgroup owns prefill_tile_rows() rows of one KV
// head and stages one partition's block ids in LDS, at most kPrefillMaxTable
// of them.
constexpr int kPrefillMaxTable = 1024;
int prefill_tile_rows();
bool prefill_mfma_supported(const DecodeArgs& a);
hipError_t launch_prefill_mfma(const DecodeArgs& a);

// FP8 caches on the tiled kernel: the blocks the sequences reach, dequantised
// to bf16 into a pool of S * nb blocks (nb = ceil(max_ctx / bs)), pool block
// s * nb + j holding logical block j of sequence s, named by tables[s][j].
struct PrefillStage {
  void* key_pool;    // [S * nb][H_kv][bs][D] bf16
  void* value_pool;
  int32_t* tables;   // [S][nb]
  int nb;
};
hipError_t launch_prefill_stage_fp8(const DecodeArgs& a, const PrefillStage& st);

}  // namespace pkv
