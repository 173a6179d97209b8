/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged KV-cache write and PagedAttention
 * decode for AMD Instinct MI355X (gfx950).
 *
 * The method: the KV cache lives in a pool of fixed-size physical blocks
 * (default 16 tokens each), allocated once; every sequence reaches its
 * blocks through a block table that maps logical block j to a physical block,
 * so a sequence's storage need not be contiguous and blocks can be shared
 * between sequences (dpshk.com PagedAttention article "企业官网建设流程全解析",
 * sections 2.1 Block / BlockTable, 2.3 sharing by reference count, 3.2 block
 * pre-allocation and FP8 storage; page "vLLM的诞生背景：大模型推理的痛点与
 * PagedAttention的破局", section "PagedAttention的破局思路"; page
 * "PagedAttention 与连续批处理：LLM Serving 的底层架构拆解", section
 * "PagedAttention：把显存做成虚拟内存").  Decode attention is
 * softmax(q K^T * scale) V over the whole context (dpshk.com article,
 * section 2.2), computed one block at a time with a running max and sum.
 *
 * Conventions for every call
 *   - All array pointers are DEVICE pointers (hipMalloc / torch CUDA tensors),
 *     row-major and densely packed in the layouts given below.
 *   - The caller owns and allocates every buffer, including the pool and the
 *     workspace; the library allocates and frees nothing and keeps no state
 *     between calls other than what a workspace holds.  Arrays are 16-byte
 *     aligned (hipMalloc returns 256): rows of the caches, queries and new
 *     K/V are read and written 16 bytes at a time, and so are parts of the
 *     workspaces (a workspace that is not is PKV_ERR_WORKSPACE).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  Buffers must stay alive
 *     until the stream has passed the call.  Calls are thread-safe.
 *   - All argument checks happen on the host before anything is enqueued; a
 *     failing check returns a status and touches no memory.  A failed launch
 *     returns PKV_ERR_HIP.  Nothing is thrown across the ABI.
 *   - Block ids in block tables and slots in slot mappings must lie inside the
 *     pool; context_lens[i] must not exceed max_blocks_per_seq * block_size.
 *     These are the caller's contract and are not checked on the device.
 *
 * Layouts (S sequences, H query heads, H_kv KV heads, D head size,
 * bs block size, T new tokens):
 *   query, out              [S][H][D]
 *   key_cache, value_cache  [num_blocks][H_kv][bs][D]   token rows of D
 *                           elements per (block, KV head) tile
 *   key_scale, value_scale  [num_blocks][H_kv] float32 (FP8 caches only)
 *   block_tables            int32 [S][max_blocks_per_seq]
 *   context_lens            int32 [S]   tokens in the cache, the current
 *                           step's token included (it must be written first)
 *   key, value (new rows)   [T][H_kv][D]
 *   slot_mapping            int32 [T]   slot = physical_block * bs + offset;
 *                           a negative slot skips the token
 *
 * Supported: D in {64, 128}; bs in {8, 16, 32}; H a multiple of H_kv.
 * Query head h reads KV head h / (H / H_kv).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_F32 = 0,       /* IEEE binary32 */
  PKV_BF16 = 1,      /* bfloat16 */
  PKV_FP8_E4M3 = 2   /* OCP FP8 E4M3FN codes (cache only) */
} pkv_dtype_t;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,       /* a required pointer is NULL */
  PKV_ERR_SHAPE = 2,      /* unsupported or inconsistent size */
  PKV_ERR_DTYPE = 3,      /* unsupported dtype or dtype combination */
  PKV_ERR_WORKSPACE = 4,  /* workspace missing or too small */
  PKV_ERR_HIP = 5         /* a HIP launch failed */
} pkv_status_t;

/*
 * paged_kv_cache_write -- scatter each new token's K and V rows into its
 * paged slot.  For token t with slot s = slot_mapping[t] >= 0, block
 * b = s / bs and offset o = s % bs, and every KV head h:
 *   key_cache[b][h][o][:] = key[t][h][:],  value_cache likewise.
 * (Block/BlockTable structure: dpshk.com article, section 2.1; the slot
 * mapping is the write side of the block table.)
 *
 *   src_dtype == cache_dtype in {PKV_F32, PKV_BF16}: the bits are copied
 *     unchanged; key_scale, value_scale and workspace are ignored (may be
 *     NULL).
 *   cache_dtype == PKV_FP8_E4M3, src_dtype in {PKV_BF16, PKV_F32}: FP8
 *     storage of blocks (dpshk.com article, section 3.2).  One float32 scale
 *     per (block, KV head), separately for K and V.  If this call writes
 *     offset 0 of block b, the scales of b are set from the largest magnitude
 *     among the tokens this call writes into b:
 *       scale = max(amax / 448, FLT_MIN)          (float32 arithmetic)
 *     otherwise the stored scales of b are kept.  Each element is stored as
 *     the E4M3FN code of the float32 quotient x / scale, rounded to nearest
 *     even, saturated to +-448 (NaN -> 0x7F).  A block's first write must
 *     include its offset 0.  Requires workspace of at least
 *     paged_kv_cache_write_workspace_size(...) bytes, zero before the first
 *     call that uses it (allocate it zero-filled); every call leaves it zero
 *     again, and calls that may run at the same time must not share it.
 *
 * Slots within one call must be distinct; duplicate slots race.
 * num_tokens == 0 returns PKV_OK after the size and dtype checks without
 * inspecting any pointer.
 */
pkv_status_t paged_kv_cache_write(
    const void* key, const void* value,
    void* key_cache, void* value_cache,
    float* key_scale, float* value_scale,
    const int32_t* slot_mapping,
    int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t num_blocks,
    int32_t src_dtype, int32_t cache_dtype,
    void* workspace, size_t workspace_bytes,
    void* stream);

/* Workspace bytes paged_kv_cache_write needs (0 unless the cache is FP8). */
size_t paged_kv_cache_write_workspace_size(
    int32_t num_tokens, int32_t num_kv_heads, int32_t num_blocks,
    int32_t cache_dtype);

/*
 * paged_attention_decode -- one query token per sequence attends over its
 * paged context (dpshk.com article, section 2.2: softmax(QK^T/sqrt(d))V,
 * evaluated over the whole context; page "PagedAttention 与连续批处理…",
 * section "PagedAttention：把显存做成虚拟内存": each page is found through
 * the page table).  For sequence i with n = context_lens[i] and head h:
 *   out[i][h][:] = sum_t softmax_t(scale * q[i][h] . K[t]) V[t],
 * t = 0..n-1, where token t of sequence i is row t % bs of physical block
 * block_tables[i][t / bs], KV head h / (H / H_kv).  n = 0 gives zeros.
 * Accumulation is float32; out has the query dtype (bf16 rounded to
 * nearest even).
 *
 *   q_dtype/cache_dtype pairs: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 *   FP8 caches are dequantised as code_value * key_scale[b][h] (value_scale
 *   likewise); scales are ignored otherwise (may be NULL).
 *   max_context_len must be >= every context_lens[i]; it sizes the grid so
 *   the host never reads device memory.
 *   partition_size (tokens, multiple of bs, or 0 = library choice, which
 *   paged_attention_decode_partition_size reports; it depends on the batch
 *   shape and the longest context, never on the lengths themselves):
 *   contexts longer than one partition are split, each partition is
 *   attended on its own, and the partial results are merged (each
 *   partition's running maximum and sum in float32, its unnormalised output
 *   in float32 for F32 queries and in bf16 for BF16 queries, whose output is
 *   bf16).  With BF16 queries and at most 4 partitions per context the
 *   decode kernel merges them itself (the last partition of a sequence's
 *   head group to finish does it); otherwise a second kernel merges them.
 *   workspace: at least paged_attention_decode_workspace_size(...) bytes
 *   (always >= 4096).  Its first paged_attention_decode_workspace_counter_bytes(...)
 *   bytes are counters (the 4096-byte work-queue header, then, when a
 *   context can span two partitions, num_seqs * num_heads int32 partition
 *   arrival counters rounded up to 256 bytes): they must be zero before
 *   the first call that uses the workspace (allocate it zero-filled) and
 *   every call leaves them zero again; the rest may hold anything.  Calls
 *   that may run at the same time must not share a workspace.
 *   num_seqs == 0 returns PKV_OK after the size and dtype checks without
 *   inspecting any pointer.
 */
pkv_status_t paged_attention_decode(
    void* out, const void* query,
    const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, int32_t q_dtype, int32_t cache_dtype,
    int32_t partition_size,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * paged_attention_decode_write -- a decode step's write and attention in one
 * call: exactly paged_kv_cache_write(key, value, key_cache, value_cache,
 * NULL, NULL, slot_mapping, num_tokens = num_seqs, num_kv_heads, head_size,
 * block_size, num_blocks, src_dtype = cache_dtype, cache_dtype) followed by
 * paged_attention_decode(...) with the other arguments (the write of the
 * step's new tokens, then attention over contexts that end with them: the
 * same two operations the dpshk.com article, sections 2.1-2.2, chains every
 * decode step).  With bf16 queries and cache on the matrix-core kernel both
 * run in the decode's launch: the item that holds a sequence's newest
 * position copies its new rows to their slot, and every item over that
 * position takes its K and V rows from key / value, which are the values
 * the write stores (a copy), so the result is bit for bit that of the two
 * calls.  Other dtype pairs run the two launches.
 *   key, value: [num_seqs][num_kv_heads][head_size], the cache's dtype;
 *   slot_mapping[i]: the slot of sequence i's position context_lens[i] - 1
 *   (block_tables[i][(n-1) / bs] * bs + (n-1) % bs), or outside
 *   [0, num_blocks * bs) for no write (that position is then read from the
 *   cache).  Slots must be distinct and the written block must not be read
 *   by another sequence of the call (copy-on-write before appending to a
 *   shared block); a slot that breaks this gives an unspecified result.
 *   Caches: PKV_BF16 or PKV_F32 (PKV_ERR_DTYPE for FP8: use the two calls).
 *   num_blocks: blocks in the pool.  Other arguments, the workspace
 *   (paged_attention_decode_workspace_size bytes) and errors are as for
 *   paged_attention_decode; num_seqs == 0 returns PKV_OK without inspecting
 *   any pointer.
 */
pkv_status_t paged_attention_decode_write(
    void* out, const void* query,
    const void* key, const void* value,
    void* key_cache, void* value_cache,
    const int32_t* slot_mapping,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, int32_t q_dtype, int32_t cache_dtype,
    int32_t partition_size,
    void* workspace, size_t workspace_bytes,
    void* stream);

/* The partition size paged_attention_decode uses for these arguments
 * (resolves partition_size == 0 to the library's choice); negative on
 * invalid arguments. */
int32_t paged_attention_decode_partition_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_context_len,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size);

/* Workspace bytes paged_attention_decode needs for these arguments. */
size_t paged_attention_decode_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_context_len,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size);

/* Leading workspace bytes of paged_attention_decode that hold counters and
 * must be zero at the call (0 on invalid arguments). */
size_t paged_attention_decode_workspace_counter_bytes(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_context_len,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size);

/*
 * The two phases of paged_attention_decode, for callers that schedule or
 * time them apart.  Same arguments and the same partition choice.
 * _partitions attends every (sequence, KV head, partition); sequences that
 * fit in one partition get their final output here.  _reduce then merges the
 * partitions of the longer sequences (a no-op launch-free return when no
 * sequence can span two partitions).  Calling _partitions then _reduce on
 * one stream equals one paged_attention_decode call.
 */
pkv_status_t paged_attention_decode_partitions(
    void* out, const void* query,
    const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, int32_t q_dtype, int32_t cache_dtype,
    int32_t partition_size,
    void* workspace, size_t workspace_bytes,
    void* stream);

pkv_status_t paged_attention_decode_reduce(
    void* out, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_context_len,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * paged_attention_prefill -- attention of several new query tokens per
 * sequence over the paged cache, causal: the prefill (or one chunk of a
 * chunked prefill) on the same block tables as decode.  Sequence i holds
 * context_lens[i] = n tokens in the cache, its num_query_tokens = M newest
 * included (written first); query token t sits at position n - M + t and
 *   out[i][t][h][:] = softmax(q[i][t][h] . K[0 .. n-M+t][h/G]^T * scale)
 *                     . V[0 .. n-M+t][h/G]
 * (the decode formula of dpshk.com article section 2.2 applied to each
 * token over the positions before it; page "PagedAttention 与连续批处理…",
 * section "连续批处理：让 GPU 永远有活干": new requests join the running
 * batch, so their prompts are processed against the same paged cache).
 *   query, out: [S][M][H][D], bf16 only (PKV_ERR_DTYPE otherwise); the
 *   caches may be bf16 or FP8.  n >= M for every sequence (the caller's
 *   contract; a token left with no position to see gets zeros).  M = 1 is
 *   decode.  Indices are 32-bit: num_kv_heads * ceil(M * G / 16) * S *
 *   ceil(max_context_len / P) must stay below 2^30 and S * M * H * D below
 *   2^31 (PKV_ERR_SHAPE otherwise).  Other arguments, partitions and the
 *   workspace (paged_attention_prefill_workspace_size bytes, its first 4096
 *   zero) are as for paged_attention_decode, except the library's choice
 *   (partition_size 0): long chunks (M * G >= 64) split a context only
 *   when the grid would leave CUs idle; other calls keep whole contexts (up
 *   to 256 blocks) when there are at least 512 (sequence, KV head, 16-row)
 *   items, and otherwise split them as decode does.
 *   Long chunks over an FP8 cache: the blocks the sequences reach are first
 *   dequantised (code * scale, float32, rounded to bf16) into a bf16 pool
 *   inside the workspace, which therefore also holds, after the partials,
 *   a table of S * ceil(max_context_len / block_size) int32 entries and two
 *   pools of that many blocks (K and V, [H_kv][bs][D] bf16 each); S *
 *   ceil(max_context_len / block_size) must stay below 2^31.  The workspace
 *   size function includes them.
 */
pkv_status_t paged_attention_prefill(
    void* out, const void* query,
    const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size,
    void* workspace, size_t workspace_bytes,
    void* stream);

/* Workspace bytes paged_attention_prefill needs (0 for invalid arguments). */
size_t paged_attention_prefill_workspace_size(
    int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_context_len,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size);

/*
 * paged_attention_decode_shared_prefix -- paged_attention_decode for a batch
 * whose tables all begin with the same physical blocks: a prompt prefix
 * shared by reference (dpshk.com article, section 2.3: blocks shared between
 * sequences with a reference count; page "PagedAttention 与连续批处理…",
 * section "PagedAttention：把显存做成虚拟内存": common prompt prefixes
 * shared, only page-aligned ones per its advice section).  The prefix is
 * read once per KV head for all sequences (rows = every sequence's query
 * heads of that KV head), each sequence's remaining positions as a decode
 * of its own, both in one launch (the prefix's items first), and the two
 * merged per (sequence, head) by the split reduce; the result is
 * paged_attention_decode's.
 *   prefix_tokens: a multiple of block_size, at most max_context_len; the
 *   first prefix_tokens / block_size entries of every table must name the
 *   same blocks (the caller's contract; the prefix is read through
 *   sequence 0's table).  A sequence shorter than the prefix sees only its
 *   own positions.  0 makes this paged_attention_decode.
 *   bf16 queries (PKV_ERR_DTYPE otherwise); bf16 or FP8 caches.  Other
 *   arguments are as for paged_attention_decode; the workspace is
 *   paged_attention_decode_shared_prefix_workspace_size bytes, its first
 *   4096 zero, and is left so.
 */
pkv_status_t paged_attention_decode_shared_prefix(
    void* out, const void* query,
    const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t prefix_tokens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size,
    void* workspace, size_t workspace_bytes,
    void* stream);

/* Workspace bytes paged_attention_decode_shared_prefix needs (0 for invalid
 * arguments). */
size_t paged_attention_decode_shared_prefix_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, int32_t prefix_tokens,
    int32_t q_dtype, int32_t cache_dtype, int32_t partition_size);

/*
 * paged_kv_block_copy -- copy whole blocks from one pool to another: the
 * copy-on-write of a shared block before a sequence writes into it (page
 * "vLLM的诞生背景：大模型推理的痛点与PagedAttention的破局", the limitations
 * paragraph: shared blocks need reference counts and copy-on-write), and
 * swapping blocks out to host memory and back in (page "PagedAttention 与连续
 * 批处理：LLM Serving 的底层架构拆解", section "PagedAttention：把显存做成虚拟内存":
 * inactive sequences' pages move to CPU memory and return when needed;
 * dpshk.com article, section 3.2: host-device copies run on a stream).
 *
 * For pair i, block block_pairs[2i] of the source pool is copied to block
 * block_pairs[2i+1] of the destination pool: the K and V tiles of every KV
 * head and, for FP8 pools, the block's K and V scales.  Both pools have the
 * layout above ([num_blocks][H_kv][bs][D], scales [num_blocks][H_kv]) and
 * the same dtype; they may be one pool (copy-on-write) or two (swap).
 *
 *   Pool pointers may be device memory or pinned host memory the device can
 *   address (hipHostMalloc, torch pin_memory): device -> host is a swap-out,
 *   host -> device a swap-in.  block_pairs is int32 [num_pairs][2] in memory
 *   the device can read.
 *   Destination blocks must be distinct, and when the pools are the same no
 *   destination may also be a source; then the result does not depend on
 *   the order of the copies.  Block ids must lie inside their pools (the
 *   caller's contract, not checked on the device).
 *   key_scale / value_scale pointers are used only for FP8 pools (may be
 *   NULL otherwise).
 *   num_pairs == 0 returns PKV_OK after the size and dtype checks without
 *   inspecting any pointer.
 */
pkv_status_t paged_kv_block_copy(
    const void* src_key_cache, const void* src_value_cache,
    const float* src_key_scale, const float* src_value_scale,
    void* dst_key_cache, void* dst_value_cache,
    float* dst_key_scale, float* dst_value_scale,
    const int32_t* block_pairs, int32_t num_pairs,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t cache_dtype,
    void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, partition choice and result as paged_attention_decode; the
 * workspace is instead a device array inside the library, one per device,
 * of PKV_DECODE_NOALLOC_MAX_WORKSPACE bytes, held until the process ends.
 * The call allocates nothing: it zeroes the array's counters (the leading
 * paged_attention_decode_workspace_counter_bytes(...)) with a small kernel
 * on `stream`, then runs the decode in it.
 *   A call whose paged_attention_decode_workspace_size(...) exceeds
 *   PKV_DECODE_NOALLOC_MAX_WORKSPACE returns PKV_ERR_WORKSPACE and enqueues
 *   nothing.  Other checks and errors are paged_attention_decode's.
 *   Every call on one device uses the same array and leaves its contents
 *   behind: calls that may run at the same time on one device race (order
 *   them on one stream, or with events).
 */
#define PKV_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)

pkv_status_t paged_attention_decode_noalloc(
    void* out, const void* query,
    const void* key_cache, const void* value_cache,
    const float* key_scale, const float* value_scale,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, int32_t q_dtype, int32_t cache_dtype,
    int32_t partition_size,
    void* stream);

/* PKV_DECODE_NOALLOC_MAX_WORKSPACE, as the library was built. */
size_t paged_attention_decode_noalloc_max_workspace(void);

/* Static, NUL-terminated description of a status code. */
const char* pkv_status_string(int32_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
