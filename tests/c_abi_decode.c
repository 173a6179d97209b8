/*
 * A decode step through the C ABI alone (no Python, no PyTorch): device
 * buffers from hipMalloc, the step's write with paged_kv_cache_write, then
 * paged_attention_decode, results copied back.  Inputs and outputs are raw
 * little-endian files in a directory given on the command line; the GPU test
 * that runs it checks the outputs against the CPU oracle.
 *
 *   c_abi_decode DIR S H H_KV D BS NUM_BLOCKS MAX_BLOCKS MAX_CTX SCALE
 *
 * reads  DIR/{q,kc,vc,key,value}.bin (bf16 bits), DIR/{tables,lens,slots}.bin
 * writes DIR/{out,kc_out,vc_out}.bin
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "pagedkv.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  void* p = malloc(bytes ? bytes : 1);
  if (fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
}

/* A device buffer of `bytes`, holding a copy of `host` unless it is NULL. */
static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess) { fprintf(stderr, "hipMalloc\n"); exit(3); }
  if (host && bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "hipMemcpy\n");
    exit(3);
  }
  return d;
}

#define CHECK(call)                                                                   \
  do {                                                                                \
    pkv_status_t st_ = (call);                                                        \
    if (st_ != PKV_OK) {                                                              \
      fprintf(stderr, "%s: %s\n", #call, pkv_status_string(st_));                     \
      return 4;                                                                       \
    }                                                                                 \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 11) { fprintf(stderr, "usage: see the file header\n"); return 1; }
  const char* dir = argv[1];
  const int S = atoi(argv[2]), H = atoi(argv[3]), H_kv = atoi(argv[4]), D = atoi(argv[5]);
  const int bs = atoi(argv[6]), nb = atoi(argv[7]), max_blocks = atoi(argv[8]);
  const int max_ctx = atoi(argv[9]);
  const float scale = (float)atof(argv[10]);
  const size_t q_bytes = (size_t)S * H * D * 2;
  const size_t pool_bytes = (size_t)nb * H_kv * bs * D * 2;
  const size_t row_bytes = (size_t)S * H_kv * D * 2;
  void* q = read_file(dir, "q.bin", q_bytes);
  void* kc = read_file(dir, "kc.bin", pool_bytes);
  void* vc = read_file(dir, "vc.bin", pool_bytes);
  void* key = read_file(dir, "key.bin", row_bytes);
  void* value = read_file(dir, "value.bin", row_bytes);
  void* tables = read_file(dir, "tables.bin", (size_t)S * max_blocks * 4);
  void* lens = read_file(dir, "lens.bin", (size_t)S * 4);
  void* slots = read_file(dir, "slots.bin", (size_t)S * 4);

  void* d_q = to_device(q, q_bytes);
  void* d_kc = to_device(kc, pool_bytes);
  void* d_vc = to_device(vc, pool_bytes);
  void* d_key = to_device(key, row_bytes);
  void* d_value = to_device(value, row_bytes);
  void* d_tables = to_device(tables, (size_t)S * max_blocks * 4);
  void* d_lens = to_device(lens, (size_t)S * 4);
  void* d_slots = to_device(slots, (size_t)S * 4);
  void* d_out = to_device(NULL, q_bytes);

  const size_t ws_bytes = paged_attention_decode_workspace_size(S, H, H_kv, D, bs, max_ctx,
                                                                PKV_BF16, PKV_BF16, 0);
  void* d_ws = to_device(NULL, ws_bytes);
  if (hipMemset(d_ws, 0, ws_bytes) != hipSuccess) { fprintf(stderr, "hipMemset\n"); return 3; }

  CHECK(paged_kv_cache_write(d_key, d_value, d_kc, d_vc, NULL, NULL, (const int32_t*)d_slots, S,
                             H_kv, D, bs, nb, PKV_BF16, PKV_BF16, NULL, 0, NULL));
  CHECK(paged_attention_decode(d_out, d_q, d_kc, d_vc, NULL, NULL, (const int32_t*)d_tables,
                               (const int32_t*)d_lens, S, H, H_kv, D, bs, max_blocks, max_ctx,
                               scale, PKV_BF16, PKV_BF16, 0, d_ws, ws_bytes, NULL));
  if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "hipDeviceSynchronize\n"); return 3; }

  void* out = malloc(q_bytes);
  if (hipMemcpy(out, d_out, q_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(kc, d_kc, pool_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(vc, d_vc, pool_bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "hipMemcpy back\n");
    return 3;
  }
  write_file(dir, "out.bin", out, q_bytes);
  write_file(dir, "kc_out.bin", kc, pool_bytes);
  write_file(dir, "vc_out.bin", vc, pool_bytes);
  printf("ok\n");
  return 0;
}
