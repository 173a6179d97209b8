// Measurement aids: what this GPU's HBM delivers to a plain read, as a
// practical ceiling for the bandwidth-bound decode kernels.
//
//   read probe:   every 16-byte vector of a buffer read once, in address
//                 order over a grid-stride loop (the best case);
//   gather probe: whole tiles of a pool read in the order of a list of tile
//                 ids (the access pattern of a paged decode: each
//                 (block, KV head) tile is contiguous, tiles are scattered).
//
// The loaded values are folded into one word that is stored only if it
// equals a value it never takes for finite test data, so the loads cannot be
// removed and nothing else is written.
#include <hip/hip_runtime.h>

#include "pagedkv_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr uint32_t kNever = 0x9e3779b9u;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4* __restrict__ buf,
                                                              size_t n_vec, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kUnroll - 1) * stride < n_vec; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n_vec; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == kNever) *sink = x;
}

// Each wave reads its own tiles, kUnroll at a time; a tile of tile_vec
// 16-byte vectors is read by the wave's lanes in address order.
__global__ __launch_bounds__(kThreads) void gather_probe_kernel(
    const uint4* __restrict__ buf, const int32_t* __restrict__ tiles, int num_tiles, int tile_vec,
    uint32_t* sink) {
  uint32_t x = 0;
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  for (int t0 = wave * kUnroll; t0 < num_tiles; t0 += waves * kUnroll) {
    int id[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) id[u] = tiles[min(t0 + u, num_tiles - 1)];
    for (int j = lane; j < tile_vec; j += 64) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = buf[(size_t)id[u] * tile_vec + j];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (t0 + u < num_tiles) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (x == kNever) *sink = x;
}

// Two workgroups of 4 waves per CU: on MI355X a streaming read peaked at
// about 6.3 TB/s with this grid and fell to 5.0-5.3 TB/s with 4 to 16
// workgroups per CU (more pages open at once); a tile gather reached
// 5.9-6.0 TB/s with 2 to 8.
unsigned probe_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return (unsigned)cus * 2;
}

}  // namespace

extern "C" {

pkv_status_t pkv_hbm_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return PKV_OK;
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return PKV_ERR_SHAPE;
  if (!buf || !sink) return PKV_ERR_NULL;
  hipLaunchKernelGGL(read_probe_kernel, dim3(probe_grid()), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(buf),
                     bytes / 16, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status_t pkv_hbm_gather_probe(const void* buf, const int32_t* tiles, int32_t num_tiles,
                                  int32_t tile_bytes, void* sink, void* stream) {
  if (num_tiles < 0 || tile_bytes <= 0 || tile_bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return PKV_ERR_SHAPE;
  if (num_tiles == 0) return PKV_OK;
  if (!buf || !tiles || !sink) return PKV_ERR_NULL;
  const unsigned waves = (unsigned)((num_tiles + kUnroll - 1) / kUnroll);
  const unsigned need = (waves + kThreads / 64 - 1) / (kThreads / 64);
  const unsigned grid = need < probe_grid() ? need : probe_grid();
  hipLaunchKernelGGL(gather_probe_kernel, dim3(grid), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(buf),
                     tiles, num_tiles, tile_bytes / 16, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
