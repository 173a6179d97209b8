// Whole-block copies between two pools: copy-on-write of a shared block
// (page "vLLM的诞生背景：大模型推理的痛点与PagedAttention的破局", limitations
// paragraph) and swapping blocks to host memory and back (page
// "PagedAttention 与连续批处理：LLM Serving 的底层架构拆解", section
// "PagedAttention：把显存做成虚拟内存"; host-device copies on a stream:
// dpshk.com article, section 3.2).
//
// A block of one pool is H_kv * bs * D elements of K and as many of V
// (every KV head's tile, contiguous in the [num_blocks][H_kv][bs][D]
// layout), plus H_kv K and H_kv V scales for FP8 pools.  One launch moves
// every pair; each thread carries kVecPerThread independent 16-byte vectors
// (all loads issued before any store), and a pair spans as many workgroups
// as its vectors need, so a launch with few pairs still fills the chip.
// Pools in pinned host memory are read or written over the bus by the same
// kernel.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kVecPerThread = 4;

__global__ __launch_bounds__(kCopyThreads) void kv_block_copy_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, uint4* __restrict__ dst_k,
    uint4* __restrict__ dst_v, const float* __restrict__ src_ks, const float* __restrict__ src_vs,
    float* __restrict__ dst_ks, float* __restrict__ dst_vs, const int32_t* __restrict__ pairs,
    long long nvec, int wpp, long long pieces, int H_kv, int scaled) {
  // nvec: 16-byte vectors of one block's K (and of its V); wpp: workgroups
  // per pair; pieces: pairs * wpp.  The grid strides over the pieces.
  for (long long g = blockIdx.x; g < pieces; g += gridDim.x) {
    const long long i = g / wpp;
    const int piece = (int)(g - i * wpp);
    const long long src = pairs[2 * i];
    const long long dst = pairs[2 * i + 1];
    uint4 v[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const long long j = ((long long)piece * kVecPerThread + u) * kCopyThreads + threadIdx.x;
      if (j < 2 * nvec) {
        const bool is_v = j >= nvec;
        const long long jj = is_v ? j - nvec : j;
        v[u] = (is_v ? src_v : src_k)[src * nvec + jj];
      }
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const long long j = ((long long)piece * kVecPerThread + u) * kCopyThreads + threadIdx.x;
      if (j < 2 * nvec) {
        const bool is_v = j >= nvec;
        const long long jj = is_v ? j - nvec : j;
        (is_v ? dst_v : dst_k)[dst * nvec + jj] = v[u];
      }
    }
    if (scaled && piece == 0) {
      for (int t = threadIdx.x; t < 2 * H_kv; t += kCopyThreads) {
        const bool is_v = t >= H_kv;
        const int h = is_v ? t - H_kv : t;
        (is_v ? dst_vs : dst_ks)[dst * H_kv + h] = (is_v ? src_vs : src_ks)[src * H_kv + h];
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_block_copy(const BlockCopyArgs& a) {
  const int elem = a.cache_dtype == PKV_F32 ? 4 : (a.cache_dtype == PKV_BF16 ? 2 : 1);
  // bs * D * elem is a multiple of 16 for every supported (bs, D, dtype)
  const long long nvec = (long long)a.H_kv * a.bs * a.D * elem / 16;
  const int wpp = (int)((2 * nvec + (long long)kCopyThreads * kVecPerThread - 1) /
                        ((long long)kCopyThreads * kVecPerThread));
  const long long pieces = (long long)a.n * wpp;
  const unsigned grid = (unsigned)(pieces < (1LL << 20) ? pieces : (1LL << 20));
  hipLaunchKernelGGL(kv_block_copy_kernel, dim3(grid), dim3(kCopyThreads), 0, a.stream,
                     reinterpret_cast<const uint4*>(a.src_k), reinterpret_cast<const uint4*>(a.src_v),
                     reinterpret_cast<uint4*>(a.dst_k), reinterpret_cast<uint4*>(a.dst_v),
                     a.src_ks, a.src_vs, a.dst_ks, a.dst_vs, a.pairs, nvec, wpp, pieces, a.H_kv,
                     a.cache_dtype == PKV_FP8_E4M3 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace pkv
