// Merge of split-context partitions.  Each partition p of a sequence left
// (m_p, l_p, acc_p): the running maximum (base-2 units), the sum of
// 2^(s - m_p) over its tokens and the unnormalised output.  One softmax over
// the whole context is recovered exactly (up to rounding) by
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// (Whole-context softmax: dpshk.com PagedAttention article, section 2.2.)
//
// One workgroup of D threads per (sequence, query head): the threads first
// reduce M and L over the partitions together (weights kept in LDS), then
// thread d sums w_p acc_p[d] with several independent loads in flight.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kCachedWeights = 2048;  // partitions whose weight is kept in LDS

template <int NWAVE>
__device__ __forceinline__ float block_max(float x, float* s_red) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = s_red[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) r = fmaxf(r, s_red[w]);
  __syncthreads();
  return r;
}

template <int NWAVE>
__device__ __forceinline__ float block_sum(float x, float* s_red) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) r += s_red[w];
  __syncthreads();
  return r;
}

template <bool OUT_BF16, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    void* __restrict__ out, const int32_t* __restrict__ lens, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const float* __restrict__ ws_acc, int H, int P, int NP) {
  constexpr int NWAVE = D / 64;
  __shared__ float s_w[kCachedWeights];
  __shared__ float s_red[NWAVE];
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int n = lens[seq];
  const int np = (n + P - 1) / P;
  if (np <= 1) return;  // written directly by the partition kernel
  const int d = threadIdx.x;
  const size_t base = ((size_t)seq * H + h) * NP;
  const float* pm = ws_m + base;
  const float* pl = ws_l + base;
  const float* pa = ws_acc + base * D + d;

  float M = kNegInf;
  for (int q = d; q < np; q += D) M = fmaxf(M, pm[q]);
  M = block_max<NWAVE>(M, s_red);
  float L = 0.f;
  for (int q = d; q < np; q += D) {
    const float w = __builtin_amdgcn_exp2f(pm[q] - M);
    if (q < kCachedWeights) s_w[q] = w;
    L = fmaf(pl[q], w, L);
  }
  L = block_sum<NWAVE>(L, s_red);  // its barrier also publishes s_w

  constexpr int U = 8;
  float o[U];
#pragma unroll
  for (int u = 0; u < U; ++u) o[u] = 0.f;
  int q = 0;
  for (; q + U <= np; q += U) {
    float a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = pa[(size_t)(q + u) * D];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int qq = q + u;
      const float w = qq < kCachedWeights ? s_w[qq] : __builtin_amdgcn_exp2f(pm[qq] - M);
      o[u] = fmaf(a[u], w, o[u]);
    }
  }
  for (; q < np; ++q) {
    const float w = q < kCachedWeights ? s_w[q] : __builtin_amdgcn_exp2f(pm[q] - M);
    o[0] = fmaf(pa[(size_t)q * D], w, o[0]);
  }
  float O = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) O += o[u];
  const float res = O / L;
  const size_t oi = ((size_t)seq * H + h) * D + d;
  if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(res);
  else reinterpret_cast<float*>(out)[oi] = res;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  dim3 grid(a.H, a.S);
  if (a.q_dtype == PKV_BF16) {
    hipLaunchKernelGGL((decode_reduce_kernel<true, D>), grid, dim3(D), 0, a.stream, a.out, a.lens,
                       a.ws_m, a.ws_l, a.ws_acc, a.H, a.P, a.NP);
  } else {
    hipLaunchKernelGGL((decode_reduce_kernel<false, D>), grid, dim3(D), 0, a.stream, a.out,
                       a.lens, a.ws_m, a.ws_l, a.ws_acc, a.H, a.P, a.NP);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a) {
  return a.D == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace pkv
