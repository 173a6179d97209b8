// Merge of split-context partitions.  Each partition p of a sequence left
// (m_p, l_p, acc_p): the running maximum (base-2 units), the sum of
// 2^(s - m_p) over its tokens and the unnormalised output.  One softmax over
// the whole context is recovered exactly (up to rounding) by
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// (Whole-context softmax: dpshk.com PagedAttention article, section 2.2.)
//
// One workgroup of D threads per (sequence, query head); thread d merges
// acc_p[d] over the partitions in batches with an online maximum, all in
// registers.  The first batch's loads do not wait for the context length:
// they are clamped to the NP partition rows the workspace holds for every
// sequence, so they are in flight together with the load of the length.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kFirst = 4;   // partitions loaded before the context length is known
constexpr int kChunk = 16;  // partitions per later batch of independent loads

// Fold partitions [q0, q0 + U) (those below np) into the running (M, L, O).
template <int U>
__device__ __forceinline__ void merge_chunk(const float (&m)[U], const float (&l)[U],
                                            const float (&a)[U], int q0, int np, float& M,
                                            float& L, float& O) {
  float mc = kNegInf;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (q0 + u < np) mc = fmaxf(mc, m[u]);
  const float mn = fmaxf(M, mc);  // finite: every partition below np holds tokens
  const float r = __builtin_amdgcn_exp2f(M - mn);  // 0 while M is still -inf
  L *= r;
  O *= r;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (q0 + u < np) {
      const float w = __builtin_amdgcn_exp2f(m[u] - mn);
      L = fmaf(l[u], w, L);
      O = fmaf(a[u], w, O);
    }
  }
  M = mn;
}

template <bool OUT_BF16, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    void* __restrict__ out, const int32_t* __restrict__ lens, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const float* __restrict__ ws_acc, int H, int P, int NP) {
  constexpr int U0 = kFirst, U = kChunk;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int d = threadIdx.x;
  const size_t base = ((size_t)seq * H + h) * NP;
  const float* pm = ws_m + base;
  const float* pl = ws_l + base;
  const float* pa = ws_acc + base * D + d;

  float m0[U0], l0[U0], a0[U0];
#pragma unroll
  for (int u = 0; u < U0; ++u) a0[u] = pa[(size_t)min(u, NP - 1) * D];
  // Keep the scheduler from putting these vector loads behind the waits for
  // the scalar loads below.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U0; ++u) {
    const int q = min(u, NP - 1);
    m0[u] = pm[q];
    l0[u] = pl[q];
  }
  const int n = lens[seq];
  const int np = (n + P - 1) / P;  // one partition: written by the partition kernel
  float M = kNegInf, L = 0.f, O = 0.f;
  merge_chunk<U0>(m0, l0, a0, 0, np, M, L, O);
  for (int q0 = U0; q0 < np; q0 += U) {
    float m[U], l[U], a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + u, np - 1);
      m[u] = pm[q];
      l[u] = pl[q];
      a[u] = pa[(size_t)q * D];
    }
    merge_chunk<U>(m, l, a, q0, np, M, L, O);
  }
  // No branch before this point, so the first chunk's loads are issued
  // before the length arrives.
  if (np <= 1) return;
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
