// Merge of split-context partitions.  Each partition p of a sequence left
// (m_p, l_p, acc_p): the running maximum (base-2 units), the sum of
// 2^(s - m_p) over its tokens and the unnormalised output.  One softmax over
// the whole context is recovered exactly (up to rounding) by
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// (Whole-context softmax: dpshk.com PagedAttention article, section 2.2.)
// acc_p is fp32 for fp32 queries and bf16 for bf16 queries.
//
// One workgroup of D threads per (sequence, query token, query head); thread d merges
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
    const float* __restrict__ ws_l, const void* __restrict__ ws_acc, int H, int P, int NP,
    int M, int pre_slots, int len_off) {
  constexpr int U0 = kFirst, U = kChunk;
  // One workgroup per row (seq * M + t) * H + h: query token t of sequence
  // seq, query head h (M = 1 for decode).
  const size_t row = blockIdx.x;
  const int st = (int)(row / H);
  const int seq = st / M;
  const int t = st - seq * M;
  const int d = threadIdx.x;
  const size_t base = row * NP;
  const float* pm = ws_m + base;
  const float* pl = ws_l + base;
  // acc_p[d] of partition q, as float
  auto acc_at = [&](int q) -> float {
    const size_t i = (base + (size_t)q) * D + d;
    if constexpr (OUT_BF16)
      return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(ws_acc)[i] << 16);
    else
      return reinterpret_cast<const float*>(ws_acc)[i];
  };

  float m0[U0], l0[U0], a0[U0];
#pragma unroll
  for (int u = 0; u < U0; ++u) a0[u] = acc_at(min(u, NP - 1));
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
  // Token t sits at position n - M + t and sees the positions up to it: its
  // partitions are the first ceil(end / P) of the sequence's.  With a shared
  // prefix split off, the prefix's pre_slots partials come first and the
  // partitions cover the positions from len_off on.
  const int end = n - M + t + 1;
  const int np = pre_slots + (max(end - len_off, 0) + P - 1) / P;
  float Mx = kNegInf, L = 0.f, O = 0.f;
  merge_chunk<U0>(m0, l0, a0, 0, np, Mx, L, O);
  for (int q0 = U0; q0 < np; q0 += U) {
    float mm[U], l[U], a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + u, np - 1);
      mm[u] = pm[q];
      l[u] = pl[q];
      a[u] = acc_at(q);
    }
    merge_chunk<U>(mm, l, a, q0, np, Mx, L, O);
  }
  // No branch before this point, so the first chunk's loads are issued
  // before the length arrives.  A sequence of at most P tokens was written
  // directly by the partition kernel.
  if (pre_slots == 0 && n <= P) return;
  const float res = L > 0.f ? O / L : 0.f;
  const size_t oi = row * D + d;
  if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(res);
  else reinterpret_cast<float*>(out)[oi] = res;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  const unsigned grid = (unsigned)((size_t)a.S * a.M * a.H);
  if (a.q_dtype == PKV_BF16) {
    hipLaunchKernelGGL((decode_reduce_kernel<true, D>), grid, dim3(D), 0, a.stream, a.out, a.lens,
                       a.ws_m, a.ws_l, a.ws_acc, a.H, a.P, a.NP, a.M, a.prefix_slots,
                       a.len_off);
  } else {
    hipLaunchKernelGGL((decode_reduce_kernel<false, D>), grid, dim3(D), 0, a.stream, a.out,
                       a.lens, a.ws_m, a.ws_l, a.ws_acc, a.H, a.P, a.NP, a.M,
                       a.prefix_slots, a.len_off);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a) {
  return a.D == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace pkv
