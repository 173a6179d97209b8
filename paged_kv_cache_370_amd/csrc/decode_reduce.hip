// Merge of split-context partitions.  Each partition p of a sequence left
// (m_p, l_p, acc_p): the running maximum (base-2 units), the sum of
// 2^(s - m_p) over its tokens and the unnormalised output.  One softmax over
// the whole context is recovered exactly (up to rounding) by
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// (Whole-context softmax: dpshk.com PagedAttention article, section 2.2.)
// acc_p is fp32 for fp32 queries and bf16 for bf16 queries.
//
// One workgroup per (sequence, query token, query head); a thread merges
// acc_p[d] (two adjacent d for bf16 partials) over the partitions in
// batches with an online maximum, all in registers.  The first batch's
// loads do not wait for the context length: they are clamped to the NP
// partition rows the workspace holds for every sequence, so they are in
// flight together with the load of the length.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kFirst = 4;   // partitions loaded before the context length is known
constexpr int kChunk = 16;  // partitions per later batch of independent loads

// Fold partitions [q0, q0 + U) (those below np) into the running (M, L, O).
template <int U, int E>
__device__ __forceinline__ void merge_chunk(const float (&m)[U], const float (&l)[U],
                                            const float (&a)[U][E], int q0, int np, float& M,
                                            float& L, float (&O)[E]) {
  float mc = kNegInf;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (q0 + u < np) mc = fmaxf(mc, m[u]);
  const float mn = fmaxf(M, mc);  // finite: every partition below np holds tokens
  const float r = __builtin_amdgcn_exp2f(M - mn);  // 0 while M is still -inf
  L *= r;
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] *= r;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (q0 + u < np) {
      const float w = __builtin_amdgcn_exp2f(m[u] - mn);
      L = fmaf(l[u], w, L);
#pragma unroll
      for (int e = 0; e < E; ++e) O[e] = fmaf(a[u][e], w, O[e]);
    }
  }
  M = mn;
}

// bf16 partials: each thread merges two adjacent elements (one 4-byte load
// per partition); fp32 partials: one element per thread.
template <bool OUT_BF16, int D>
__global__ __launch_bounds__(OUT_BF16 ? D / 2 : D) void decode_reduce_kernel(
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
  constexpr int E = OUT_BF16 ? 2 : 1;
  const int d = threadIdx.x * E;
  const size_t base = row * NP;
  const float* pm = ws_m + base;
  const float* pl = ws_l + base;
  // acc_p[d .. d + E) of partition q, as floats
  auto acc_at = [&](int q, float (&v)[E]) {
    const size_t i = (base + (size_t)q) * D + d;
    if constexpr (OUT_BF16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(
          reinterpret_cast<const uint16_t*>(ws_acc) + i);
      v[0] = bf16_lo(w);
      v[1] = bf16_hi(w);
    } else {
      v[0] = reinterpret_cast<const float*>(ws_acc)[i];
    }
  };

  float m0[U0], l0[U0], a0[U0][E];
#pragma unroll
  for (int u = 0; u < U0; ++u) acc_at(min(u, NP - 1), a0[u]);
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
  float Mx = kNegInf, L = 0.f, O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  merge_chunk<U0, E>(m0, l0, a0, 0, np, Mx, L, O);
  for (int q0 = U0; q0 < np; q0 += U) {
    float mm[U], l[U], a[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + u, np - 1);
      mm[u] = pm[q];
      l[u] = pl[q];
      acc_at(q, a[u]);
    }
    merge_chunk<U, E>(mm, l, a, q0, np, Mx, L, O);
  }
  // No branch before this point, so the first chunk's loads are issued
  // before the length arrives.  A sequence of at most P tokens was written
  // directly by the partition kernel.
  if (pre_slots == 0 && n <= P) return;
  const size_t oi = row * D + d;
  if constexpr (OUT_BF16) {
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + oi) =
        (uint32_t)f32_to_bf16(L > 0.f ? O[0] / L : 0.f) |
        ((uint32_t)f32_to_bf16(L > 0.f ? O[1] / L : 0.f) << 16);
  } else {
    reinterpret_cast<float*>(out)[oi] = L > 0.f ? O[0] / L : 0.f;
  }
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  const unsigned grid = (unsigned)((size_t)a.S * a.M * a.H);
  if (a.q_dtype == PKV_BF16) {
    hipLaunchKernelGGL((decode_reduce_kernel<true, D>), grid, dim3(D / 2), 0, a.stream, a.out, a.lens,
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
