// Merge of split-context partitions.  Each partition p of a sequence left
// (m_p, l_p, acc_p): the running maximum (base-2 units), the sum of
// 2^(s - m_p) over its tokens and the unnormalised output.  One softmax over
// the whole context is recovered exactly (up to rounding) by
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// (Whole-context softmax: dpshk.com PagedAttention article, section 2.2.)
// acc_p is fp32 for fp32 queries and bf16 for bf16 queries.
//
// One workgroup per (sequence, query token, query head), in four groups of
// threads that each take a quarter of the partition slots; a thread merges
// acc_p[d] (two adjacent d for bf16 partials) over its group's partitions in
// batches with an online maximum, in registers, and the groups' states
// merge through LDS.  The first batch's loads do not wait for the context
// length: they are clamped to the NP partition rows the workspace holds for
// every sequence, so they are in flight together with the load of the
// length.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kFirst = 4;   // partitions loaded before the context length is known
constexpr int kFirstWide = 16;  // the same with several thread groups per row
constexpr int kChunk = 16;  // partitions per later batch of independent loads
constexpr int kRowWaves = 4;  // most thread groups that split one row's partition slots

// Fold partitions [q0, q0 + U) (those below hi) into the running (M, L, O).
// A batch without a valid partition leaves the state as it is.
template <int U, int E>
__device__ __forceinline__ void merge_chunk(const float (&m)[U], const float (&l)[U],
                                            const float (&a)[U][E], int q0, int hi, float& M,
                                            float& L, float (&O)[E]) {
  float mc = kNegInf;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (q0 + u < hi) mc = fmaxf(mc, m[u]);
  if (mc == kNegInf) return;  // same for every thread of the row
  const float mn = fmaxf(M, mc);
  const float r = __builtin_amdgcn_exp2f(M - mn);  // 0 while M is still -inf
  L *= r;
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] *= r;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (q0 + u < hi) {
      const float w = __builtin_amdgcn_exp2f(m[u] - mn);
      L = fmaf(l[u], w, L);
#pragma unroll
      for (int e = 0; e < E; ++e) O[e] = fmaf(a[u][e], w, O[e]);
    }
  }
  M = mn;
}

// bf16 partials: a thread merges two adjacent elements (one 4-byte load per
// partition); fp32 partials: one element.  With many partition slots, up to
// kRowWaves groups of threads (blockDim.x / (D / E); one wave each for bf16,
// D = 128) take a contiguous share of the slots each, so a long context's
// partials are read in few round trips; the groups' states merge through
// LDS.
template <bool OUT_BF16, int D, int U0>
__global__ __launch_bounds__((OUT_BF16 ? D / 2 : D) * kRowWaves) void decode_reduce_kernel(
    void* __restrict__ out, const int32_t* __restrict__ lens, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const void* __restrict__ ws_acc, int H, int P, int NP,
    int M, int pre_slots, int len_off) {
  constexpr int U = kChunk;
  constexpr int E = OUT_BF16 ? 2 : 1;
  constexpr int TPR = D / E;  // threads per group
  __shared__ float s_M[kRowWaves], s_L[kRowWaves];
  __shared__ float s_O[kRowWaves][D];
  // One workgroup per row (seq * M + t) * H + h: query token t of sequence
  // seq, query head h (M = 1 for decode).
  const size_t row = blockIdx.x;
  const int st = (int)(row / H);
  const int seq = st / M;
  const int t = st - seq * M;
  const int grp = (int)threadIdx.x / TPR;
  const int d = ((int)threadIdx.x - grp * TPR) * E;
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
  // This group's slots: [lo, lo + cw), of which those below np hold tokens.
  const int groups = (int)blockDim.x / TPR;
  const int cw = (NP + groups - 1) / groups;
  const int lo = grp * cw;

  float m0[U0], l0[U0], a0[U0][E];
#pragma unroll
  for (int u = 0; u < U0; ++u) acc_at(min(lo + u, NP - 1), a0[u]);
  // Keep the scheduler from putting these vector loads behind the waits for
  // the scalar loads below.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U0; ++u) {
    const int q = min(lo + u, NP - 1);
    m0[u] = pm[q];
    l0[u] = pl[q];
  }
  const int n = lens[seq];
  // Token t sits at position n - M + t and sees the positions up to it: its
  // partitions are the first ceil(end / P) of the sequence's.  With a shared
  // prefix split off, the prefix's pre_slots partials come first and the
  // partitions cover the positions from len_off on.
  const int end = n - M + t + 1;
  // (never more than the NP slots a row holds, whatever the length says)
  const int np = min(NP, pre_slots + (max(end - len_off, 0) + P - 1) / P);
  const int hi = min(np, lo + cw);
  float Mx = kNegInf, L = 0.f, O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  merge_chunk<U0, E>(m0, l0, a0, lo, hi, Mx, L, O);
  for (int q0 = lo + U0; q0 < hi; q0 += U) {
    float mm[U], l[U], a[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + u, hi - 1);
      mm[u] = pm[q];
      l[u] = pl[q];
      acc_at(q, a[u]);
    }
    merge_chunk<U, E>(mm, l, a, q0, hi, Mx, L, O);
  }
  // No branch before this point, so the first chunk's loads are issued
  // before the length arrives.  A sequence of at most P tokens was written
  // directly by the partition kernel (the same for the whole workgroup).
  if (pre_slots == 0 && n <= P) return;
  const size_t oi = row * D + d;
  auto store = [&](float Lr, const float (&Or)[E]) {
    if constexpr (OUT_BF16) {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + oi) =
          (uint32_t)f32_to_bf16(Lr > 0.f ? Or[0] / Lr : 0.f) |
          ((uint32_t)f32_to_bf16(Lr > 0.f ? Or[1] / Lr : 0.f) << 16);
    } else {
      reinterpret_cast<float*>(out)[oi] = Lr > 0.f ? Or[0] / Lr : 0.f;
    }
  };
  if (groups == 1) {
    store(L, O);
    return;
  }
  if (d == 0) {
    s_M[grp] = Mx;
    s_L[grp] = L;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) s_O[grp][d + e] = O[e];
  __syncthreads();
  if (grp != 0) return;
  float Mt = kNegInf;
#pragma unroll
  for (int g = 0; g < kRowWaves; ++g)
    if (g < groups) Mt = fmaxf(Mt, s_M[g]);
  float Lt = 0.f, Ot[E];
#pragma unroll
  for (int e = 0; e < E; ++e) Ot[e] = 0.f;
#pragma unroll
  for (int g = 0; g < kRowWaves; ++g) {
    if (g >= groups) break;
    const float w = s_M[g] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(s_M[g] - Mt);
    Lt = fmaf(s_L[g], w, Lt);
#pragma unroll
    for (int e = 0; e < E; ++e) Ot[e] = fmaf(s_O[g][d + e], w, Ot[e]);
  }
  store(Lt, Ot);
}

// Thread groups per row: one while a row has few slots (more groups would
// only add idle waves: measured slower up to 8 slots), up to kRowWaves for
// long contexts (32K tokens in 512-token partitions: 10.6 -> 8.0 us).
int row_groups(int NP) { return NP > 32 ? kRowWaves : (NP > 8 ? 2 : 1); }

template <bool OUT_BF16, int D, int U0>
hipError_t launch_u(const DecodeArgs& a, int groups) {
  const unsigned grid = (unsigned)((size_t)a.S * a.M * a.H);
  hipLaunchKernelGGL((decode_reduce_kernel<OUT_BF16, D, U0>), grid,
                     dim3((OUT_BF16 ? D / 2 : D) * groups), 0, a.stream, a.out, a.lens, a.ws_m,
                     a.ws_l, a.ws_acc, a.H, a.P, a.NP, a.M, a.prefix_slots, a.len_off);
  return hipGetLastError();
}

// With several groups per row each group's first batch is its whole share
// of up to 16 slots, in flight before the context length arrives.
template <bool OUT_BF16, int D>
hipError_t launch_q(const DecodeArgs& a) {
  const int groups = row_groups(a.NP);
  return groups > 1 ? launch_u<OUT_BF16, D, kFirstWide>(a, groups)
                    : launch_u<OUT_BF16, D, kFirst>(a, groups);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  return a.q_dtype == PKV_BF16 ? launch_q<true, D>(a) : launch_q<false, D>(a);
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a) {
  return a.D == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace pkv
