// Merge of split-context partitions.  Each partition p of a sequence left
// (m_p, l_p, acc_p): the running maximum (base-2 units), the sum of
// 2^(s - m_p) over its tokens and the unnormalised output.  One softmax over
// the whole context is recovered exactly (up to rounding) by
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// (Whole-context softmax: dpshk.com PagedAttention article, section 2.2.)
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(128) void decode_reduce_kernel(
    void* __restrict__ out, const int32_t* __restrict__ lens, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const float* __restrict__ ws_acc, int H, int D, int P, int NP) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int n = lens[seq];
  const int np = (n + P - 1) / P;
  if (np <= 1) return;  // written directly by the partition kernel
  const size_t base = ((size_t)seq * H + h) * NP;
  const float* pm = ws_m + base;
  const float* pl = ws_l + base;
  const float* pa = ws_acc + base * D;
  float M = kNegInf;
  for (int q = 0; q < np; ++q) M = fmaxf(M, pm[q]);
  float L = 0.f;
  for (int q = 0; q < np; ++q) L = fmaf(pl[q], __builtin_amdgcn_exp2f(pm[q] - M), L);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float O = 0.f;
    for (int q = 0; q < np; ++q) O = fmaf(pa[(size_t)q * D + d], __builtin_amdgcn_exp2f(pm[q] - M), O);
    const float o = O / L;
    const size_t oi = ((size_t)seq * H + h) * D + d;
    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(o);
    else reinterpret_cast<float*>(out)[oi] = o;
  }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a) {
  dim3 grid(a.H, a.S);
  if (a.q_dtype == PKV_BF16) {
    hipLaunchKernelGGL(decode_reduce_kernel<true>, grid, dim3(128), 0, a.stream, a.out, a.lens,
                       a.ws_m, a.ws_l, a.ws_acc, a.H, a.D, a.P, a.NP);
  } else {
    hipLaunchKernelGGL(decode_reduce_kernel<false>, grid, dim3(128), 0, a.stream, a.out, a.lens,
                       a.ws_m, a.ws_l, a.ws_acc, a.H, a.D, a.P, a.NP);
  }
  return hipGetLastError();
}

}  // namespace pkv
