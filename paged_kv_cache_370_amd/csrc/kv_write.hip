// Paged KV write: scatter new K/V rows into their slots (copy), or quantise
// them to OCP E4M3FN with per-(block, KV head) scales.
//
// Block structure: dpshk.com PagedAttention article ("企业官网建设流程全解析"),
// section 2.1 (fixed-size blocks of token rows); FP8 storage of blocks: same
// article, section 3.2.  The slot mapping (slot = block * bs + offset) is the
// write side of the block table (page "vLLM的诞生背景…", section
// "PagedAttention的破局思路").
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// One 16-byte vector per thread: a token's K and V rows (every KV head,
// 2 * H_kv * row_vec vectors; row bytes D * elem are 128..512, a multiple of
// 16) span wpt workgroups, so each thread makes one dependent load (its
// token's slot, uniform over the workgroup) before its copy.  The grid
// strides over (token, piece) pairs when there are more than it holds.
__global__ __launch_bounds__(256) void kv_write_copy_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int32_t* __restrict__ slots, int H_kv, int row_vec, int bs, int wpt, long long pieces,
    int num_slots) {
  const int per_token = H_kv * row_vec;  // 16-byte vectors per token per K or V
  for (long long g = blockIdx.x; g < pieces; g += gridDim.x) {
    const long long t = g / wpt;
    const int i = (int)(g - t * wpt) * 256 + (int)threadIdx.x;
    const int s = slots[t];
    if (s < 0 || s >= num_slots || i >= 2 * per_token) continue;
    const bool is_v = i >= per_token;
    const int j = is_v ? i - per_token : i;
    const int h = j / row_vec;
    const int v = j - h * row_vec;
    const int b = s / bs;
    const int o = s - b * bs;
    const size_t src = (size_t)t * per_token + j;
    const size_t dst = (((size_t)b * H_kv + h) * bs + o) * row_vec + v;
    if (is_v) value_cache[dst] = value[src];
    else key_cache[dst] = key[src];
  }
}

// Slots the pool holds (slot values are int32, so at most INT32_MAX + 1);
// a slot at or past it is skipped like a negative one.
int pool_slots(const WriteArgs& a) {
  const long long n = (long long)a.num_blocks * a.bs;
  return n > 0x7fffffffLL ? 0x7fffffff : (int)n;
}

// ---------------------------------------------------------------- FP8 path
// Workspace: one entry per (block, KV head) of four 32-bit words: amax of K
// and of V (float bits), the call's rows in it, and "fresh" (its offset 0 is
// written).  All zero between calls.  Two launches:
//   1. per (token, KV head) row: atomicMax of the row's |K| and |V| on the
//      float bits (non-negative floats order like their unsigned bit
//      patterns), count the row in, and mark the entry fresh at offset 0;
//   2. per row: pick the scale (fresh: from amax; else the stored one) and
//      encode; then count the row out, and the entry's last row returns it
//      to zero.  A row counts out only after its own read of the entry has
//      returned (an explicit wait), so the last one clears it after every
//      read; no cache maintenance is needed (the entry's words change only
//      at the L2, by atomics and by the last row's store).
constexpr int kEntryWords = 4;  // amax K, amax V, rows, fresh
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt not waited for

// Row geometry of the FP8 write kernels: a lane handles VEC consecutive
// source elements (one 16-byte load), LPR lanes cover a (token, KV head) row
// of D elements, and a wave handles RPW rows at once.
template <typename ST, int D>
struct Fp8Rows {
  static constexpr int VEC = 16 / (int)sizeof(ST);
  static constexpr int LPR = D / VEC;
  static constexpr int RPW = 64 / LPR;
};

// The lane's VEC source elements as floats (bf16 bits or fp32).
template <typename ST>
__device__ __forceinline__ void load_src(const ST* p, float (&x)[16 / sizeof(ST)]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  if constexpr (sizeof(ST) == 4) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

// Maximum over the LPR lanes of a row (aligned groups of LPR lanes).
template <int LPR>
__device__ __forceinline__ float row_group_max(float x) {
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Per (token, KV head) row: amax of |K| and |V| over the row, folded into the
// block's entry with atomicMax on the float bits (NaN wins, as in an ordinary
// maximum), and the block marked fresh when the row is its offset 0.
template <typename ST, int D>
__global__ __launch_bounds__(256) void fp8_amax_kernel(
    const ST* __restrict__ key, const ST* __restrict__ value,
    const int32_t* __restrict__ slots, int T, int bs, int H_kv, int num_slots,
    uint32_t* __restrict__ entries) {
  using R = Fp8Rows<ST, D>;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int row = gw * R::RPW + lane / R::LPR;
  const int part = lane % R::LPR;
  const bool ok = row < T * H_kv;
  const int rr = ok ? row : 0;
  const int t = rr / H_kv;
  const int h = rr - t * H_kv;
  float xk[R::VEC], xv[R::VEC];
  load_src<ST>(key + (size_t)rr * D + part * R::VEC, xk);
  load_src<ST>(value + (size_t)rr * D + part * R::VEC, xv);
  float mk = 0.f, mv = 0.f, nk = 0.f, nv = 0.f;
#pragma unroll
  for (int i = 0; i < R::VEC; ++i) {
    mk = fmaxf(mk, fabsf(xk[i]));
    mv = fmaxf(mv, fabsf(xv[i]));
    nk = (xk[i] != xk[i]) ? 1.f : nk;
    nv = (xv[i] != xv[i]) ? 1.f : nv;
  }
  mk = row_group_max<R::LPR>(mk);
  mv = row_group_max<R::LPR>(mv);
  nk = row_group_max<R::LPR>(nk);
  nv = row_group_max<R::LPR>(nv);
  const int s = ok ? slots[t] : -1;
  if (part == 0 && s >= 0 && s < num_slots) {
    const int b = s / bs;
    const int o = s - b * bs;
    const uint32_t bk = nk > 0.f ? 0x7fc00000u : __float_as_uint(mk);
    const uint32_t bv = nv > 0.f ? 0x7fc00000u : __float_as_uint(mv);
    uint32_t* e = entries + ((size_t)b * H_kv + h) * kEntryWords;
    atomicMax(&e[0], bk);
    atomicMax(&e[1], bv);
    atomicAdd(&e[2], 1u);
    if (o == 0) atomicOr(&e[3], 1u);
  }
}

__device__ __forceinline__ float fp8_scale_from_amax(uint32_t bits) {
  const float s = __uint_as_float(bits) / 448.0f;
  const float flt_min = 1.17549435e-38f;
  return (s < flt_min) ? flt_min : s;  // NaN stays NaN
}

// Per (token, KV head) row: the block's scales (set from amax when the
// block is fresh, else the stored ones), then the row's codes, VEC per lane
// in one store.
template <typename ST, int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(
    const ST* __restrict__ key, const ST* __restrict__ value,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    float* __restrict__ key_scale, float* __restrict__ value_scale,
    const int32_t* __restrict__ slots, int T, int bs, int H_kv, int num_slots,
    uint32_t* __restrict__ entries) {
  using R = Fp8Rows<ST, D>;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int row = gw * R::RPW + lane / R::LPR;
  const int part = lane % R::LPR;
  if (row >= T * H_kv) return;
  const int t = row / H_kv;
  const int h = row - t * H_kv;
  const int s = slots[t];
  if (s < 0 || s >= num_slots) return;
  const int b = s / bs;
  const int o = s - b * bs;
  const size_t sidx = (size_t)b * H_kv + h;
  float xk[R::VEC], xv[R::VEC];
  load_src<ST>(key + (size_t)row * D + part * R::VEC, xk);
  load_src<ST>(value + (size_t)row * D + part * R::VEC, xv);
  float sk, sv;
  uint32_t* e = entries + sidx * kEntryWords;
  const uint4 ent = *reinterpret_cast<const uint4*>(e);  // amax K, amax V, rows, fresh
  if (ent.w) {
    sk = fp8_scale_from_amax(ent.x);
    sv = fp8_scale_from_amax(ent.y);
    if (part == 0) {  // every token of the block stores the same value
      key_scale[sidx] = sk;
      value_scale[sidx] = sv;
    }
  } else {
    sk = key_scale[sidx];
    sv = value_scale[sidx];
  }
  if (part == 0) {
    // Count the row out once the wave's read of the entry has returned;
    // the entry's last row returns it to zero for the next call.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    asm volatile("" ::: "memory");
    if (atomicSub(&e[2], 1u) == 1u) *reinterpret_cast<uint4*>(e) = make_uint4(0u, 0u, 0u, 0u);
  }
  // Correctly rounded float32 quotient: the double quotient rounded once more
  // to float equals the float quotient (53 >= 2*24 + 2).
  const double dk = (double)sk, dv = (double)sv;
  uint32_t ck[R::VEC / 4], cv[R::VEC / 4];
#pragma unroll
  for (int i = 0; i < R::VEC / 4; ++i) {
    ck[i] = cv[i] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ck[i] |= f32_to_e4m3((float)((double)xk[4 * i + j] / dk)) << (8 * j);
      cv[i] |= f32_to_e4m3((float)((double)xv[4 * i + j] / dv)) << (8 * j);
    }
  }
  uint8_t* kd = key_cache + (sidx * bs + o) * D + part * R::VEC;
  uint8_t* vd = value_cache + (sidx * bs + o) * D + part * R::VEC;
  if constexpr (R::VEC == 8) {
    *reinterpret_cast<uint2*>(kd) = make_uint2(ck[0], ck[1]);
    *reinterpret_cast<uint2*>(vd) = make_uint2(cv[0], cv[1]);
  } else {
    *reinterpret_cast<uint32_t*>(kd) = ck[0];
    *reinterpret_cast<uint32_t*>(vd) = cv[0];
  }
}

template <typename ST, int D>
hipError_t fp8_launch(const WriteArgs& a) {
  uint32_t* entries = reinterpret_cast<uint32_t*>(a.workspace);
  const ST* key = reinterpret_cast<const ST*>(a.key);
  const ST* value = reinterpret_cast<const ST*>(a.value);
  const int num_slots = pool_slots(a);  // slots past the pool are skipped
  const int rows = a.T * a.H_kv;
  const int waves = (rows + Fp8Rows<ST, D>::RPW - 1) / Fp8Rows<ST, D>::RPW;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((fp8_amax_kernel<ST, D>), dim3(blocks), dim3(256), 0, a.stream, key, value,
                     a.slots, a.T, a.bs, a.H_kv, num_slots, entries);
  hipLaunchKernelGGL((fp8_quant_kernel<ST, D>), dim3(blocks), dim3(256), 0, a.stream, key, value,
                     reinterpret_cast<uint8_t*>(a.key_cache),
                     reinterpret_cast<uint8_t*>(a.value_cache), a.key_scale, a.value_scale,
                     a.slots, a.T, a.bs, a.H_kv, num_slots, entries);
  return hipGetLastError();
}

}  // namespace

size_t kv_write_fp8_workspace(int num_blocks, int H_kv) {
  return (size_t)num_blocks * H_kv * kEntryWords * sizeof(uint32_t);
}

hipError_t launch_kv_write_copy(const WriteArgs& a) {
  const int elem = a.cache_dtype == PKV_F32 ? 4 : 2;
  const int row_vec = a.D * elem / 16;
  const int wpt = (2 * a.H_kv * row_vec + 255) / 256;
  const long long pieces = (long long)a.T * wpt;
  const unsigned grid = (unsigned)(pieces < (1LL << 20) ? pieces : (1LL << 20));
  hipLaunchKernelGGL(kv_write_copy_kernel, dim3(grid), dim3(256), 0, a.stream,
                     reinterpret_cast<const uint4*>(a.key), reinterpret_cast<const uint4*>(a.value),
                     reinterpret_cast<uint4*>(a.key_cache), reinterpret_cast<uint4*>(a.value_cache),
                     a.slots, a.H_kv, row_vec, a.bs, wpt, pieces, pool_slots(a));
  return hipGetLastError();
}

hipError_t launch_kv_write_fp8(const WriteArgs& a) {
  if (a.src_dtype == PKV_BF16) {
    return a.D == 64 ? fp8_launch<uint16_t, 64>(a) : fp8_launch<uint16_t, 128>(a);
  }
  return a.D == 64 ? fp8_launch<float, 64>(a) : fp8_launch<float, 128>(a);
}

}  // namespace pkv
