// PagedAttention decode, vector-ALU kernel: one workgroup per (sequence,
// KV head [, chunk of its query heads], context partition).
//
// What is computed: softmax(q K^T * scale) V over the sequence's context
// (dpshk.com PagedAttention article "企业官网建设流程全解析", section 2.2),
// with K/V reached block by block through the block table (page
// "PagedAttention 与连续批处理…", section "PagedAttention：把显存做成虚拟内存").
// The article's per-block loop is kept as the iteration order, but the
// softmax is ONE softmax over the whole context, carried across blocks with a
// running maximum and sum (online softmax); partitions of a long context are
// merged by the reduce kernel with the same rule.
//
// Lane layout (wave64): lane = 16 * row + col.  A wave covers 4 token rows at
// a time; the 16 lanes of a DPP row hold one token's row, E = D / 16
// consecutive elements per lane, so every load instruction of a wave reads 4
// whole token rows (4 * D * elem bytes, contiguous within a block tile).
// Each DPP row runs its own online softmax over the tokens it sees; the 4
// rows x NW waves are merged through LDS at the end.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

struct ValuParams {
  const void* q;
  const void* kc;
  const void* vc;
  const float* ks;
  const float* vs;
  const int32_t* tables;
  const int32_t* lens;
  void* out;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int H, H_kv, G, chunks, max_blocks, P, NP, max_ctx;
  float scale_log2;
};

template <typename QT, typename CT, int D, int BS, int GMAX, int NW>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(ValuParams p) {
  constexpr int E = D / 16;                     // elements per lane per row
  constexpr int TPB = BS / 4;                   // token rows per DPP row per block
  using CS = typename CT::storage;
  constexpr int NWORDS = E * (int)sizeof(CS) / 4;
  constexpr int NSP = NW * 4;                   // sub-partials merged at the end

  __shared__ float s_m[NSP][GMAX];
  __shared__ float s_l[NSP][GMAX];
  __shared__ float s_acc[NSP][GMAX][D];

  const int part = blockIdx.x;
  const int chunk = blockIdx.y % p.chunks;
  const int kvh = blockIdx.y / p.chunks;
  const int seq = blockIdx.z;
  const int n = min(p.lens[seq], p.max_ctx);  // the grid covers max_ctx tokens
  const int start = part * p.P;
  if (part > 0 && start >= n) return;
  const int end = min(n, start + p.P);
  const int h0 = kvh * p.G + chunk * GMAX;
  const int nh = min(GMAX, p.G - chunk * GMAX);
  const int H = p.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int col = lane & 15;

  // Query rows of this chunk's heads, pre-multiplied by scale * log2(e) so the
  // softmax runs in base 2.
  float qr[GMAX][E];
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
#pragma unroll
    for (int e = 0; e < E; ++e) qr[j][e] = 0.f;
    if (j < nh) {
      const size_t qoff = ((size_t)seq * H + h0 + j) * D + col * E;
      if constexpr (sizeof(typename QT::storage) == 4) {
        const float* qp = reinterpret_cast<const float*>(p.q) + qoff;
#pragma unroll
        for (int e = 0; e < E; ++e) qr[j][e] = qp[e] * p.scale_log2;
      } else {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qoff;
#pragma unroll
        for (int e = 0; e < E; ++e) qr[j][e] = __uint_as_float((uint32_t)qp[e] << 16) * p.scale_log2;
      }
    }
  }

  float m[GMAX], l[GMAX], acc[GMAX][E];
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[j][e] = 0.f;
  }

  const int first_blk = start / BS;
  const int nblk = (n > start) ? (end + BS - 1) / BS - first_blk : 0;
  const size_t block_stride = (size_t)p.H_kv * BS * D;
  const CS* kbase = reinterpret_cast<const CS*>(p.kc) + (size_t)kvh * BS * D + col * E;
  const CS* vbase = reinterpret_cast<const CS*>(p.vc) + (size_t)kvh * BS * D + col * E;
  const int32_t* trow = p.tables + (size_t)seq * p.max_blocks;

  for (int jb = wave; jb < nblk; jb += NW) {
    const int blk = first_blk + jb;
    const int phys = trow[blk];
    const CS* kt = kbase + (size_t)phys * block_stride;
    const CS* vt = vbase + (size_t)phys * block_stride;
    float kf[TPB][E], vf[TPB][E];
    bool valid[TPB];
#pragma unroll
    for (int k = 0; k < TPB; ++k) {
      const int r = 4 * k + row;
      valid[k] = blk * BS + r < end;
      Words<NWORDS> kw, vw;
#pragma unroll
      for (int w = 0; w < NWORDS; ++w) { kw.w[w] = 0u; vw.w[w] = 0u; }
      if (valid[k]) {
        kw = load_words<NWORDS>(kt + r * D);
        vw = load_words<NWORDS>(vt + r * D);
      }
      words_to_f32<CT, E>(kw.w, kf[k]);
      words_to_f32<CT, E>(vw.w, vf[k]);
    }
    float ksc = 1.f, vsc = 1.f;
    if constexpr (sizeof(CS) == 1) {
      ksc = p.ks[(size_t)phys * p.H_kv + kvh];
      vsc = p.vs[(size_t)phys * p.H_kv + kvh];
    }
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      float s[TPB];
      float mloc = kNegInf;
#pragma unroll
      for (int k = 0; k < TPB; ++k) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot = fmaf(qr[j][e], kf[k][e], dot);
        dot = row_sum16(dot);
        if constexpr (sizeof(CS) == 1) dot *= ksc;
        s[k] = valid[k] ? dot : kNegInf;
        mloc = fmaxf(mloc, s[k]);
      }
      const float m_new = fmaxf(m[j], mloc);
      const float ms = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[j] - ms);
      float psum = 0.f;
      float pk[TPB];
#pragma unroll
      for (int k = 0; k < TPB; ++k) {
        pk[k] = __builtin_amdgcn_exp2f(s[k] - ms);
        psum += pk[k];
      }
      l[j] = fmaf(l[j], alpha, psum);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float a = acc[j][e] * alpha;
#pragma unroll
        for (int k = 0; k < TPB; ++k) {
          if constexpr (sizeof(CS) == 1) a = fmaf(pk[k] * vsc, vf[k][e], a);
          else a = fmaf(pk[k], vf[k][e], a);
        }
        acc[j][e] = a;
      }
      m[j] = m_new;
    }
  }

  // Merge the NW * 4 row-level softmax states.
  const int sp = wave * 4 + row;
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    if (col == 0) {
      s_m[sp][j] = m[j];
      s_l[sp][j] = l[j];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) s_acc[sp][j][col * E + e] = acc[j][e];
  }
  __syncthreads();

  const bool single = n <= p.P;
  for (int idx = tid; idx < nh * D; idx += NW * 64) {
    const int j = idx / D;
    const int d = idx - j * D;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < NSP; ++k) M = fmaxf(M, s_m[k][j]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int k = 0; k < NSP; ++k) {
        const float w = __builtin_amdgcn_exp2f(s_m[k][j] - M);
        L = fmaf(s_l[k][j], w, L);
        O = fmaf(s_acc[k][j][d], w, O);
      }
    }
    const int h = h0 + j;
    if (single) {
      const float o = L > 0.f ? O / L : 0.f;
      const size_t oi = ((size_t)seq * H + h) * D + d;
      if constexpr (sizeof(typename QT::storage) == 4) reinterpret_cast<float*>(p.out)[oi] = o;
      else reinterpret_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(o);
    } else {
      const size_t pi = ((size_t)seq * H + h) * p.NP + part;
      if constexpr (sizeof(typename QT::storage) == 4) p.ws_acc[pi * D + d] = O;
      else reinterpret_cast<uint16_t*>(p.ws_acc)[pi * D + d] = f32_to_bf16(O);
      if (d == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = L;
      }
    }
  }
}

template <typename QT, typename CT, int D, int BS, int GMAX>
hipError_t launch_g(const DecodeArgs& a, int chunks) {
  constexpr int NW = GMAX >= 8 ? 2 : 4;
  ValuParams p;
  p.q = a.q; p.kc = a.key_cache; p.vc = a.value_cache; p.ks = a.key_scale; p.vs = a.value_scale;
  p.tables = a.tables; p.lens = a.lens; p.out = a.out;
  p.ws_m = a.ws_m; p.ws_l = a.ws_l; p.ws_acc = a.ws_acc;
  p.H = a.H; p.H_kv = a.H_kv; p.G = a.H / a.H_kv; p.chunks = chunks;
  p.max_blocks = a.max_blocks; p.P = a.P; p.NP = a.NP; p.max_ctx = a.max_ctx;
  p.scale_log2 = a.scale * kLog2e;
  dim3 grid(a.NP, a.H_kv * chunks, a.S);
  hipLaunchKernelGGL((decode_valu_kernel<QT, CT, D, BS, GMAX, NW>), grid, dim3(NW * 64), 0,
                     a.stream, p);
  return hipGetLastError();
}

template <typename QT, typename CT, int D, int BS>
hipError_t launch_bs(const DecodeArgs& a) {
  const int G = a.H / a.H_kv;
  if (G == 1) return launch_g<QT, CT, D, BS, 1>(a, 1);
  if (G == 2) return launch_g<QT, CT, D, BS, 2>(a, 1);
  if (G <= 4) return launch_g<QT, CT, D, BS, 4>(a, 1);
  return launch_g<QT, CT, D, BS, 8>(a, (G + 7) / 8);
}

template <typename QT, typename CT, int D>
hipError_t launch_d(const DecodeArgs& a) {
  switch (a.bs) {
    case 8: return launch_bs<QT, CT, D, 8>(a);
    case 16: return launch_bs<QT, CT, D, 16>(a);
    default: return launch_bs<QT, CT, D, 32>(a);
  }
}

template <typename QT, typename CT>
hipError_t launch_qc(const DecodeArgs& a) {
  return a.D == 64 ? launch_d<QT, CT, 64>(a) : launch_d<QT, CT, 128>(a);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a) {
  if (a.cache_dtype == PKV_F32) return launch_qc<F32, F32>(a);
  if (a.cache_dtype == PKV_BF16) return launch_qc<BF16, BF16>(a);
  return launch_qc<BF16, FP8>(a);
}

}  // namespace pkv
