// PagedAttention decode on the matrix cores: one workgroup per (sequence,
// KV head, chunk of up to 16 of its query heads, context partition).
//
// What is computed: softmax(q K^T * scale) V over the sequence's context
// (dpshk.com PagedAttention article "企业官网建设流程全解析", section 2.2), K/V
// reached block by block through the block table (page "PagedAttention 与连续
// 批处理…", section "PagedAttention：把显存做成虚拟内存").  ONE softmax over
// the whole context, carried across 32-token chunks with a running maximum
// and sum; partitions are merged by the reduce kernel.
//
// Why MFMA here: the query heads that share a KV head turn both products
// into small dense contractions, [16 tokens x D] . [D x 16 heads] for the
// scores and [D x 32 tokens] . [32 tokens x 16 heads] for P V, so every K/V
// byte fetched from HBM feeds up to 16 heads without vector-ALU dot
// products.  Heads beyond the group are zero columns.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64; l = 16 q + r):
//   A: lane l holds A[r][8q .. 8q+7]    B: lane l holds B[8q .. 8q+7][r]
//   C: lane l holds C[4q .. 4q+3][r]
// Scores S^T = K . Q^T take K rows as A straight from HBM: lane l loads
// D/4 contiguous elements of token r, and the contraction index d is permuted
// identically in K and Q (d = (D/4) q + 8 c + e for step c), which leaves the
// dot products unchanged.  The result gives every lane ONE head (column r)
// and four tokens, so the running max / sum are per lane.  For P V the lane's
// eight probabilities (tokens 4q..4q+3 of both 16-token halves) are exactly
// the B operand of O^T = V^T . P^T; V^T fragments come from the V tile staged
// in LDS through ds_read_b64_tr_b16, which hands lane i of a 16-lane group
// element (i % 4) of the 8-byte row addressed by lane 4 e + i / 4.
//
// Masking: loads use clamped (always valid) addresses and never branch; the
// scores of tokens past the partition end are replaced by -inf and their V
// rows by zeros before any product, so poisoned or stale slots cannot leak.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kChunk = 32;      // tokens per pipeline step (two 16-token tiles)
constexpr int kMaxTable = 256;  // block-table entries one partition may span

struct MfmaParams {
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
  int H, H_kv, G, chunks, max_blocks, P, NP;
  float scale_log2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 4 OCP E4M3FN codes -> 4 bf16 (2 dwords).  Every E4M3 value is a bf16 value,
// so the conversion is exact.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Orders this wave's LDS accesses: the V tile is written and then read back
// by other lanes of the same wave (and rewritten by the next chunk), and the
// waves of a workgroup run different numbers of chunks, so a workgroup
// barrier cannot be used inside the loop.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <typename CT, int D>
struct Geometry {
  using CS = typename CT::storage;
  static constexpr int ELEM = (int)sizeof(CS);
  static constexpr int DQ = D / 4;              // d elements per lane per K row
  static constexpr int NKC = D / 32;            // k-steps of the score MFMA
  static constexpr int NMD = D / 16;            // 16-wide d tiles of the output
  static constexpr int KV4 = DQ * ELEM / 16;    // uint4 per lane per K tile
  static constexpr int PR = D * ELEM / 16;      // 16-byte pieces per V row
  static constexpr int RPI = 64 / PR;           // V rows per wave load
  static constexpr int VI = kChunk / RPI;       // V wave loads per chunk
  static constexpr int VS = D + 16;             // LDS V row stride (bf16), padded
};

// Registers that carry one chunk from HBM to the products.  K and V have one
// buffer each: within an iteration the V tile of chunk i goes to LDS before
// the V loads of chunk i+NW are issued into the same registers, and the K
// rows of chunk i feed the score products before the K loads of chunk i+NW
// are issued, so both loads are in flight while chunk i finishes.
template <typename CT, int D>
struct KStage {
  using Gm = Geometry<CT, D>;
  uint4 k[2][Gm::KV4];
  float ksc[2], vsc[2];  // FP8 scales of the lane's two 4-token groups
};

template <typename CT, int D>
struct VStage {
  uint4 v[Geometry<CT, D>::VI];
};

template <typename CT, int D>
__device__ __forceinline__ void keep_live(const VStage<CT, D>& vs, const KStage<CT, D>& ks) {
#pragma unroll
  for (int j = 0; j < Geometry<CT, D>::VI; ++j)
    asm volatile("" ::"v"(vs.v[j].x), "v"(vs.v[j].y), "v"(vs.v[j].z), "v"(vs.v[j].w));
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int i = 0; i < Geometry<CT, D>::KV4; ++i)
      asm volatile("" ::"v"(ks.k[T][i].x), "v"(ks.k[T][i].y), "v"(ks.k[T][i].z),
                   "v"(ks.k[T][i].w));
}

template <int BS>
__device__ __forceinline__ size_t row_index(const int* s_tab, int t, int first_blk, int H_kv,
                                            int kvh) {
  const int phys = s_tab[t / BS - first_blk];
  return ((size_t)phys * H_kv + kvh) * BS + (t % BS);
}

template <typename CT, int D, int BS>
__device__ __forceinline__ void load_k(KStage<CT, D>& st, const MfmaParams& p, int c0, int end,
                                       int first_blk, const int* s_tab, int kvh, int lane) {
  using Gm = Geometry<CT, D>;
  using CS = typename CT::storage;
  const int q = lane >> 4, r = lane & 15;
  const CS* kc = reinterpret_cast<const CS*>(p.kc);
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int t = min(c0 + 16 * T + r, end - 1);  // clamped: masked later
    const size_t row = row_index<BS>(s_tab, t, first_blk, p.H_kv, kvh);
    const uint4* src = reinterpret_cast<const uint4*>(kc + row * D + Gm::DQ * q);
#pragma unroll
    for (int i = 0; i < Gm::KV4; ++i) st.k[T][i] = src[i];
    if constexpr (Gm::ELEM == 1) {
      const int ts = min(c0 + 16 * T + 4 * q, end - 1);
      const size_t si = (size_t)s_tab[ts / BS - first_blk] * p.H_kv + kvh;
      st.ksc[T] = p.ks[si];
      st.vsc[T] = p.vs[si];
    }
  }
}

template <typename CT, int D, int BS>
__device__ __forceinline__ void load_v(VStage<CT, D>& st, const MfmaParams& p, int c0, int end,
                                       int first_blk, const int* s_tab, int kvh, int lane) {
  using Gm = Geometry<CT, D>;
  using CS = typename CT::storage;
  const CS* vc = reinterpret_cast<const CS*>(p.vc);
#pragma unroll
  for (int j = 0; j < Gm::VI; ++j) {
    const int t = min(c0 + j * Gm::RPI + lane / Gm::PR, end - 1);
    const size_t row = row_index<BS>(s_tab, t, first_blk, p.H_kv, kvh);
    st.v[j] = reinterpret_cast<const uint4*>(vc + row * D)[lane % Gm::PR];
  }
}

// V rows of one chunk -> this wave's LDS tile as bf16 (rows past the end as
// zeros).
template <typename CT, int D>
__device__ __forceinline__ void store_v(const VStage<CT, D>& st, int c0, int end, uint16_t* s_v,
                                        int lane) {
  using Gm = Geometry<CT, D>;
  const bool full = c0 + kChunk <= end;
  wave_lds_sync();  // the previous chunk's transpose reads are done
#pragma unroll
  for (int j = 0; j < Gm::VI; ++j) {
    const int row = j * Gm::RPI + lane / Gm::PR;
    const int piece = lane % Gm::PR;
    uint4 v = st.v[j];
    if (!full) {  // uniform: only the last chunk of a partition is ragged
      const bool ok = c0 + row < end;
      v.x = ok ? v.x : 0u;
      v.y = ok ? v.y : 0u;
      v.z = ok ? v.z : 0u;
      v.w = ok ? v.w : 0u;
    }
    if constexpr (Gm::ELEM == 2) {
      *reinterpret_cast<uint4*>(s_v + row * Gm::VS + piece * 8) = v;
    } else {
      const uint2 a = fp8x4_to_bf16x4(v.x), b = fp8x4_to_bf16x4(v.y);
      const uint2 c = fp8x4_to_bf16x4(v.z), d = fp8x4_to_bf16x4(v.w);
      uint4* dst = reinterpret_cast<uint4*>(s_v + row * Gm::VS + piece * 16);
      dst[0] = make_uint4(a.x, a.y, b.x, b.y);
      dst[1] = make_uint4(c.x, c.y, d.x, d.y);
    }
  }
  wave_lds_sync();  // the tile is visible to every lane of the wave
}

// Scores S^T = K . Q^T of both 16-token tiles: lane (q, r) gets head r,
// tokens 16 T + 4 q + i.
template <typename CT, int D>
__device__ __forceinline__ void scores(const KStage<CT, D>& st,
                                       const bf16x8_t (&qf)[Geometry<CT, D>::NKC],
                                       f32x4_t (&s)[2]) {
  using Gm = Geometry<CT, D>;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    s[T] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Gm::NKC; ++c) {
      bf16x8_t a;
      if constexpr (Gm::ELEM == 2) {
        a = as_bf16x8(st.k[T][c]);  // bytes 16c..16c+15 of the lane's row slice
      } else {
        const uint4 w = st.k[T][c / 2];  // bytes 8c..8c+7 of the lane's 32-byte slice
        const uint32_t w0 = (c & 1) ? w.z : w.x;
        const uint32_t w1 = (c & 1) ? w.w : w.y;
        const uint2 lo = fp8x4_to_bf16x4(w0), hi = fp8x4_to_bf16x4(w1);
        a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
      s[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], s[T], 0, 0, 0);
    }
  }
}

// Online softmax update with this chunk's scores, then O^T += V^T . P^T.
template <int D>
__device__ __forceinline__ void softmax_pv(const f32x4_t (&s)[2], const float (&fk)[2],
                                           const float (&fv)[2], bool scaled_v, int c0, int end,
                                           const uint16_t* s_v, f32x4_t (&acc)[D / 16], float& m,
                                           float& lsum, int lane) {
  constexpr int VS = D + 16;
  const int q = lane >> 4, r = lane & 15;
  const bool full = c0 + kChunk <= end;
  float x[2][4];
  float mc = kNegInf;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = full || (c0 + 16 * T + 4 * q + i < end);
      x[T][i] = ok ? s[T][i] * fk[T] : kNegInf;
      mc = fmaxf(mc, x[T][i]);
    }
  }
  mc = fmaxf(mc, __shfl_xor(mc, 16));
  mc = fmaxf(mc, __shfl_xor(mc, 32));
  const float m_new = fmaxf(m, mc);  // finite: the chunk holds >= 1 valid token
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  m = m_new;

  float pv[2][4];
  float ps = 0.f;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(x[T][i] - m_new);
      ps += e;
      pv[T][i] = scaled_v ? e * fv[T] : e;
    }
  }
  lsum = fmaf(lsum, alpha, ps);
#pragma unroll
  for (int md = 0; md < D / 16; ++md) acc[md] *= alpha;

  // P^T operand: tokens 4q..4q+3 then 16+4q..16+4q+3 of this chunk.
  const bf16x8_t pb = as_bf16x8(make_uint4(pack_bf16x2(pv[0][0], pv[0][1]),
                                           pack_bf16x2(pv[0][2], pv[0][3]),
                                           pack_bf16x2(pv[1][0], pv[1][1]),
                                           pack_bf16x2(pv[1][2], pv[1][3])));
  const int trow = 4 * q + (r >> 2);
  const int tcol = 4 * (r & 3);
#pragma unroll
  for (int md = 0; md < D / 16; ++md) {
    const uint16_t* p0 = s_v + trow * VS + 16 * md + tcol;
    const uint16_t* p1 = p0 + 16 * VS;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    const bf16x8_t a = as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
    acc[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[md], 0, 0, 0);
  }
}

template <typename CT, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(MfmaParams p) {
  using Gm = Geometry<CT, D>;
  constexpr int VTILE = kChunk * Gm::VS;        // bf16 elements per wave
  constexpr int MERGE = NW * 16 * D;            // fp32 partial outputs
  constexpr int UNION_BYTES = (VTILE * NW * 2 > MERGE * 4) ? VTILE * NW * 2 : MERGE * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[UNION_BYTES];
  __shared__ int s_tab[kMaxTable];
  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];

  const int part = blockIdx.x;
  const int hc = blockIdx.y % p.chunks;
  const int kvh = blockIdx.y / p.chunks;
  const int seq = blockIdx.z;
  const int n = p.lens[seq];
  const int start = part * p.P;
  if (part > 0 && start >= n) return;
  const int end = min(n, start + p.P);
  const int h0 = kvh * p.G + hc * 16;
  const int nh = min(16, p.G - hc * 16);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;

  // Block ids of this partition, fetched once.
  const int first_blk = start / BS;
  const int nblk = end > start ? (end - 1) / BS - first_blk + 1 : 0;
  const int32_t* trow = p.tables + (size_t)seq * p.max_blocks + first_blk;
  for (int i = tid; i < nblk; i += NW * 64) s_tab[i] = trow[i];

  // Q operand: lane (q, r) holds head r, elements (D/4) q + 8 c .. + 8.
  bf16x8_t qf[Gm::NKC];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(p.q) + ((size_t)seq * p.H + h0 + min(r, nh - 1)) * D +
        Gm::DQ * q);
    const bool live = r < nh;
#pragma unroll
    for (int c = 0; c < Gm::NKC; ++c) {
      uint4 v = qp[c];
      v.x = live ? v.x : 0u;
      v.y = live ? v.y : 0u;
      v.z = live ? v.z : 0u;
      v.w = live ? v.w : 0u;
      qf[c] = as_bf16x8(v);
    }
  }
  __syncthreads();

  f32x4_t acc[Gm::NMD];
#pragma unroll
  for (int md = 0; md < Gm::NMD; ++md) acc[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  uint16_t* s_v = reinterpret_cast<uint16_t*>(s_raw) + wave * VTILE;
  const int nch = (end - start + kChunk - 1) / kChunk;
  int ci = wave;
  if (ci < nch) {
    KStage<CT, D> ks;
    VStage<CT, D> vs;
    load_v<CT, D, BS>(vs, p, start + ci * kChunk, end, first_blk, s_tab, kvh, lane);
    load_k<CT, D, BS>(ks, p, start + ci * kChunk, end, first_blk, s_tab, kvh, lane);
    while (true) {
      const int c0 = start + ci * kChunk;
      // The next chunk index is clamped so that every load is unconditional
      // (a redundant last prefetch hits the cache).
      const int cn = start + min(ci + NW, nch - 1) * kChunk;
      store_v<CT, D>(vs, c0, end, s_v, lane);
      load_v<CT, D, BS>(vs, p, cn, end, first_blk, s_tab, kvh, lane);
      f32x4_t sc[2];
      scores<CT, D>(ks, qf, sc);
      float fk[2], fv[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        fk[T] = p.scale_log2;
        fv[T] = 1.f;
        if constexpr (Gm::ELEM == 1) {
          fk[T] *= ks.ksc[T];
          fv[T] = ks.vsc[T];
        }
      }
      load_k<CT, D, BS>(ks, p, cn, end, first_blk, s_tab, kvh, lane);
      softmax_pv<D>(sc, fk, fv, Gm::ELEM == 1, c0, end, s_v, acc, m, lsum, lane);
      ci += NW;
      if (ci >= nch) break;
    }
    // The last prefetch is dead on the exit path; this use keeps the compiler
    // from sinking the prefetch loads into the next iteration, which would
    // serialise every load with its use.
    keep_live(vs, ks);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // Merge the NW wave-level softmax states of this partition.
  __syncthreads();  // every wave is done with its V tile (s_raw is reused)
  float* s_acc = reinterpret_cast<float*>(s_raw);
  if (q == 0) {
    s_m[wave][r] = m;
    s_l[wave][r] = lsum;
  }
#pragma unroll
  for (int md = 0; md < Gm::NMD; ++md)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[(wave * 16 + r) * D + 16 * md + 4 * q + i] = acc[md][i];
  __syncthreads();

  const bool single = n <= p.P;
  for (int idx = tid; idx < nh * D; idx += NW * 64) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(s_m[w][g] - M);
        L = fmaf(s_l[w][g], wt, L);
        O = fmaf(s_acc[(w * 16 + g) * D + d], wt, O);
      }
    }
    const int h = h0 + g;
    if (single) {
      const float o = L > 0.f ? O / L : 0.f;
      reinterpret_cast<uint16_t*>(p.out)[((size_t)seq * p.H + h) * D + d] = f32_to_bf16(o);
    } else {
      const size_t pi = ((size_t)seq * p.H + h) * p.NP + part;
      p.ws_acc[pi * D + d] = O;
      if (d == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = L;
      }
    }
  }
}

template <typename CT, int D, int BS>
hipError_t launch_bs(const DecodeArgs& a) {
  constexpr int NW = 4;
  MfmaParams p;
  p.q = a.q; p.kc = a.key_cache; p.vc = a.value_cache; p.ks = a.key_scale; p.vs = a.value_scale;
  p.tables = a.tables; p.lens = a.lens; p.out = a.out;
  p.ws_m = a.ws_m; p.ws_l = a.ws_l; p.ws_acc = a.ws_acc;
  p.H = a.H; p.H_kv = a.H_kv; p.G = a.H / a.H_kv; p.chunks = (p.G + 15) / 16;
  p.max_blocks = a.max_blocks; p.P = a.P; p.NP = a.NP;
  p.scale_log2 = a.scale * kLog2e;
  dim3 grid(a.NP, a.H_kv * p.chunks, a.S);
  hipLaunchKernelGGL((decode_mfma_kernel<CT, D, BS, NW>), grid, dim3(NW * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <typename CT, int D>
hipError_t launch_d(const DecodeArgs& a) {
  switch (a.bs) {
    case 8: return launch_bs<CT, D, 8>(a);
    case 16: return launch_bs<CT, D, 16>(a);
    default: return launch_bs<CT, D, 32>(a);
  }
}

template <typename CT>
hipError_t launch_c(const DecodeArgs& a) {
  return a.D == 64 ? launch_d<CT, 64>(a) : launch_d<CT, 128>(a);
}

}  // namespace

// Grouped heads (G >= 2) with bf16 queries run here; one head per KV head
// keeps the vector-ALU kernel, which needs fewer registers for the same bytes.
bool decode_mfma_supported(const DecodeArgs& a) {
  return a.q_dtype == PKV_BF16 && (a.cache_dtype == PKV_BF16 || a.cache_dtype == PKV_FP8_E4M3) &&
         a.H / a.H_kv >= 2 && (a.P + a.bs - 1) / a.bs <= kMaxTable;
}

hipError_t launch_decode_mfma(const DecodeArgs& a) {
  if (a.cache_dtype == PKV_BF16) return launch_c<BF16>(a);
  return launch_c<FP8>(a);
}

}  // namespace pkv
