// Multi-token paged attention for long prefill chunks on gfx950 matrix cores.
//
// Each query token of a chunk is a decode step over the positions up to its
// own (PagedAttention article on dpshk.com, section 2.2, applied per token;
// new requests join the running batch and their prompts attend over the same
// paged cache: page "PagedAttention 与连续批处理…", continuous-batching
// section).  With many tokens per sequence the work is a dense contraction,
// so this kernel is built for the matrix cores rather than for HBM:
//
//   * rows of a KV head are the (token, head) pairs m * G + g of its G query
//     heads; a workgroup owns a tile of 128 rows, each of its 4 waves 32 rows
//     (two 16-row MFMA groups that share every K and V fragment read; or, by
//     kGroups, 8 waves of 16 rows);
//   * the workgroup walks its keys in chunks of 64: K and V rows are gathered
//     through the block table straight into LDS by loads to LDS (no register
//     staging), double-buffered so chunk c+1 streams in while chunk c is
//     multiplied;
//   * S^T = K . Q^T and O^T += V^T . P^T on v_mfma_f32_16x16x32_bf16, with
//     the online softmax between them in registers (the decode kernel's
//     formulation: a lane holds one row, so row reductions are two swizzles);
//   * LDS rows are XOR-swizzled (K in 16-byte pieces, V in 32-byte halves of
//     them) so the K fragment reads (ds_read_b128) and the V transposed reads
//     (ds_read_b64_tr_b16) are free of bank conflicts without padding, which
//     the DMA cannot insert;
//   * row sums come from the matrix cores (an all-ones tile times P^T), and
//     the accumulators are rescaled only when a row maximum grows by more
//     than 2^8 (tested on each lane's own maximum; the row maximum crosses
//     lanes with the gfx950 permlane swaps only then);
//   * FP8 caches are first dequantised to a bf16 pool (stage_fp8_kernel).
//
// A tile needs only the keys below its last row's position; rows of earlier
// tokens mask the newest keys of the last chunks.  Long contexts may be split
// into partitions whose partials (running max in base-2 units, sum, and
// unnormalised output) the split reduce merges per (token, head); a
// sequence that fits one partition is finished here.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_v;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_v;
typedef __attribute__((address_space(3))) i16x4_v lds_i16x4_v;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBM = 128;        // rows per workgroup tile
// 16-row MFMA groups per wave: 2 (4 waves of 32 rows, every K and V fragment
// read shared by both groups) or 1 (8 waves of 16 rows: half the registers,
// so twice the waves per SIMD to cover each wave's dependent chain).
constexpr int kGroups = 2;
template <int NG>
struct Waves { static constexpr int N = kBM / (16 * NG); };
constexpr int kKC = 64;         // keys per LDS chunk
constexpr float kMaxInit = -1e30f;  // running max before any key (finite: no inf - inf)

struct PrefillParams {
  const uint16_t* q;   // [S][M][H][D] bf16
  uint16_t* out;       // [S][M][H][D] bf16
  const uint16_t* kc;  // [num_blocks][H_kv][BS][D] bf16
  const uint16_t* vc;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_m;  // [S][M][H][NP] when NP > 1
  float* ws_l;
  float* ws_acc;  // [S][M][H][NP][D]
  int M, H, H_kv, G, max_blocks, P, NP;
  int max_ctx;  // longest context the grid covers; longer lengths are cut to it
  int RT;       // row tiles per KV head: ceil(M * G / kBM)
  int total;    // workgroups with work: S * H_kv * NP * RT
  int per_xcd;  // ceil(total / 8)
  float scale_log2;
};

struct StageParams {
  const uint8_t* kc;  // [num_blocks][H_kv][bs][D] E4M3FN codes
  const uint8_t* vc;
  const float* ks;    // [num_blocks][H_kv]
  const float* vs;
  const int32_t* tables;
  const int32_t* lens;
  uint16_t* sk;       // [S * nb][H_kv][bs][D] bf16 pool
  uint16_t* sv;
  int32_t* staged_tab;  // [S][nb]
  int H_kv, D, bs, max_blocks, max_ctx, nb;
};

__device__ __forceinline__ bf16x8_v to_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_v, v); }

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// s_waitcnt with vmcnt(N) and lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8), then a workgroup barrier.  The compiler
// barriers keep memory operations on their side; no fence is used, because a
// workgroup release fence waits for every LDS DMA in flight, the next
// chunk's included.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 32-bit LDS address of a shared-memory object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}

// Inside the chunk loop every LDS read is inline assembly that ends with its
// own wait.  The compiler cannot tell which LDS bytes a DMA in flight will
// write, so before any LDS read it can see it would wait for all of them,
// the next chunk's included, and the copy would no longer overlap the
// products.  The chunk data itself is ordered by the explicit waits and
// barriers of wait_vm_barrier.

// NKC 16-byte K fragment reads at the lane's addresses + OFF.
template <int OFF>
__device__ __forceinline__ void lds_read_k(uint4 (&a)[4], const uint32_t (&ad)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n"
      "ds_read_b128 %1, %5 offset:%8\n"
      "ds_read_b128 %2, %6 offset:%8\n"
      "ds_read_b128 %3, %7 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read_k(uint4 (&a)[2], const uint32_t (&ad)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n"
      "ds_read_b128 %1, %3 offset:%4\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1])
      : "v"(ad[0]), "v"(ad[1]), "i"(OFF));
}

// Block ids of a chunk's DMA rounds from the LDS table slice.
__device__ __forceinline__ void lds_read_tab(int (&v)[4], const uint32_t (&ad)[4]) {
  asm volatile(
      "ds_read_b32 %0, %4\n"
      "ds_read_b32 %1, %5\n"
      "ds_read_b32 %2, %6\n"
      "ds_read_b32 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
}
__device__ __forceinline__ void lds_read_tab(int (&v)[1], const uint32_t (&ad)[1]) {
  asm volatile(
      "ds_read_b32 %0, %1\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0])
      : "v"(ad[0]));
}
__device__ __forceinline__ void lds_read_tab(int (&v)[2], const uint32_t (&ad)[2]) {
  asm volatile(
      "ds_read_b32 %0, %2\n"
      "ds_read_b32 %1, %3\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1])
      : "v"(ad[0]), "v"(ad[1]));
}

// Eight transposing reads (ds_read_b64_tr_b16) for two 16-wide d tiles: at
// each of the lane's two addresses + OFF + {0, 1, 2, 3} * STEP, the 16-key
// quarters of a 64-key chunk.
template <int OFF, int STEP>
__device__ __forceinline__ void lds_read_v(uint2 (&v)[8], uint32_t ad0, uint32_t ad1) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%10\n"
      "ds_read_b64_tr_b16 %1, %8 offset:%11\n"
      "ds_read_b64_tr_b16 %2, %8 offset:%12\n"
      "ds_read_b64_tr_b16 %3, %8 offset:%13\n"
      "ds_read_b64_tr_b16 %4, %9 offset:%10\n"
      "ds_read_b64_tr_b16 %5, %9 offset:%11\n"
      "ds_read_b64_tr_b16 %6, %9 offset:%12\n"
      "ds_read_b64_tr_b16 %7, %9 offset:%13\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(ad0), "v"(ad1), "i"(OFF), "i"(OFF + STEP), "i"(OFF + 2 * STEP), "i"(OFF + 3 * STEP));
}

// v_max_f32 without the canonicalising moves fmaxf adds around lane swaps.
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Maximum over the four lanes of a row (l, l^16, l^32, l^48) with the gfx950
// lane swaps (no LDS round trip).
__device__ __forceinline__ float max4_rows(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2f(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// v_max3_f32 (the compiler does not form it from fmaxf).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int D, int NG>
struct Layout {
  static constexpr int NW = Waves<NG>::N;           // waves per workgroup
  static constexpr int PR = D / 8;                  // 16-byte pieces per row
  static constexpr int RB = 256 / (2 * D);          // rows per 256 bytes
  static constexpr int ROW = 2 * D;                 // bytes per row
  static constexpr int TILE = kKC * ROW;            // bytes of a K or V chunk
  static constexpr int CHUNK = 2 * TILE;            // K tile then V tile
  static constexpr int ROUNDS = kKC * PR / (64 * NW);  // DMA rounds per wave and chunk
  static constexpr int RPI = 64 / PR;               // rows per wave DMA instruction
  static constexpr int NKC = D / 32;                // k-steps of the score products
  static constexpr int NMD = D / 16;                // 16-wide d tiles of O^T
  // Physical 16-byte piece of logical piece p in row k: XOR with bits of the
  // row index, so the K fragment reads (ds_read_b128, lane (q4, r) reading
  // row r, logical piece (D/32) q4 + c) meet no bank conflicts.  The row's
  // bit 2 is also folded into bit 3: with the row XORed in unchanged, a
  // probe of exactly this read pattern took 8 LDS cycles per instruction on
  // gfx950 (half of them counted as bank conflicts), with this swizzle 4, the
  // cost of a conflict-free 1 KiB read (D = 128 and 64).  Rows k, k + 16 and
  // k + 32 share the pattern.
  __device__ static __forceinline__ int swz(int k) {
    const int s = (k ^ ((k & 4) << 1)) & 15;
    return (s / RB) & (PR - 1);
  }
  __device__ static __forceinline__ int phys(int k, int p) { return p ^ swz(k); }
  // V tile: XOR of the 32-byte half-piece index, so the 4 rows of a
  // transposed read group (and 8 consecutive rows) sit in distinct banks.
  __device__ static __forceinline__ int vswz(int k) { return 2 * ((k / RB) & (PR / 2 - 1)); }
};

// Buffer descriptor of one cache block's (KV head) tile: base, no stride,
// records up to 2^31 bytes (a tile is at most 8 KiB), and the gfx9 word 3
// (raw buffer: 32-bit data, no format conversion).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

// Gathers keys c0 .. c0 + kKC - 1 of KV head kvh into buffer `buf` (K and V
// tiles).  Wave w of NW, round i fills bytes [(NW i + w) KiB, +1 KiB) of each
// tile, lane l the physical piece 64 (NW i + w) + l, and fetches the logical piece
// that the swizzle stores there.  One round covers RPI <= 8 rows of one
// cache block, so its block id is one table entry.  Keys at or past kend
// are read as key kend - 1 (a real row of the same block; masked later).
template <int D, int BS, int NG>
__device__ __forceinline__ void issue_chunk(char* buf, const PrefillParams& p, uint32_t tab,
                                            int elast, int kvh, int start, int c0, int kend,
                                            int wave, int lane,
                                            const uint32_t (&koff)[Layout<D, NG>::ROUNDS],
                                            const uint32_t (&voff)[Layout<D, NG>::ROUNDS]) {
  using L = Layout<D, NG>;
  int blk[L::ROUNDS];
  uint32_t ta[L::ROUNDS];
  const int cidx = (c0 - start) / BS;
#pragma unroll
  for (int i = 0; i < L::ROUNDS; ++i)
    ta[i] = tab + 4 * min(cidx + (L::RPI * (i * L::NW + wave)) / BS, elast);
  lds_read_tab(blk, ta);
  if (c0 + kKC <= kend) {
    // Whole chunk below kend: a uniform row base per round plus the lane's
    // fixed byte offset (c0 is a multiple of the block size).
#pragma unroll
    for (int i = 0; i < L::ROUNDS; ++i) {
      const int b = __builtin_amdgcn_readfirstlane(blk[i]);
      const size_t rb = ((size_t)b * p.H_kv + kvh) * (size_t)(BS * D * 2);
      const char* kb = reinterpret_cast<const char*>(p.kc) + rb;
      const char* vb = reinterpret_cast<const char*>(p.vc) + rb;
      const int lds = (i * L::NW + wave) * 1024;
      // Buffer loads: the block's base in a scalar descriptor, the lane's
      // 32-bit offset as is (no 64-bit vector address arithmetic).
      __builtin_amdgcn_raw_ptr_buffer_load_lds(block_rsrc(kb), (lds_void*)(buf + lds), 16, koff[i],
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(block_rsrc(vb), (lds_void*)(buf + L::TILE + lds), 16,
                                               voff[i], 0, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < L::ROUNDS; ++i) {
    const int k = L::RPI * (i * L::NW + wave) + lane / L::PR;
    const int pp = lane % L::PR;
    const int t = min(c0 + k, kend - 1);
    const size_t row = ((size_t)blk[i] * p.H_kv + kvh) * BS + (t % BS);
    const size_t offk = row * D + 8 * (pp ^ L::swz(k));  // XOR is its own inverse
    const size_t offv = row * D + 8 * (pp ^ L::vswz(k));
    const int lds = (i * L::NW + wave) * 1024;
    __builtin_amdgcn_global_load_lds(p.kc + offk, (lds_void*)(buf + lds), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(p.vc + offv, (lds_void*)(buf + L::TILE + lds), 16, 0, 0);
  }
}

// One chunk from buffer SEL: scores of both row groups, online softmax,
// O^T update.  kad: the lane's K fragment addresses in buffer 0 (key r,
// logical pieces (D/32) q4 + c); vad: the lane's V address in buffer 0 for
// d tile 0, XORed with 32 md for tile md.  e[j]: keys below it are visible
// to this lane's row of group j; full[j] (uniform): no mask for group j.
template <int D, int NG, int SEL>
__device__ __forceinline__ void compute_chunk(const uint32_t (&kad)[D / 32], uint32_t vad,
                                              const uint4 (&qf)[NG][D / 32],
                                              f32x4_v (&acc)[NG][D / 16], float (&m)[NG],
                                              f32x4_v (&lacc)[NG], const int (&e)[NG],
                                              const bool (&full)[NG], int c0, float sl,
                                              int lane) {
  using L = Layout<D, NG>;
  constexpr int KOFF = SEL * L::CHUNK;
  const int q4 = lane >> 4;
  f32x4_v s[NG][4];
  // S^T = K . Q^T, 16 keys per tile T: lane (q4, r) holds key 16 T + r,
  // contraction elements (D/4) q4 + 8 c .. + 7 (the Q fragments use the same
  // order).  The swizzle of row 16 T + r does not depend on T.
#define PKV_SCORE_TILE(T)                                                                     \
  {                                                                                           \
    uint4 a[L::NKC];                                                                          \
    lds_read_k<KOFF + (T) * 16 * L::ROW>(a, kad);                                             \
    _Pragma("unroll") for (int j = 0; j < NG; ++j) s[j][T] = f32x4_v{0.f, 0.f, 0.f, 0.f};    \
    _Pragma("unroll") for (int c = 0; c < L::NKC; ++c) {                                      \
      _Pragma("unroll") for (int j = 0; j < NG; ++j) s[j][T] =                                \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(a[c]), to_bf16x8(qf[j][c]),       \
                                                  s[j][T], 0, 0, 0);                          \
    }                                                                                         \
  }
  PKV_SCORE_TILE(0)
  PKV_SCORE_TILE(1)
  PKV_SCORE_TILE(2)
  PKV_SCORE_TILE(3)
#undef PKV_SCORE_TILE
  // Online softmax per group: lane (q4, r) holds row r, keys 16 T + 4 q4 + i
  // (scores in raw units; sl > 0 turns them into base-2 logits).  The
  // running maximum m moves only when a row's chunk maximum exceeds it by
  // more than 8 (wave-uniform test), so most chunks skip the rescale of the
  // accumulators; the exponents stay below 2^8, and acc and l always share
  // one reference, so the normalised result is unchanged.
  uint4 pb[NG][2];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    float mt;  // the lane's maximum over its 16 keys, raw units
    if (!full[j]) {
      const int rel = e[j] - c0 - 4 * q4;  // keys 16 T + i below it are visible
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(16 * T + i < rel)) s[j][T][i] = kNegInf;
    }
    {
      float t0 = max3f(s[j][0][0], s[j][0][1], s[j][0][2]);
      float t1 = max3f(s[j][0][3], s[j][1][0], s[j][1][1]);
      float t2 = max3f(s[j][1][2], s[j][1][3], s[j][2][0]);
      float t3 = max3f(s[j][2][1], s[j][2][2], s[j][2][3]);
      float t4 = max3f(s[j][3][0], s[j][3][1], s[j][3][2]);
      t0 = max3f(t0, t1, t2);
      t3 = max3f(t3, t4, s[j][3][3]);
      mt = max2f(t0, t3);
    }
    // A row's maximum passes m + 8 only where one of its four lanes' does
    // (the factor is positive and rounding is monotonic), so the row
    // maximum across lanes is needed only on a rescale.
    if (__any(mt * sl > m[j] + 8.f)) {
      const float m_new = fmaxf(m[j], max4_rows(mt) * sl);
      const float alpha = __builtin_amdgcn_exp2f(m[j] - m_new);
      m[j] = m_new;
      lacc[j] *= alpha;
#pragma unroll
      for (int md = 0; md < L::NMD; ++md) acc[j][md] *= alpha;
    }
    float x[4][4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[T][i] = __builtin_amdgcn_exp2f(fmaf(s[j][T][i], sl, -m[j]));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[j][u] = make_uint4(bf16x2_rne(x[2 * u][0], x[2 * u][1]),
                            bf16x2_rne(x[2 * u][2], x[2 * u][3]),
                            bf16x2_rne(x[2 * u + 1][0], x[2 * u + 1][1]),
                            bf16x2_rne(x[2 * u + 1][2], x[2 * u + 1][3]));
    }
  }
  // O^T += V^T . P^T.  Transposed reads: lane (q4, r) addresses key
  // 32 u + 4 q4 + r / 4 (and + 16) at d = 16 md + 4 (r % 4) and receives
  // V[those 4 keys][16 md + r]; v[4h + 2u] / v[4h + 2u + 1] are the two
  // 16-key halves of 32-key half u for d tile md + h.
  constexpr int VOFF = SEL * L::CHUNK + L::TILE;
  // Row sums: an all-ones 16 x 32 tile times P^T leaves sum_k P[row][k] in
  // every element of the lane's row (the sum of the same bf16 weights the
  // products use).
  const bf16x8_v ones = to_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int j = 0; j < NG; ++j)
      lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, to_bf16x8(pb[j][u]), lacc[j], 0, 0, 0);
#pragma unroll
  for (int md = 0; md < L::NMD; md += 2) {
    uint2 v[8];
    lds_read_v<VOFF, 16 * L::ROW>(v, vad ^ (32u * md), vad ^ (32u * (md + 1)));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint2 lo = v[4 * h + 2 * u], hi = v[4 * h + 2 * u + 1];
        const bf16x8_v va = to_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int j = 0; j < NG; ++j)
          acc[j][md + h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, to_bf16x8(pb[j][u]),
                                                                    acc[j][md + h], 0, 0, 0);
      }
    }
  }
}

template <int D, int BS, int NG>
__global__ __launch_bounds__(Waves<NG>::N * 64, 2) void prefill_mfma_kernel(PrefillParams p) {
  using L = Layout<D, NG>;
  __shared__ int s_tab[kPrefillMaxTable];
  __shared__ __attribute__((aligned(1024))) char s_buf[2 * L::CHUNK];

  // Workgroup b runs on XCD b % 8; each XCD takes a contiguous range of
  // tiles, so the row tiles of one (sequence, KV head, partition) share that
  // XCD's L2.  Within it the tiles of later tokens (more keys) go first.
  const int b = blockIdx.x;
  const int lin = (b & 7) * p.per_xcd + (b >> 3);
  if (lin >= p.total) return;
  const int unit = lin / p.RT;
  const int rt = p.RT - 1 - (lin - unit * p.RT);
  const int part = unit % p.NP;
  const int sk = unit / p.NP;
  const int seq = sk / p.H_kv;
  const int kvh = sk - seq * p.H_kv;

  // wave through readfirstlane: the compiler then keeps it and everything
  // derived from it (row ranges, DMA rounds) in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, r = lane & 15;
  const int n = min(p.lens[seq], p.max_ctx);
  const int MG = p.M * p.G;
  const int r0 = rt * kBM;
  const int rlast = min(r0 + kBM, MG) - 1;
  const int base = n - p.M + 1;  // keys below base + m: visible to token m
  const int start = part * p.P;
  const int pend = min(n, start + p.P);
  const int kend = min(pend, base + rlast / p.G);
  const bool single = n <= p.P;
  const int nch = kend > start ? (kend - start + kKC - 1) / kKC : 0;
  // A context within one partition is finished by partition 0 alone (the
  // split reduce skips it); otherwise a partition no row of the tile sees
  // has nothing to add.
  if (single ? part > 0 : nch == 0) return;

  const int t0 = start / BS;
  const int elast = nch > 0 ? (kend - 1) / BS - t0 : 0;  // last table entry used
  if (nch > 0) {
    const int32_t* trow = p.tables + (size_t)seq * p.max_blocks + t0;
    for (int i = tid; i <= elast; i += L::NW * 64) s_tab[i] = trow[i];
  }

  // This lane's rows (one per group) and their query fragments.
  uint4 qf[NG][L::NKC];
  int e[NG];
  size_t orow[NG];
  bool live[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int rho = r0 + 16 * NG * wave + 16 * j + r;
    live[j] = rho <= rlast;
    const int rc = min(rho, rlast);
    const int m = rc / p.G;
    orow[j] = ((size_t)seq * p.M + m) * p.H + (size_t)kvh * p.G + (rc - m * p.G);
    const uint16_t* qrow = p.q + orow[j] * D + (D / 4) * q4;
#pragma unroll
    for (int c = 0; c < L::NKC; ++c) {
      qf[j][c] = *reinterpret_cast<const uint4*>(qrow + 8 * c);
      if (p.scale_log2 < 0.f) {  // fold the scale's sign into Q (exact)
        qf[j][c].x ^= 0x80008000u; qf[j][c].y ^= 0x80008000u;
        qf[j][c].z ^= 0x80008000u; qf[j][c].w ^= 0x80008000u;
      }
    }
    e[j] = min(pend, base + rc / p.G);
  }
  // Positive factor from raw scores to base-2 logits (a zero scale becomes a
  // tiny positive one: every weight is then 1 up to rounding, as it should).
  const float sl = fmaxf(fabsf(p.scale_log2), 1e-30f);
  // Uniform per group: a group's first row has the smallest end.
  int gfull[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j)
    gfull[j] = min(pend, base + min(r0 + 16 * (NG * wave + j), rlast) / p.G);

  // LDS addresses (buffer 0; buffer 1 and the V tile are immediate offsets).
  const uint32_t buf0 = lds_addr(s_buf);
  const uint32_t tab = lds_addr(s_tab);
  uint32_t kad[L::NKC];
#pragma unroll
  for (int c = 0; c < L::NKC; ++c)
    kad[c] = buf0 + r * L::ROW + 16 * L::phys(r, (D / 32) * q4 + c);
  uint32_t vad;
  {
    const int k0 = 4 * q4 + (r >> 2);
    const int sw = L::vswz(k0);
    // piece (2 md + (r&3)/2) ^ sw = 2 (md ^ (sw/2)) + (r&3)/2: bits 5.. of
    // the address hold md ^ (sw / 2), which the loop XORs with md
    vad = (buf0 + k0 * L::ROW + 8 * (r & 1) + 16 * ((r & 3) >> 1)) | (32u * (sw >> 1));
  }

  // The lane's byte offsets within a block row base for each DMA round.
  uint32_t koff[L::ROUNDS], voff[L::ROUNDS];
#pragma unroll
  for (int i = 0; i < L::ROUNDS; ++i) {
    const int k = L::RPI * (i * L::NW + wave) + lane / L::PR;
    const int pp = lane % L::PR;
    koff[i] = 2u * (uint32_t)((k % BS) * D + 8 * (pp ^ L::swz(k)));
    voff[i] = 2u * (uint32_t)((k % BS) * D + 8 * (pp ^ L::vswz(k)));
  }

  f32x4_v acc[NG][L::NMD];
  float m[NG];
  f32x4_v lacc[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
#pragma unroll
    for (int md = 0; md < L::NMD; ++md) acc[j][md] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    m[j] = kMaxInit;
    lacc[j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }

  __syncthreads();  // the table slice is in LDS
  if (nch > 0)
    issue_chunk<D, BS, NG>(s_buf, p, tab, elast, kvh, start, start, kend, wave, lane, koff, voff);
  for (int ch = 0; ch < nch; ch += 2) {
    {  // even chunk, buffer 0
      const int c0 = start + ch * kKC;
      if (ch + 1 < nch) {
        issue_chunk<D, BS, NG>(s_buf + L::CHUNK, p, tab, elast, kvh, start, c0 + kKC, kend, wave,
                               lane, koff, voff);
        wait_vm_barrier<2 * L::ROUNDS>();
      } else {
        wait_vm_barrier<0>();
      }
      bool full[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) full[j] = c0 + kKC <= gfull[j];
      compute_chunk<D, NG, 0>(kad, vad, qf, acc, m, lacc, e, full, c0, sl, lane);
      wait_vm_barrier<63>();  // every wave is done with buffer 0
    }
    if (ch + 1 < nch) {  // odd chunk, buffer 1
      const int c0 = start + (ch + 1) * kKC;
      if (ch + 2 < nch) {
        issue_chunk<D, BS, NG>(s_buf, p, tab, elast, kvh, start, c0 + kKC, kend, wave, lane, koff,
                               voff);
        wait_vm_barrier<2 * L::ROUNDS>();
      } else {
        wait_vm_barrier<0>();
      }
      bool full[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) full[j] = c0 + kKC <= gfull[j];
      compute_chunk<D, NG, 1>(kad, vad, qf, acc, m, lacc, e, full, c0, sl, lane);
      wait_vm_barrier<63>();  // every wave is done with buffer 1
    }
  }

  // Lane (q4, r) of group j holds O^T[16 md + 4 q4 + i][row r].
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const float l = lacc[j][0];
    if (!live[j]) continue;
    if (single) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* o = p.out + orow[j] * D + 4 * q4;
#pragma unroll
      for (int md = 0; md < L::NMD; ++md) {
        const f32x4_v a = acc[j][md];
        *reinterpret_cast<uint2*>(o + 16 * md) =
            make_uint2(bf16x2_rne(a[0] * inv, a[1] * inv), bf16x2_rne(a[2] * inv, a[3] * inv));
      }
    } else {
      const size_t pi = orow[j] * p.NP + part;
      // bf16 partial outputs, as the decode kernel writes them.
      uint16_t* o = reinterpret_cast<uint16_t*>(p.ws_acc) + pi * D + 4 * q4;
#pragma unroll
      for (int md = 0; md < L::NMD; ++md) {
        typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_v;
        const f32x4_v a = acc[j][md];
        const u32x2_v w = {bf16x2_rne(a[0], a[1]), bf16x2_rne(a[2], a[3])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_v*>(o + 16 * md));
      }
      if (q4 == 0) {
        p.ws_m[pi] = m[j];
        p.ws_l[pi] = l;
      }
    }
  }
}

template <int D, int BS>
hipError_t launch_db(const DecodeArgs& a) {
  PrefillParams p;
  p.q = reinterpret_cast<const uint16_t*>(a.q);
  p.out = reinterpret_cast<uint16_t*>(a.out);
  p.kc = reinterpret_cast<const uint16_t*>(a.key_cache);
  p.vc = reinterpret_cast<const uint16_t*>(a.value_cache);
  p.tables = a.tables;
  p.lens = a.lens;
  p.ws_m = a.ws_m; p.ws_l = a.ws_l; p.ws_acc = a.ws_acc;
  p.M = a.M; p.H = a.H; p.H_kv = a.H_kv; p.G = a.H / a.H_kv;
  p.max_blocks = a.max_blocks; p.P = a.P; p.NP = a.NP; p.max_ctx = a.max_ctx;
  p.RT = (a.M * p.G + kBM - 1) / kBM;
  const long long total = (long long)a.S * a.H_kv * a.NP * p.RT;
  p.total = (int)total;
  p.per_xcd = (int)((total + 7) / 8);
  p.scale_log2 = a.scale * kLog2e;
  const unsigned grid = (unsigned)(8LL * p.per_xcd);
  hipLaunchKernelGGL((prefill_mfma_kernel<D, BS, kGroups>), dim3(grid),
                     dim3(Waves<kGroups>::N * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  switch (a.bs) {
    case 8: return launch_db<D, 8>(a);
    case 16: return launch_db<D, 16>(a);
    case 32: return launch_db<D, 32>(a);
    default: return hipErrorInvalidValue;
  }
}

// FP8 caches on the tiled kernel.  Its K and V rows travel from HBM to LDS
// by DMA, with no register step to decode them in, so a call over an FP8
// cache first dequantises the blocks its sequences reach into a bf16 pool
// (one pool block per (sequence, logical block)) with a table of its own,
// and the tiled kernel runs on that.  Each element becomes the bf16 nearest
// to code * scale[block][KV head] (the dequantisation of the FP8 block
// storage: dpshk.com article, section 3.2), computed in float32.
// Workgroup w stages logical block j = w % nb of sequence w / nb: table
// entry w names pool block w; blocks at or past the sequence's length are
// left unwritten (the tiled kernel reads no position at or past it).
__global__ __launch_bounds__(256) void stage_fp8_kernel(StageParams p) {
  const int w = blockIdx.x;
  const int seq = w / p.nb;
  const int j = w - seq * p.nb;
  if (threadIdx.x == 0) p.staged_tab[w] = w;
  const int n = min(p.lens[seq], p.max_ctx);
  if (j * p.bs >= n) return;
  const int b = p.tables[(size_t)seq * p.max_blocks + j];
  const int per_head = p.bs * p.D;  // codes per (block, KV head), a multiple of 16
  const size_t per_block = (size_t)p.H_kv * per_head;
  const uint4* src[2] = {reinterpret_cast<const uint4*>(p.kc + (size_t)b * per_block),
                         reinterpret_cast<const uint4*>(p.vc + (size_t)b * per_block)};
  uint4* dst[2] = {reinterpret_cast<uint4*>(p.sk + (size_t)w * per_block),
                   reinterpret_cast<uint4*>(p.sv + (size_t)w * per_block)};
  const float* sc[2] = {p.ks + (size_t)b * p.H_kv, p.vs + (size_t)b * p.H_kv};
  const int pieces = (int)(per_block / 16);
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    for (int i = threadIdx.x; i < pieces; i += 256) {
      const uint4 c = src[kv][i];
      const float s = sc[kv][(16 * i) / per_head];
      const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
      uint32_t o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float f0, f1, f2, f3;
        fp8x2_to_f32<false>(cw[e], f0, f1);
        fp8x2_to_f32<true>(cw[e], f2, f3);
        o[2 * e] = bf16x2_rne(f0 * s, f1 * s);
        o[2 * e + 1] = bf16x2_rne(f2 * s, f3 * s);
      }
      dst[kv][2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[kv][2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

}  // namespace

int prefill_tile_rows() { return kBM; }

bool prefill_mfma_supported(const DecodeArgs& a) {
  return a.q_dtype == PKV_BF16 && a.cache_dtype == PKV_BF16 && (a.D == 64 || a.D == 128) &&
         (a.P + a.bs - 1) / a.bs + 1 <= kPrefillMaxTable;
}

hipError_t launch_prefill_mfma(const DecodeArgs& a) {
  if (a.S == 0) return hipSuccess;
  return a.D == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

hipError_t launch_prefill_stage_fp8(const DecodeArgs& a, const PrefillStage& st) {
  if (a.S == 0) return hipSuccess;
  StageParams p;
  p.kc = reinterpret_cast<const uint8_t*>(a.key_cache);
  p.vc = reinterpret_cast<const uint8_t*>(a.value_cache);
  p.ks = a.key_scale; p.vs = a.value_scale;
  p.tables = a.tables; p.lens = a.lens;
  p.sk = reinterpret_cast<uint16_t*>(st.key_pool);
  p.sv = reinterpret_cast<uint16_t*>(st.value_pool);
  p.staged_tab = st.tables;
  p.H_kv = a.H_kv; p.D = a.D; p.bs = a.bs; p.max_blocks = a.max_blocks; p.max_ctx = a.max_ctx;
  p.nb = st.nb;
  const unsigned grid = (unsigned)((long long)a.S * st.nb);
  hipLaunchKernelGGL(stage_fp8_kernel, dim3(grid), dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace pkv
