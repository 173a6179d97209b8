// PagedAttention decode on the matrix cores, for query heads grouped over a
// shared KV head.
//
// What is computed: softmax(q K^T * scale) V over the sequence's context
// (dpshk.com PagedAttention article "企业官网建设流程全解析", section 2.2), K/V
// reached block by block through the block table (page "PagedAttention 与连续
// 批处理…", section "PagedAttention：把显存做成虚拟内存").  ONE softmax over
// the whole context, carried across 32-token chunks with a running maximum
// and sum; partitions of a long context are merged by the reduce kernel.
//
// Work items are (KV head [x chunk of 16 of its query heads], sequence,
// partition).  The grid is persistent (as many workgroups as are resident
// at once): every workgroup first turns the context lengths into
// per-sequence partition offsets (an LDS scan), then takes items from one
// of 8 work queues with an atomic counter, so no workgroup is launched for a
// partition past its sequence's end and uneven items balance dynamically.
// Queue x holds the items congruent to x mod 8 and is served by workgroups
// blockIdx.x = x mod 8, which the hardware places on XCD x; with the KV head
// as the fastest item index each XCD's L2 then serves a fixed set of KV
// heads (blocks shared between sequences come from HBM once per XCD).  The
// last items of the order (about one per workgroup) form a ninth queue that
// every workgroup serves once its own queue is empty, so XCDs that run
// slower than the others do not set the end of the kernel.  The last
// workgroup to finish resets the counters to zero for the next call.
// Items are software-pipelined: the next item is claimed during the current
// one's last step, its block ids and Q are fetched during the merge, and its
// first chunk follows.  A workgroup holds no item in reserve: the workgroups
// on a CU are served by age, so a reserve held by a young one would start
// late and set the kernel's end.
//
// Why MFMA: the query heads that share a KV head turn both products into
// small dense contractions, [16 tokens x D] . [D x 16 heads] for the scores
// and [D x 32 tokens] . [32 tokens x 16 heads] for P V, so every K/V byte
// fetched from HBM feeds up to 16 heads without vector-ALU dot products.
// Heads beyond the group are zero columns.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64; l = 16 q + r):
//   A: lane l holds A[r][8q .. 8q+7]    B: lane l holds B[8q .. 8q+7][r]
//   C: lane l holds C[4q .. 4q+3][r]
// Every lane loads D/4 contiguous elements of ONE token (token r of a
// 16-token tile, elements (D/4) q ..) from both K and V, so one block-table
// lookup per tile addresses both.  The K slice is the A operand of
// S^T = K . Q^T directly: the contraction index d is permuted identically in
// K and Q (d = (D/4) q + 8 c + e at step c), which leaves every dot product
// unchanged.  The result gives each lane ONE head (column r) and four tokens,
// so the running max and sum are per lane.  For P V the lane's eight
// probabilities (tokens 4q..4q+3 of two consecutive tiles) are exactly the B
// operand of O^T = V^T . P^T; V^T fragments come from the V tile staged in
// LDS as bf16 through ds_read_b64_tr_b16, which hands lane i of a 16-lane
// group element (i % 4) of the 8-byte row addressed by lane 4 e + i / 4.
// Tile rows are padded to D + 16 elements (a 288-byte stride for D = 128):
// the 8 rows one transpose read touches then fall on distinct LDS banks, and
// every address stays a per-lane base plus an immediate offset.
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
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kMaxTable = kDecodeMaxTable;  // block-table entries one partition may span
constexpr int kMaxScanSeqs = 512;  // sequences whose offsets a workgroup keeps in LDS
constexpr int kNW = 4;              // waves per workgroup
constexpr int kNT = 2;              // 16-token tiles per pipeline step
// Work-queue counters sit 256 bytes apart: device-scope atomics are resolved
// beyond the per-XCD L2s, and counters sharing a line would serialise there.
constexpr int kCounterStride = 64;
// Initial running maximum: finite, so a step whose tokens are all masked
// leaves (m, l, acc) unchanged instead of producing 2^(-inf - -inf).  Scores
// are far above it for any finite input.
constexpr float kRunMaxInit = -1e30f;

// A step with nothing left to prefetch still issues its loads (branching
// around them would cost registers and waits); they read row 0 of this
// array, one cache line shared by every lane, and the values are never used.
// 256 bytes hold one cache row of D = 128 bf16 elements and one scale.
__device__ __attribute__((aligned(256))) unsigned char g_dummy_row[256];

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
  int* arrivals;  // [S][Y] arrivals of a row group's partitions (fused merge)
  int fused;      // the last partition of a row group to arrive merges its partials
  int* sched;  // claim counter of queue x at [x * kCounterStride], of the shared
               // queue at [8 * kCounterStride], finished-workgroup counter at
               // [9 * kCounterStride]
  int S, H, H_kv, G, chunks, max_blocks, P, NP;
  int M;  // query tokens per sequence (1 for decode)
  int max_ctx;    // longest context the launch covers; longer lengths are cut to it
  int tab_off;    // table entry of the launch's position 0 (len_off / bs)
  // Split attention over a shared prefix (zero / plain values otherwise):
  int len_off;        // positions below it are not this launch's: n = lens - len_off
  int prefix;         // > 0: the launch also holds the prefix's items, first
  int pre_items;      // items over the prefix: H_kv x pre_chunks x pre_slots
  int pre_chunks;     // 16-row chunks of the prefix's rows, the S x G (sequence, head) pairs
  int pre_slots;      // partial slots of the prefix (its partitions), slots 0 .. of a row
  int slot_off;       // partial slot of partition 0 (of the positions after the prefix)
  int np_stride;      // partial slots per row
  int force_partial;  // write partials even when a context fits one partition
  int young_from;  // first workgroup that runs only its first item
  int group_major;  // each per-XCD queue takes whole (sequence, partition) groups
  float scale_log2;
  // Write fused into a decode (kModeDecodeWrite): sequence s's new K and V
  // rows ([S][H_kv][D], the cache's element type) go to slot slots[s] (none
  // outside [0, num_slots)), the slot of its position lens[s] - 1.  (Last,
  // so the other kinds' argument offsets do not move.)
  const void* new_k;
  const void* new_v;
  const int32_t* slots;
  int num_slots;  // slots of the pool: a slot at or past it (or negative) is not written
};

// Item kinds of a launch: one query token per sequence; several causal
// tokens per sequence; or a prefix whose blocks every table shares read once
// for all sequences, with one token per sequence over the positions after
// it.  That last kind holds two sorts of items: the prefix's, whose rows are
// the (sequence, head) pairs of all sequences of a KV head (each masked at
// its sequence's length), first, then each sequence's own positions; both
// leave partials that the split reduce merges.  The split parameters are
// read only by that kind, so the others keep their scalar registers.
enum : int { kModeDecode = 0, kModeCausal = 1, kModeSplitPrefix = 3, kModeDecodeWrite = 4 };

template <int MODE>
constexpr bool kSplit = MODE == kModeSplitPrefix;

// Context length the launch sees for sequence i.
// A length above the launch's bound (a broken caller contract) is cut to
// it, so no item, partial slot or table entry lies past what the grid and
// workspace were sized for.
template <int MODE>
__device__ __forceinline__ int seq_len(const MfmaParams& p, int i) {
  if constexpr (MODE == kModeSplitPrefix) return min(max(0, p.lens[i] - p.len_off), p.max_ctx);
  return min(p.lens[i], p.max_ctx);
}

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
  static constexpr int DQ = D / 4;            // elements per lane per token row
  static constexpr int NKC = D / 32;          // k-steps of the score MFMA
  static constexpr int NMD = D / 16;          // 16-wide d tiles of the output
  static constexpr int KV4 = DQ * ELEM / 16;  // uint4 per lane per tile (K, and V)
  static constexpr int CHUNK = 16 * kNT;      // tokens per pipeline step
  static constexpr int PR = D * ELEM / 16;    // 16-byte pieces per cache row
  static constexpr int RPI = 64 / PR;         // rows per wave load of V
  static constexpr int VS = D + 16;           // LDS row stride of the V tile (bf16)
};

// Registers that carry one chunk from HBM to the products.  K and V have one
// buffer each: within an iteration the V tile of chunk i goes to LDS before
// the V loads of chunk i+NW are issued into the same registers, and the K
// rows of chunk i feed the score products before the K loads of chunk i+NW
// are issued, so both loads are in flight while chunk i finishes.
template <typename CT, int D>
struct KStage {
  uint4 k[kNT][Geometry<CT, D>::KV4];
  float ksc[kNT], vsc[kNT];  // FP8 scales of the lane's 4-token groups
};

template <typename CT, int D>
struct VStage {
  uint4 v[kNT][Geometry<CT, D>::KV4];  // the chunk's V rows, kNT*KV4 wave loads
};

// Where a step's loads read from: the caches and FP8 scales, or the dummy row.
struct Src {
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
};

// One work item's view of its partition.
// Rows: the (query token, head) pairs of one KV head, row m * G + g for
// token m and head kvh * G + g (with one token per sequence, row = head).
// An item covers nh <= 16 consecutive rows from r0.
struct Part {
  int seq, kvh, r0, nh, start, end, first_blk;
  int pre;  // an item over the shared prefix (split-prefix launches; 0 otherwise)
  int sub;  // position whose K and V rows are read from the new rows, not the
            // cache (write fused into a decode; -1 otherwise)
};

// Index of a row's [D] vector in q / out ([S][M][H][D]) and of its partial.
template <int MODE>
__device__ __forceinline__ size_t row_of(const MfmaParams& p, const Part& w, int rho) {
  if constexpr (MODE == kModeCausal) {
    const int m = rho / p.G;
    return ((size_t)w.seq * p.M + m) * p.H + (size_t)w.kvh * p.G + (rho - m * p.G);
  } else {
    if constexpr (MODE == kModeSplitPrefix) {
      if (w.pre) {  // row rho of a prefix item: head rho % G of sequence rho / G
        const int sq = rho / p.G;
        return (size_t)sq * p.H + (size_t)w.kvh * p.G + (rho - sq * p.G);
      }
    }
    return (size_t)w.seq * p.H + (size_t)w.kvh * p.G + rho;
  }
}

// Block ids of a chunk (tokens c0 .. c0 + CHUNK - 1) are CHUNK / BS
// consecutive entries ctab[0 ..]; a chunk starts on a block boundary.
template <typename CT, int D, int BS>
__device__ __forceinline__ size_t token_row(const MfmaParams& p, const Part& w, const int* ctab,
                                            int c0, int t, int lane) {
  const int phys = ctab[(t - c0) / BS];
  return (((size_t)phys * p.H_kv + w.kvh) * BS + (t % BS)) * D + Geometry<CT, D>::DQ * (lane >> 4);
}

// V rows are fetched whole: wave load j covers rows j*RPI .. of the chunk,
// lane l the 16-byte piece l % PR of row j*RPI + l / PR, so every load
// instruction reads whole token rows (fully used cache lines).
template <typename CT, int D, int BS, int MODE>
__device__ __forceinline__ void load_v(VStage<CT, D>& st, const MfmaParams& p, const Src& src,
                                       const Part& w, const int* ctab, int c0, int lane) {
  using CS = typename CT::storage;
  using Gm = Geometry<CT, D>;
  constexpr int PR = Gm::PR, RPI = Gm::RPI;
  const CS* vc = reinterpret_cast<const CS*>(src.v);
  uint4* flat = &st.v[0][0];
#pragma unroll
  for (int j = 0; j < kNT * Gm::KV4; ++j) {
    const int t = min(c0 + j * RPI + lane / PR, w.end - 1);  // clamped: masked later
    const int phys = ctab[(t - c0) / BS];
    const size_t row = ((size_t)phys * p.H_kv + w.kvh) * BS + (t % BS);
    const CS* vrow = vc + row * D;
    if constexpr (MODE == kModeDecodeWrite) {
      if (t == w.sub)  // the new row, as the fused write stores it
        vrow = reinterpret_cast<const CS*>(p.new_v) + ((size_t)w.seq * p.H_kv + w.kvh) * D;
    }
    flat[j] = reinterpret_cast<const uint4*>(vrow)[lane % PR];
  }
}

template <typename CT, int D, int BS, int MODE>
__device__ __forceinline__ void load_k(KStage<CT, D>& st, const MfmaParams& p, const Src& src,
                                       const Part& w, const int* ctab, int c0, int lane) {
  using CS = typename CT::storage;
  const CS* kc = reinterpret_cast<const CS*>(src.k);
#pragma unroll
  for (int T = 0; T < kNT; ++T) {
    const int t = min(c0 + 16 * T + (lane & 15), w.end - 1);  // clamped: masked later
    const uint4* krow =
        reinterpret_cast<const uint4*>(kc + token_row<CT, D, BS>(p, w, ctab, c0, t, lane));
    if constexpr (MODE == kModeDecodeWrite) {
      if (t == w.sub)  // the new row, as the fused write stores it
        krow = reinterpret_cast<const uint4*>(
            reinterpret_cast<const CS*>(p.new_k) + ((size_t)w.seq * p.H_kv + w.kvh) * D +
            Geometry<CT, D>::DQ * (lane >> 4));
    }
#pragma unroll
    for (int i = 0; i < Geometry<CT, D>::KV4; ++i) st.k[T][i] = krow[i];
    if constexpr (Geometry<CT, D>::ELEM == 1) {
      // the lane's scores are tokens 16T + 4q + i: one block for every bs >= 4
      const int ts = min(c0 + 16 * T + 4 * (lane >> 4), w.end - 1);
      const size_t si = (size_t)ctab[(ts - c0) / BS] * p.H_kv + w.kvh;
      st.ksc[T] = src.ks[si];
      st.vsc[T] = src.vs[si];
    }
  }
}

// The chunk's V rows -> this wave's LDS tile as bf16 (rows past the end as
// zeros), in the order load_v fetched them.
template <typename CT, int D>
__device__ __forceinline__ void store_v(const VStage<CT, D>& st, int c0, int end, uint16_t* s_v,
                                        int lane) {
  using Gm = Geometry<CT, D>;
  const bool full = c0 + Gm::CHUNK <= end;
  wave_lds_sync();  // the previous chunk's transpose reads are done
#pragma unroll
  for (int T = 0; T < kNT; ++T) {
#pragma unroll
    for (int i = 0; i < Gm::KV4; ++i) {
      const int j = T * Gm::KV4 + i;
      const int row = j * Gm::RPI + lane / Gm::PR;
      const int piece = lane % Gm::PR;
      uint4 v = st.v[T][i];
      if (!full) {
        const bool ok = c0 + row < end;
        v.x = ok ? v.x : 0u; v.y = ok ? v.y : 0u; v.z = ok ? v.z : 0u; v.w = ok ? v.w : 0u;
      }
      if constexpr (Gm::ELEM == 2) {
        *reinterpret_cast<uint4*>(s_v + row * Gm::VS + piece * 8) = v;
      } else {
        const uint2 a = fp8x4_to_bf16x4(v.x), b = fp8x4_to_bf16x4(v.y);
        const uint2 c = fp8x4_to_bf16x4(v.z), d = fp8x4_to_bf16x4(v.w);
        // A lane's 32 bytes are two 16-byte halves; pieces 4..7 of a row
        // store their upper half first, so the 8 lanes of one store phase
        // cover 8 different 16-byte bank groups (32-byte steps alone repeat
        // after 4 lanes).
        const bool sw = (piece & 4) != 0;
        const uint4 h0 = make_uint4(sw ? c.x : a.x, sw ? c.y : a.y, sw ? d.x : b.x, sw ? d.y : b.y);
        const uint4 h1 = make_uint4(sw ? a.x : c.x, sw ? a.y : c.y, sw ? b.x : d.x, sw ? b.y : d.y);
        uint16_t* base = s_v + row * Gm::VS + piece * 16;
        *reinterpret_cast<uint4*>(base + (sw ? 8 : 0)) = h0;
        *reinterpret_cast<uint4*>(base + (sw ? 0 : 8)) = h1;
      }
    }
  }
  wave_lds_sync();  // the tile is visible to every lane of the wave
}

// Scores S^T = K . Q^T of the chunk's tiles: lane (q, r) gets head r,
// tokens 16 T + 4 q + i.
template <typename CT, int D>
__device__ __forceinline__ void scores(const KStage<CT, D>& st, const uint4* s_qf,
                                       f32x4_t (&s)[kNT], int lane) {
  using Gm = Geometry<CT, D>;
  // Q operand fragments, kept in LDS to spare registers: lane (q, r) reads
  // head r, elements (D/4) q + 8 c .. + 8, stored as s_qf[c][lane].
  bf16x8_t qf[Gm::NKC];
#pragma unroll
  for (int c = 0; c < Gm::NKC; ++c) qf[c] = as_bf16x8(s_qf[c * 64 + lane]);
#pragma unroll
  for (int T = 0; T < kNT; ++T) {
    s[T] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Gm::NKC; ++c) {
      bf16x8_t a;
      if constexpr (Gm::ELEM == 2) {
        a = as_bf16x8(st.k[T][c]);  // bytes 16c..16c+15 of the lane's slice
      } else {
        const uint4 w = st.k[T][c / 2];  // bytes 8c..8c+7 of the lane's 32-byte slice
        const uint2 lo = fp8x4_to_bf16x4((c & 1) ? w.z : w.x);
        const uint2 hi = fp8x4_to_bf16x4((c & 1) ? w.w : w.y);
        a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
      s[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], s[T], 0, 0, 0);
    }
  }
}

// Online softmax update with this chunk's scores, then O^T += V^T . P^T.
template <int D>
__device__ __forceinline__ void softmax_pv(const f32x4_t (&s)[kNT], const float (&fk)[kNT],
                                           const float (&fv)[kNT], bool scaled_v, int c0,
                                           int full_end, int end, const uint16_t* s_v,
                                           f32x4_t (&acc)[D / 16], float& m, float& lsum,
                                           int lane) {
  // end: this lane's row sees tokens below it; full_end (uniform, <= every
  // row's end): a chunk below it needs no mask.
  constexpr int VS = D + 16;
  const int q = lane >> 4, r = lane & 15;
  const bool full = c0 + 16 * kNT <= full_end;
  float x[kNT][4];
  float mc = kNegInf;
#pragma unroll
  for (int T = 0; T < kNT; ++T) {
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

  float pv[kNT][4];
  float ps = 0.f;
#pragma unroll
  for (int T = 0; T < kNT; ++T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(x[T][i] - m_new);
      ps += e;
      pv[T][i] = scaled_v ? e * fv[T] : e;
    }
  }
  lsum = fmaf(lsum, alpha, ps);
  // Unconditional: a branch around the rescale makes the register allocator
  // reconcile the accumulators with copies, whose sources include registers
  // the prefetch loads are filling, which forces a wait on those loads.
#pragma unroll
  for (int md = 0; md < D / 16; ++md) acc[md] *= alpha;

  // Transpose reads: lane j of group q addresses row 4q + j/4 (and + 16) at
  // d = 16 md + 4 (j % 4).
  const uint16_t* rowp = s_v + (4 * q + (r >> 2)) * VS + 4 * (r & 3);
#pragma unroll
  for (int u = 0; u < kNT / 2; ++u) {
    // P^T operand: tokens 4q..4q+3 of tile 2u, then of tile 2u+1.
    const bf16x8_t pb = as_bf16x8(make_uint4(pack_bf16x2(pv[2 * u][0], pv[2 * u][1]),
                                             pack_bf16x2(pv[2 * u][2], pv[2 * u][3]),
                                             pack_bf16x2(pv[2 * u + 1][0], pv[2 * u + 1][1]),
                                             pack_bf16x2(pv[2 * u + 1][2], pv[2 * u + 1][3])));
#pragma unroll
    for (int md = 0; md < D / 16; ++md) {
      const uint16_t* p0 = rowp + 32 * u * VS + 16 * md;
      const uint16_t* p1 = p0 + 16 * VS;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
      const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
      const bf16x8_t a = as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
      acc[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[md], 0, 0, 0);
    }
  }
  // Interleave the transpose reads with the products (two reads, one MFMA)
  // instead of issuing all reads first: that holds 2 fragments, not 2 * NMD.
#pragma unroll
  for (int i = 0; i < (kNT / 2) * (D / 16); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
}

// Item order of the sequence scan: first every full partition (P tokens) of
// every sequence, then every sequence's last, shorter partition (a sequence
// of length 0 has one empty item, which writes zeros).  Sequences are taken
// in order of decreasing size of that last partition (longest processing
// time first): with whole contexts as items (P at least the longest
// context) the longest contexts start first and the shortest run last,
// which keeps the end of the kernel balanced across workgroups.
//   s_seq[k]:   the sequence at sorted position k and its context length n,
//               packed as n << kSeqBits | sequence (n < 2^(31 - kSeqBits))
//   s_full[k]:  full partitions of the sequences at positions 0..k-1
//               (s_full[S] = F)
//   s_rag[k]:   short partitions of the sequences at positions 0..k-1
//               (s_rag[S] = R)
// Returns F (and R in *n_rag).  Every thread of the workgroup calls it.
//
// The sort is a stable counting sort on the last partition's size in blocks
// (clamped to kSortKeys - 1), so every workgroup computes the same order:
// thread t holds sequences t and t + 256, i.e. wave w holds the 64-sequence
// chunks w and w + 4; per-chunk key counts give each sequence the number of
// equal keys in earlier chunks, and a ballot within the wave its rank among
// equal keys in its own chunk.  s_tmp: 9 KiB of LDS scratch.
constexpr int kSortKeys = 256;
constexpr int kSeqBits = 9;  // sequence index bits of an s_seq entry
static_assert((1 << kSeqBits) >= kMaxScanSeqs, "sequence index field");

// Inclusive sum over the 64 lanes of a wave on the DPP network: shifts of
// 1, 2, 4 and 8 within each 16-lane row (lanes past a row's start add 0),
// then row 0's and row 1's last lanes broadcast into the rows after them.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Items of one sorted position: its full partitions and its short (or
// only) one.
__device__ __forceinline__ void seq_items(int packed, int P, int& nf, int& nr) {
  const int n = packed >> kSeqBits;
  nf = n / P;
  nr = (n % P != 0 || n == 0) ? 1 : 0;
}

// First phase of the scan: the thread's context lengths are requested
// (their loads stay in flight) and the LDS counts are cleared.
constexpr int kScanChunks = kMaxScanSeqs / 64;  // 64-sequence chunks
template <int MODE>
__device__ __forceinline__ void scan_begin(const MfmaParams& p, int* s_tmp, int (&len)[2]) {
  constexpr int NTH = kNW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (p.S + 63) >> 6;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * NTH;
    len[r] = i < p.S ? seq_len<MODE>(p, i) : -1;
  }
  for (int k = tid; k < nch * kSortKeys; k += NTH) s_tmp[k] = 0;
  unsigned long long* mask =
      reinterpret_cast<unsigned long long*>(s_tmp + (kScanChunks + 1) * kSortKeys) +
      wave * kSortKeys;
  for (int k = lane; k < kSortKeys; k += 64) mask[k] = 0ull;
}

// Full partitions in sequence order (they all hold P tokens, so their order
// does not matter for longest-first): s_full[i] = (F_i << 1) | r_i, F_i the
// full partitions of sequences before i and r_i whether sequence i ends in
// a shorter (or empty) partition; s_full[S] = F << 1.  A workgroup whose
// first item is a full partition can start it from this alone, before the
// sort of the last partitions.  Returns F.
__device__ int full_offsets(const MfmaParams& p, int* s_full, int* s_red, const int (&len)[2]) {
  constexpr int NTH = kNW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int nf[2], rg[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int n = max(len[r], 0);
    nf[r] = len[r] >= 0 ? n / p.P : 0;
    rg[r] = len[r] >= 0 && (n % p.P != 0 || n == 0) ? 1 : 0;
  }
  const int inc0 = wave_inclusive_sum(nf[0]);
  const int inc1 = wave_inclusive_sum(nf[1]);
  if (lane == 63) {
    s_red[wave] = inc0;
    s_red[kNW + wave] = inc1;
  }
  __syncthreads();
  int e0 = inc0 - nf[0], e1 = inc1 - nf[1], t0 = 0, t1 = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const int a = s_red[w], b = s_red[kNW + w];
    e0 += w < wave ? a : 0;
    e1 += w < wave ? b : 0;
    t0 += a;
    t1 += b;
  }
  // sequences tid (offset e0) and NTH + tid (after all of the first NTH)
  if (len[0] >= 0) s_full[tid] = (e0 << 1) | rg[0];
  if (len[1] >= 0) s_full[NTH + tid] = ((t0 + e1) << 1) | rg[1];
  if (tid == 0) s_full[p.S] = (t0 + t1) << 1;
  __syncthreads();  // s_full complete; s_red free again
  return t0 + t1;
}

template <int MODE, int BS>
__device__ void build_offsets(const MfmaParams& p, uint16_t* s_rag, int* s_seq,
                             int* s_red, int* s_tmp, const int (&len)[2],
                             int* n_rag) {
  constexpr int NTH = kNW * 64;
  constexpr int NCH = kScanChunks;
  static_assert(kMaxScanSeqs <= 2 * NTH && kSortKeys == NTH, "two sequences, one key per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (p.S + 63) >> 6;       // chunks holding sequences
  int* cnt = s_tmp;                       // [NCH][kSortKeys]
  int* first = s_tmp + NCH * kSortKeys;   // [kSortKeys]: sequences with a larger key
  // [kNW][kSortKeys] 64-bit lane masks: the lanes of a wave's chunk holding each key
  unsigned long long* mask =
      reinterpret_cast<unsigned long long*>(s_tmp + (NCH + 1) * kSortKeys) + wave * kSortKeys;
  __syncthreads();  // the counts cleared by scan_begin
  int key[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * NTH;
    key[r] = -1;
    if (len[r] >= 0) {
      const int n = len[r];
      const int last = n > 0 ? n - ((n - 1) / p.P) * p.P : 0;  // tokens of the last partition
      key[r] = min((last + BS - 1) / BS, kSortKeys - 1);
      atomicAdd(&cnt[(i >> 6) * kSortKeys + key[r]], 1);
    }
  }
  __syncthreads();
  {
    // thread t owns key kSortKeys - 1 - t: a scan over threads then runs over
    // keys in decreasing order
    const int k = kSortKeys - 1 - tid;
    int run = 0;
    for (int c = 0; c < nch; ++c) {
      const int v = cnt[c * kSortKeys + k];
      cnt[c * kSortKeys + k] = run;  // equal keys in earlier chunks
      run += v;
    }
    const int incl = wave_inclusive_sum(run);
    if (lane == 63) s_red[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) before += w < wave ? s_red[w] : 0;
    first[k] = before + incl - run;
  }
  __syncthreads();
  // Rank among equal keys within the wave's chunk: the key's lane mask (an
  // OR, so the result does not depend on the order of the atomics), counted
  // below the lane.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * NTH;
    const bool valid = key[r] >= 0;
    if (r == 1 && p.S <= NTH) break;  // uniform: no second round
    if (valid) atomicOr(&mask[key[r]], 1ull << lane);
    wave_lds_sync();
    if (valid) {
      const int rank = __builtin_popcountll(mask[key[r]] & ((1ull << lane) - 1ull));
      s_seq[first[key[r]] + cnt[(i >> 6) * kSortKeys + key[r]] + rank] = (len[r] << kSeqBits) | i;
    }
    wave_lds_sync();
    if (valid) mask[key[r]] = 0ull;  // ready for the wave's second chunk
    wave_lds_sync();
  }
  __syncthreads();

  // Short (or only) partitions before each sorted position: one pass of a
  // wave sum, one barrier.
  const int per = (p.S + NTH - 1) / NTH;
  const int base = tid * per;
  int nr = 0;
  for (int k = 0; k < per; ++k) {
    const int pos = base + k;
    if (pos < p.S) {
      int f, r;
      seq_items(s_seq[pos], p.P, f, r);
      nr += r;
    }
  }
  const int incr = wave_inclusive_sum(nr);
  if (lane == 63) s_red[2 * kNW + wave] = incr;
  __syncthreads();
  int er = incr - nr, R = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const int rw = s_red[2 * kNW + w];
    er += w < wave ? rw : 0;
    R += rw;
  }
  for (int k = 0; k < per; ++k) {
    const int pos = base + k;
    if (pos < p.S) {
      int f, r;
      seq_items(s_seq[pos], p.P, f, r);
      s_rag[pos] = (uint16_t)er;
      er += r;
    }
  }
  if (tid == 0) s_rag[p.S] = (uint16_t)R;
  __syncthreads();
  *n_rag = R;
}

// Largest i in [0, S) with off[i] <= rest, for non-decreasing off with
// off[0] <= rest < off[S].
template <typename T>
__device__ __forceinline__ int find_seq(const T* off, int S, int rest) {
  int lo = 0, hi = S;  // off[lo] <= rest < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int)off[mid] <= rest) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Largest i in [0, S) with full[i] >> 1 <= rest (full offsets in sequence
// order, flag bit 0; see full_offsets).
__device__ __forceinline__ int find_full(const int* full, int S, int rest) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((full[mid] >> 1) <= rest) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Decoded work item: its partition and whether it exists (without the
// sequence scan, items past a sequence's end are placeholders).
struct Item {
  bool live;
  int part, n;
  Part w;
};

// The workgroup's LDS view of the item order.
struct Order {
  const int* full;      // full partitions before each sequence, in sequence order (full_offsets)
  const uint16_t* rag;  // short partitions before each sorted position
  const int* seq;       // n << kSeqBits | sequence, by sorted position
};

// Items [lo, hi) in super-rows of 8 Y: eight consecutive (sequence,
// partition) groups of Y row-group items each.  Position j of a super-row
// becomes row group j / 8 of group j % 8, so the queue that takes every
// eighth item runs all the row groups of one group; a last, shorter
// super-row keeps the plain order.
__device__ __forceinline__ int group_major(int item, int lo, int hi, int Y) {
  const int span = 8 * Y;
  const int j = item - lo;
  const int sr = j / span;
  if (lo + (sr + 1) * span > hi) return item;
  const int r = j - sr * span;
  return lo + sr * span + (r & 7) * Y + (r >> 3);
}

template <int BS, bool SCAN, int MODE>
__device__ __forceinline__ Item decode_item(const MfmaParams& p, int item, int Y, int n_full,
                                            int n_items, const Order& o) {
  Item it;
  it.w.pre = 0;
  it.w.sub = -1;
  if constexpr (MODE == kModeSplitPrefix) {
    // Items [0, pre_items) are the prefix's: KV head x 16-row chunk of the
    // S x G rows (fastest) and prefix partition, over sequence 0's table
    // (every table holds the prefix's blocks).
    if (item < p.pre_items) {
      const int Yp = p.H_kv * p.pre_chunks;
      const int y = item % Yp;
      it.part = item / Yp;
      it.n = p.prefix;
      it.live = true;
      it.w.pre = 1;
      it.w.seq = 0;
      it.w.kvh = y / p.pre_chunks;
      it.w.r0 = (y - it.w.kvh * p.pre_chunks) * 16;
      it.w.nh = min(16, p.S * p.G - it.w.r0);
      it.w.start = it.part * p.P;
      it.w.end = min(it.n, it.w.start + p.P);
      it.w.first_blk = it.w.start / BS;
      return it;
    }
    item -= p.pre_items;
  }
  if constexpr (MODE != kModeSplitPrefix) {
    if (p.group_major) {
      // full partitions and last partitions separately: an early first item
      // (a full partition) is decoded before the last partitions are counted
      const int fl = SCAN ? Y * n_full : 0;
      item = item < fl ? group_major(item, 0, fl, Y) : group_major(item, fl, n_items, Y);
    }
  }
  const int y = item % Y;
  const int rest = item / Y;
  int seq;
  if constexpr (SCAN) {
    // Values read from LDS are per-lane to the compiler; the item is uniform
    // over the workgroup, so move them to scalar registers.
    if (rest < n_full) {
      // A full partition of sequence i.  Its length stands in as
      // (full partitions) x P, plus one if a shorter partition follows: the
      // same partition ends, the same "fits one partition" test and the same
      // partition count as the true length.  Causal rows need the true
      // length (their positions), read from memory.
      const int i = __builtin_amdgcn_readfirstlane(find_full(o.full, p.S, rest));
      const int e0 = __builtin_amdgcn_readfirstlane(o.full[i]);
      const int e1 = __builtin_amdgcn_readfirstlane(o.full[i + 1]);
      seq = i;
      it.part = rest - (e0 >> 1);
      if constexpr (MODE == kModeCausal)
        it.n = __builtin_amdgcn_readfirstlane(seq_len<MODE>(p, i));
      else
        it.n = ((e1 >> 1) - (e0 >> 1)) * p.P + (e0 & 1);
    } else {
      const int pos = __builtin_amdgcn_readfirstlane(find_seq(o.rag, p.S, rest - n_full));
      const int packed = __builtin_amdgcn_readfirstlane(o.seq[pos]);
      it.part = (packed >> kSeqBits) / p.P;
      seq = min(packed & ((1 << kSeqBits) - 1), p.S - 1);
      it.n = packed >> kSeqBits;
    }
    it.live = true;
  } else {
    seq = rest / p.NP;
    it.part = rest - seq * p.NP;
    it.n = seq_len<MODE>(p, seq);
    it.live = it.part == 0 || it.part * p.P < it.n;
  }
  it.w.seq = seq;
  it.w.kvh = y / p.chunks;
  const int hc = y - it.w.kvh * p.chunks;
  it.w.r0 = hc * 16;
  it.w.nh = min(16, p.M * p.G - hc * 16);
  it.w.start = it.part * p.P;
  it.w.end = min(it.n, it.w.start + p.P);
  it.w.first_blk = it.w.start / BS;
  if constexpr (MODE == kModeDecodeWrite) {
    // the partition holding the sequence's newest position reads that
    // position's rows from the new rows (when the call writes them)
    const int slot = p.slots[seq];
    if (it.n > 0 && it.w.end == it.n && slot >= 0 && slot < p.num_slots) it.w.sub = it.n - 1;
  }
  return it;
}

// Block ids of an item, one slice per wave: wave w processes chunks
// w, w + NW, w + 2 NW, .. of the item, and lane l of the wave holds the id of
// block l % EPC of its chunk number l / EPC (EPC = CHUNK / BS blocks per
// chunk; 64 entries cover the kMaxTable blocks an item may span).  Each wave
// writes and reads only its own slice in LDS, so no workgroup barrier guards
// it.  Entries past the item's blocks repeat the row's last entry and are
// never used; a suffix launch's positions start tab_off entries into the
// row, and the clamp keeps every read inside the row.  Plain loads: the compiler tracks them exactly, so they never
// force a wait on the chunk pipeline.
template <typename CT, int D, int BS, int MODE>
__device__ __forceinline__ int fetch_tab(const MfmaParams& p, const Part& w, int wave, int lane) {
  constexpr int EPC = Geometry<CT, D>::CHUNK / BS;
  const int blk = w.first_blk + (wave + kNW * (lane / EPC)) * EPC + lane % EPC;
  // a prefix item's positions start at 0
  const int off = MODE == kModeSplitPrefix && w.pre ? 0 : p.tab_off;
  return p.tables[(size_t)w.seq * p.max_blocks + min(off + blk, p.max_blocks - 1)];
}

__device__ __forceinline__ void store_tab(int tab, int* wtab, int lane) {
  wtab[lane] = tab;
  wave_lds_sync();  // the slice is visible to every lane of the wave
}

// Q operand fragments of an item, one element per thread (thread t owns
// element t), shared by the waves; heads past the group are zeros.
template <typename CT, int D, int MODE>
__device__ __forceinline__ uint4 fetch_q(const MfmaParams& p, const Part& w, int tid) {
  using Gm = Geometry<CT, D>;
  // fragment c = tid / 64 for lane l = (q, r) = tid % 64; threads past the
  // fragments load a clamped one they never store (no branch, no early wait)
  const int i = min(tid, Gm::NKC * 64 - 1);
  const int c = i >> 6, l = i & 63;
  const int hq = l & 15;
  return *reinterpret_cast<const uint4*>(
      reinterpret_cast<const uint16_t*>(p.q) +
      row_of<MODE>(p, w, w.r0 + min(hq, w.nh - 1)) * D + Gm::DQ * (l >> 4) + 8 * c);
}

template <typename CT, int D>
__device__ __forceinline__ void store_q(uint4 v, const Part& w, uint4* qf, int tid) {
  if (tid < Geometry<CT, D>::NKC * 64) {
    const bool z = (tid & 15) < w.nh;  // head (tid % 64) % 16 of fragment tid / 64
    qf[tid] = make_uint4(z ? v.x : 0u, z ? v.y : 0u, z ? v.z : 0u, z ? v.w : 0u);
  }
}

// Fused merge of split partitions (one query token per sequence, at most
// kFusedMaxPartitions partitions per context).  Each partition item leaves
// (m_p, l_p, acc_p) for its rows; one softmax over the whole context is
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p
// (dpshk.com PagedAttention article, section 2.2), the reduce kernel's
// arithmetic in the same order.  No workgroup waits for another: the
// partials are stored at agent scope (coherent across the XCDs' L2s), and
// each wave, once those stores are complete, counts itself into the row
// group's arrival counter with one atomic.  That happens at the wave's last
// chunk step of its next item, after a wait for everything the wave has in
// flight (at that point only the K rows of the step it is about to compute,
// so the wait costs little); the atomic's result is read after the next
// item's barrier X.  The wave that brings the count to 4 x (partitions)
// is the last: its workgroup merges the group (agent-scope loads) and
// returns the counter to zero.
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt not waited for

__device__ __forceinline__ void wait_stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no compiler motion of memory accesses across
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ int arrive(const MfmaParams& p, int group) {
  return __hip_atomic_fetch_add(p.arrivals + group, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int MODE>
__device__ __forceinline__ void merge_group(const MfmaParams& p, int group, int np) {
  const int Y = p.H_kv * p.chunks;
  Part w{};
  w.seq = group / Y;
  const int y = group - w.seq * Y;
  w.kvh = y / p.chunks;
  w.r0 = (y - w.kvh * p.chunks) * 16;
  w.nh = min(16, p.M * p.G - w.r0);
  // Thread t merges 4 consecutive d of one row, as the epilogue writes them.
  for (int idx = (int)threadIdx.x * 4; idx < w.nh * D; idx += kNW * 64 * 4) {
    const int g = idx / D;
    const int d = idx - g * D;
    const size_t row = row_of<MODE>(p, w, w.r0 + g);
    float pm[kFusedMaxPartitions], pl[kFusedMaxPartitions];
    unsigned long long pa[kFusedMaxPartitions];
#pragma unroll
    for (int u = 0; u < kFusedMaxPartitions; ++u) {
      const size_t pi = row * p.NP + min(u, np - 1);
      pa[u] = __hip_atomic_load(reinterpret_cast<unsigned long long*>(
                                    reinterpret_cast<uint16_t*>(p.ws_acc) + pi * D + d),
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pm[u] = __hip_atomic_load(p.ws_m + pi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pl[u] = __hip_atomic_load(p.ws_l + pi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < kFusedMaxPartitions; ++u)
      if (u < np) M = fmaxf(M, pm[u]);
    float L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kFusedMaxPartitions; ++u) {
      if (u < np) {
        const float wt = __builtin_amdgcn_exp2f(pm[u] - M);
        L = fmaf(pl[u], wt, L);
        const uint32_t lo = (uint32_t)pa[u], hi = (uint32_t)(pa[u] >> 32);
        O[0] = fmaf(bf16_lo(lo), wt, O[0]);
        O[1] = fmaf(bf16_hi(lo), wt, O[1]);
        O[2] = fmaf(bf16_lo(hi), wt, O[2]);
        O[3] = fmaf(bf16_hi(hi), wt, O[3]);
      }
    }
    const bool ok = L > 0.f;
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + d) =
        make_uint2(pack_bf16x2(ok ? O[0] / L : 0.f, ok ? O[1] / L : 0.f),
                   pack_bf16x2(ok ? O[2] / L : 0.f, ok ? O[3] / L : 0.f));
  }
}

// The fused write's share of an item (kModeDecodeWrite): the item holding a
// sequence's newest position, in its first row chunk, copies the new K and
// V rows of its KV head to their slot; lanes [0, PR) of wave 0 hold the K
// row's 16-byte pieces and lanes [PR, 2 PR) the V row's.  The pieces are
// requested with the item's block ids, so they have arrived when the item
// stores them.
template <typename CT, int D, int MODE>
__device__ __forceinline__ bool copies_row(const Item& it, int wave, int lane) {
  return MODE == kModeDecodeWrite && it.live && it.w.sub >= 0 && it.w.r0 == 0 && wave == 0 &&
         lane < 2 * Geometry<CT, D>::PR;
}

template <typename CT, int D, int MODE>
__device__ __forceinline__ uint4 fetch_new_row(const MfmaParams& p, const Item& it, int wave,
                                               int lane) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (MODE == kModeDecodeWrite) {
    if (copies_row<CT, D, MODE>(it, wave, lane)) {
      using CS = typename CT::storage;
      constexpr int PR = Geometry<CT, D>::PR;
      const CS* from = reinterpret_cast<const CS*>(lane >= PR ? p.new_v : p.new_k) +
                       ((size_t)it.w.seq * p.H_kv + it.w.kvh) * D;
      v = reinterpret_cast<const uint4*>(from)[lane % PR];
    }
  }
  return v;
}

template <typename CT, int D, int BS, bool SCAN, int MODE>
__global__ __launch_bounds__(kNW * 64) void decode_mfma_kernel(MfmaParams p) {
  using Gm = Geometry<CT, D>;
  static_assert(kMaxTable == kNW * 64, "one table entry per thread");
  static_assert(Gm::NKC <= kNW, "one Q fragment row per wave");
  constexpr int VTILE = Gm::CHUNK * Gm::VS;  // bf16 elements per wave
  // fp32 partial outputs, rows padded by 4 floats: the 16-byte writes of
  // 8 lanes (8 rows, same columns) then fall on distinct banks.
  constexpr int MS = D + 4;
  constexpr int MERGE = kNW * 16 * MS;
  constexpr int UNION_BYTES = (VTILE * kNW * 2 > MERGE * 4) ? VTILE * kNW * 2 : MERGE * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[UNION_BYTES];
  __shared__ int s_wtab[kNW][kMaxTable / kNW];
  __shared__ uint4 s_qf[Gm::NKC * 64];
  __shared__ float s_m[kNW][16];
  __shared__ float s_l[kNW][16];
  __shared__ int s_red[3 * kNW];
  __shared__ int s_next[2];  // next claimed item, queue flag
  __shared__ int s_zero[4];  // block id 0 for the dummy row
  __shared__ int s_full[SCAN ? kMaxScanSeqs + 1 : 1];
  __shared__ uint16_t s_rag[SCAN ? kMaxScanSeqs + 1 : 1];
  __shared__ int s_seq[SCAN ? kMaxScanSeqs : 1];
  static_assert(UNION_BYTES >= (kMaxScanSeqs / 64 + 1) * kSortKeys * 4 + kNW * kSortKeys * 8,
                "sort scratch");
  const Order order{s_full, s_rag, s_seq};

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps selects scalar
  const int lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;
  const int Y = p.H_kv * p.chunks;
  // Items over a shared prefix, numbered before the others (split-prefix
  // launches).
  const int n_pre = MODE == kModeSplitPrefix ? p.pre_items : 0;

  // Items [0, n_local) form the per-XCD queues: queue `queue` holds items
  // k * nq + queue.  Workgroup b starts with item b (no atomic traffic at
  // launch); claim c of the queue's counter is item (queue_wgs + c) * nq +
  // queue.  Items [n_local, total) form the shared queue: its claim c is
  // item n_local + c.  A workgroup claims its next item at the start of the
  // current item's last chunk step, so the claim's latency is hidden, and
  // starts it after a short pause for its block ids, Q and first chunk.  A
  // CU serves its resident workgroups by age (the youngest runs at about a
  // third of the oldest's rate while the others are busy): that pause is
  // longest for the young ones, and the other workgroups on the CU fill it.
  // With bf16 caches and three or more workgroups per CU the youngest on
  // each CU (blockIdx.x >= young_from) runs only its first item: it helps
  // while the queues fill the CU, and an item it claimed later would start
  // late and end last.
  const int nq = min(8, (int)gridDim.x);
  const int queue = blockIdx.x % nq;
  const int queue_wgs = ((int)gridDim.x - queue + nq - 1) / nq;
  int* claim_ctr = p.sched + queue * kCounterStride;
  int* shared_ctr = p.sched + 8 * kCounterStride;
  int* done_ctr = p.sched + 9 * kCounterStride;
  if (tid == 0) s_next[0] = blockIdx.x;
  if (tid < 4) s_zero[tid] = 0;
  int len[2] = {-1, -1};
  if constexpr (SCAN) scan_begin<MODE>(p, reinterpret_cast<int*>(s_raw), len);
  constexpr int EPC = Gm::CHUNK / BS;  // block ids per chunk
  const Src dummy{g_dummy_row, g_dummy_row, reinterpret_cast<const float*>(g_dummy_row),
                  reinterpret_cast<const float*>(g_dummy_row)};
  const Src cache{p.kc, p.vc, p.ks, p.vs};
  Part dummy_part{};  // token 0 of block 0, KV head 0: row 0 of the dummy
  dummy_part.end = 1;
  dummy_part.sub = -1;

  KStage<CT, D> ks;
  VStage<CT, D> vs;
  // A wave without a chunk of its first item runs a masked step on
  // whatever its registers hold: selects turn those scores into -inf and V
  // rows into zeros, but the FP8 V scale multiplies p = 0, so it must not be
  // left uninitialised (0 * NaN = NaN).
#pragma unroll
  for (int T = 0; T < kNT; ++T) ks.ksc[T] = ks.vsc[T] = 0.f;

  int total, n_full = 0;
  Item it{};
  int tab_first = 0;
  uint4 q_first = make_uint4(0u, 0u, 0u, 0u);
  uint4 new_row = make_uint4(0u, 0u, 0u, 0u);  // the fused write's pieces of the item
  // Uniform: the first item is a full partition, found from the full
  // offsets alone; its block ids and Q are fetched and its first chunk's
  // loads issued before the sort of the last partitions, which then runs
  // while they are in flight.
  bool early = false;
  if constexpr (SCAN) {
    n_full = full_offsets(p, s_full, s_red, len);  // has barriers: s_next is visible
    const int first = __builtin_amdgcn_readfirstlane(s_next[0]);
    if constexpr (MODE == kModeSplitPrefix)
      early = first >= n_pre && first - n_pre < Y * n_full;
    else
      early = first < Y * n_full;
    if (early) {
      it = decode_item<BS, SCAN, MODE>(p, first, Y, n_full, 0, order);
      tab_first = fetch_tab<CT, D, BS, MODE>(p, it.w, wave, lane);
      q_first = fetch_q<CT, D, MODE>(p, it.w, tid);
      new_row = fetch_new_row<CT, D, MODE>(p, it, wave, lane);
      store_tab(tab_first, s_wtab[wave], lane);  // the wave's own slice
      wave_lds_sync();
      const int nvalid = (it.w.end - it.w.start + Gm::CHUNK - 1) / Gm::CHUNK;
      if (nvalid > wave) {
        const int c0 = it.w.start + wave * Gm::CHUNK;
        load_v<CT, D, BS, MODE>(vs, p, cache, it.w, s_wtab[wave], c0, lane);
        load_k<CT, D, BS, MODE>(ks, p, cache, it.w, s_wtab[wave], c0, lane);
      }
    }
    int n_rag;
    // has barriers; s_raw is free until the first chunk's V rows are stored
    build_offsets<MODE, BS>(p, s_rag, s_seq, s_red, reinterpret_cast<int*>(s_raw), len, &n_rag);
    total = Y * (n_full + n_rag) + n_pre;
  } else {
    total = n_pre + Y * p.S * p.NP;
    __syncthreads();
  }
  // About one shared item per workgroup, and never so many that a static
  // item would fall in the shared range.
  const int n_local = total - max(0, min((int)gridDim.x, total - 2 * (int)gridDim.x - 16));
  // Uniform (thread 0 decides, every thread reads it back after barrier
  // Y): this workgroup's own queue is empty and it claims from the shared
  // one.  Kept uniform so its selects stay scalar.
  int use_shared = 0;
  int cur = s_next[0];
  // Uniform: this workgroup runs its first item and claims no other (only
  // while every queue keeps a workgroup that claims: workgroup `queue`).
  const bool stop = (int)blockIdx.x >= p.young_from && p.young_from >= nq;
  // Otherwise the first item's block ids and Q are requested together (one
  // memory round trip before the first chunk's loads, not two).
  if (!early) {
    it = decode_item<BS, SCAN, MODE>(p, min(cur, total - 1), Y, n_full, total - n_pre, order);
    tab_first = fetch_tab<CT, D, BS, MODE>(p, it.w, wave, lane);
    q_first = fetch_q<CT, D, MODE>(p, it.w, tid);
    new_row = fetch_new_row<CT, D, MODE>(p, it, wave, lane);
  }
  if (cur < total) {
    if (!early) store_tab(tab_first, s_wtab[wave], lane);
    store_q<CT, D>(q_first, it.w, s_qf, tid);
  }
  __syncthreads();

  // Fused merge: the row group (sequence x Y + y) of the previous item,
  // whose partials this workgroup stored and has not yet counted in (-1:
  // none), and the group's partition count.  Uniform.
  int pg = -1, pnp = 0;
  const bool fused = (MODE == kModeDecode || MODE == kModeDecodeWrite) && p.fused != 0;
  // Uniform: the item's first chunk is still to be requested (every item's
  // but an early first one's, which went out before the sort).
  bool prime = !early;

  while (cur < total) {
    if (prime && it.live) {
      const int nvalid = (it.w.end - it.w.start + Gm::CHUNK - 1) / Gm::CHUNK;
      if (nvalid > wave) {
        const int c0 = it.w.start + wave * Gm::CHUNK;
        load_v<CT, D, BS, MODE>(vs, p, cache, it.w, s_wtab[wave], c0, lane);
        load_k<CT, D, BS, MODE>(ks, p, cache, it.w, s_wtab[wave], c0, lane);
      }
    }
    prime = false;
    if constexpr (MODE == kModeDecodeWrite) {
      // The fused write's store (nothing in this launch reads the slot: the
      // items over the position take the rows from new_k / new_v).
      if (copies_row<CT, D, MODE>(it, wave, lane)) {
        using CS = typename CT::storage;
        const int slot = p.slots[it.w.seq];
        const size_t dst = (((size_t)(slot / BS) * p.H_kv + it.w.kvh) * BS + slot % BS) * D;
        CS* to = const_cast<CS*>(reinterpret_cast<const CS*>(lane >= Gm::PR ? p.vc : p.kc)) + dst;
        reinterpret_cast<uint4*>(to)[lane % Gm::PR] = new_row;
      }
    }
    // The claim of the next item, made at the start of wave 0's last step
    // (before its loads) and used only after barrier X.
    // (Only thread 0 sets and reads it: initialising it in the other lanes
    // would make the compiler wait for every pending load first.)
    int claim;
    // The wave's arrival count for group pg (lane 0 only, likewise).
    int arr;

    f32x4_t acc[Gm::NMD];
#pragma unroll
    for (int md = 0; md < Gm::NMD; ++md) acc[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = kRunMaxInit, lsum = 0.f;

    uint16_t* s_v = reinterpret_cast<uint16_t*>(s_raw) + wave * VTILE;
    const int nvalid = it.live ? (it.w.end - it.w.start + Gm::CHUNK - 1) / Gm::CHUNK : 0;
    // A wave with no chunk of this item runs one fully masked step, which
    // leaves its state at (kRunMaxInit, 0, 0), so that every wave reaches
    // the loads below.
    const int* ctab = s_wtab[wave];  // this chunk's block ids
    // Causal rows (several query tokens per sequence): token m of a
    // sequence of n cached tokens sits at position n - M + m and sees
    // positions up to it.  With one token per sequence every row sees the
    // whole partition.
    int full_end = it.w.end, row_end = it.w.end;
    if constexpr (MODE == kModeCausal) {
      const int base = it.n - p.M + 1;  // end of token 0's row
      row_end = min(it.w.end, base + (it.w.r0 + r) / p.G);
      full_end = min(it.w.end, base + it.w.r0 / p.G);
    } else if constexpr (MODE == kModeSplitPrefix) {
      if (it.w.pre) {
        // Row r of a prefix item belongs to sequence (r0 + r) / G, which
        // sees the prefix only up to its own length.
        const int sq = min((it.w.r0 + r) / p.G, p.S - 1);
        row_end = min(it.w.end, p.lens[sq]);
        full_end = __all(row_end >= it.w.end) ? it.w.end : it.w.start;
      }
    }
    int ci = wave;
    do {
      const int c0 = it.w.start + ci * Gm::CHUNK;
      const bool last = ci + kNW >= nvalid;
      if (last && pg >= 0) {
        // The previous item's partial stores are older than anything
        // else in flight but this step's K rows.
        wait_stores_complete();
        if (lane == 0) arr = arrive(p, pg);
      }
      if (last && tid == 0 && !stop) claim = atomicAdd(use_shared ? shared_ctr : claim_ctr, 1);
      // Where the prefetch goes: this wave's next chunk of the item, else
      // (last step) the dummy row (scalar selects, no branch).
      const Src src = last ? dummy : cache;
      const Part lw = last ? dummy_part : it.w;
      const int* ntab = last ? s_zero : ctab + EPC;
      const int cn = last ? 0 : c0 + kNW * Gm::CHUNK;
      store_v<CT, D>(vs, c0, it.w.end, s_v, lane);
      load_v<CT, D, BS, MODE>(vs, p, src, lw, ntab, cn, lane);
      // Keep the scheduler from sinking the prefetch below the products:
      // the loads must be in flight while this chunk is computed.
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t sc[kNT];
      scores<CT, D>(ks, s_qf, sc, lane);
      float fk[kNT], fv[kNT];
#pragma unroll
      for (int T = 0; T < kNT; ++T) {
        fk[T] = p.scale_log2;
        fv[T] = 1.f;
        if constexpr (Gm::ELEM == 1) {
          fk[T] *= ks.ksc[T];
          fv[T] = ks.vsc[T];
        }
      }
      load_k<CT, D, BS, MODE>(ks, p, src, lw, ntab, cn, lane);
      __builtin_amdgcn_sched_barrier(0);
      softmax_pv<D>(sc, fk, fv, Gm::ELEM == 1, c0, full_end, row_end, s_v, acc, m, lsum, lane);
      ci += kNW;
      ctab += EPC;
    } while (ci < nvalid);
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    __syncthreads();  // X: the V tiles are free
    if (tid == 0) {
      // A claim past the local items moves this workgroup to the shared
      // queue for good; that first shared claim is the only one made here.
      int item;
      if (stop) {
        item = total;  // no claim was made
      } else if (!use_shared) {
        item = (queue_wgs + claim) * nq + queue;
        if (item >= n_local) {
          use_shared = 1;
          item = n_local + atomicAdd(shared_ctr, 1);
        }
      } else {
        item = n_local + claim;
      }
      s_next[0] = item;
      s_next[1] = use_shared;
    }
    // s_red is free after the prologue: flag of the wave that arrived last.
    if (pg >= 0 && lane == 0) s_red[wave] = arr == kNW * pnp - 1;

    // Merge the wave-level softmax states of this partition.
    float* s_acc = reinterpret_cast<float*>(s_raw);
    if (q == 0) {
      s_m[wave][r] = m;
      s_l[wave][r] = lsum;
    }
#pragma unroll
    for (int md = 0; md < Gm::NMD; ++md)
      *reinterpret_cast<f32x4_t*>(&s_acc[(wave * 16 + r) * MS + 16 * md + 4 * q]) = acc[md];
    __syncthreads();  // Y

    // The next item is known now: its block ids and Q are requested here
    // and stored after barrier Z, so their latency overlaps the epilogue.
    const int nn = __builtin_amdgcn_readfirstlane(s_next[0]);
    use_shared = __builtin_amdgcn_readfirstlane(s_next[1]);
    const bool merge_prev =
        pg >= 0 && __builtin_amdgcn_readfirstlane(s_red[0] | s_red[1] | s_red[2] | s_red[3]);
    const Item ni =
        decode_item<BS, SCAN, MODE>(p, min(nn, total - 1), Y, n_full, total - n_pre, order);
    const uint4 row_nn = fetch_new_row<CT, D, MODE>(p, ni, wave, lane);
    const int tab_nn = fetch_tab<CT, D, BS, MODE>(p, ni.w, wave, lane);
    const uint4 q_nn = fetch_q<CT, D, MODE>(p, ni.w, tid);

    // Thread t merges 4 consecutive d of one head: one 16-byte LDS read per
    // wave state and one 16-byte (8-byte for bf16) store, so few stores
    // are left for the next item's first wait to drain.
    if (it.live) {
      const bool single = !kSplit<MODE> && it.n <= p.P;
      for (int idx = tid * 4; idx < it.w.nh * D; idx += kNW * 64 * 4) {
        const int g = idx / D;
        const int d = idx - g * D;
        // Every wave's m is finite (at least kRunMaxInit); waves without
        // tokens carry l = 0 and acc = 0 and get weight 0 or add nothing.
        float M = kRunMaxInit;
#pragma unroll
        for (int k = 0; k < kNW; ++k) M = fmaxf(M, s_m[k][g]);
        float L = 0.f;
        float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < kNW; ++k) {
          const float wt = __builtin_amdgcn_exp2f(s_m[k][g] - M);
          L = fmaf(s_l[k][g], wt, L);
          const float4 a = *reinterpret_cast<const float4*>(&s_acc[(k * 16 + g) * MS + d]);
          O.x = fmaf(a.x, wt, O.x);
          O.y = fmaf(a.y, wt, O.y);
          O.z = fmaf(a.z, wt, O.z);
          O.w = fmaf(a.w, wt, O.w);
        }
        const size_t row = row_of<MODE>(p, it.w, it.w.r0 + g);
        if (single) {
          const bool ok = L > 0.f;
          const float ox = ok ? O.x / L : 0.f, oy = ok ? O.y / L : 0.f;
          const float oz = ok ? O.z / L : 0.f, ow = ok ? O.w / L : 0.f;
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + d) =
              make_uint2(pack_bf16x2(ox, oy), pack_bf16x2(oz, ow));
        } else {
          const size_t pi = kSplit<MODE> ? row * p.np_stride + it.part + (it.w.pre ? 0 : p.slot_off)
                                         : row * p.NP + it.part;
          // bf16 partial output (the result is rounded to bf16 anyway);
          // streaming store: the reduce kernel reads the partial once.
          // Partial writes interleaved with the K/V reads cost far more
          // HBM time than their bytes, so they are kept small.
          const u32x2_t o4 = {pack_bf16x2(O.x, O.y), pack_bf16x2(O.z, O.w)};
          uint16_t* pa = reinterpret_cast<uint16_t*>(p.ws_acc) + pi * D + d;
          if (fused) {
            // agent scope: the merging workgroup may sit on another XCD
            __hip_atomic_store(reinterpret_cast<unsigned long long*>(pa),
                               __builtin_bit_cast(unsigned long long, o4), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (d == 0) {
              __hip_atomic_store(p.ws_m + pi, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(p.ws_l + pi, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          } else {
            __builtin_nontemporal_store(o4, reinterpret_cast<u32x2_t*>(pa));
            if (d == 0) {
              p.ws_m[pi] = M;
              p.ws_l[pi] = L;
            }
          }
        }
      }
    }
    if (fused) {
      if (merge_prev) {
        merge_group<D, MODE>(p, pg, pnp);
        if (tid == 0)
          __hip_atomic_store(p.arrivals + pg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // This item's partials are counted in at the next item's last step.
      const bool split = it.live && it.n > p.P;
      pg = __builtin_amdgcn_readfirstlane(split ? it.w.seq * Y + it.w.kvh * p.chunks + it.w.r0 / 16
                                                : -1);
      pnp = __builtin_amdgcn_readfirstlane((it.n + p.P - 1) / p.P);
    }
    __syncthreads();  // Z: merge reads of s_raw / s_m / s_l and s_next done

    // The claimed item starts as the prologue starts the first: block ids
    // and Q to LDS (every read of the previous item's was before barrier
    // X), then, at the loop's top, every wave's first chunk.
    cur = nn;
    it = ni;
    new_row = row_nn;
    if (cur < total) {
      store_tab(tab_nn, s_wtab[wave], lane);
      store_q<CT, D>(q_nn, it.w, s_qf, tid);
      __syncthreads();
      prime = true;
    }
  }
  // The last item's partials.
  if (pg >= 0) {
    wait_stores_complete();
    if (lane == 0) s_red[wave] = arrive(p, pg) == kNW * pnp - 1;
    __syncthreads();
    if (s_red[0] | s_red[1] | s_red[2] | s_red[3]) {
      merge_group<D, MODE>(p, pg, pnp);
      if (tid == 0)
        __hip_atomic_store(p.arrivals + pg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // The last workgroup to finish returns the counters to zero.
  if (tid == 0 && atomicAdd(done_ctr, 1) == (int)gridDim.x - 1) {
    for (int x = 0; x < 8; ++x) atomicExch(p.sched + x * kCounterStride, 0);
    atomicExch(shared_ctr, 0);
    atomicExch(done_ctr, 0);
  }
}

// Workgroups of a persistent launch: as many as are resident at once (CUs x
// the kernel's occupancy, a multiple of the 8 XCDs), never more than items;
// *young_from is the first workgroup that runs only its first item.  The
// occupancy query runs once per kernel variant and device.
template <typename CT, int D, int BS, bool SCAN, int MODE>
unsigned persistent_grid(long long items, int* young_from) {
  constexpr int kMaxDev = 64;
  static int resident[kMaxDev];  // per device, for this kernel variant only
  static int cu_count[kMaxDev];
  const void* kern = reinterpret_cast<const void*>(decode_mfma_kernel<CT, D, BS, SCAN, MODE>);
  int dev = 0;
  int per_dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDev) {
    per_dev = resident[dev];
    cus = cu_count[dev];
  }
  if (per_dev <= 0) {
    int blocks = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kern, kNW * 64, 0) != hipSuccess ||
        blocks <= 0)
      blocks = 1;
    per_dev = (cus * blocks + 7) / 8 * 8;
    if (dev >= 0 && dev < kMaxDev) {
      resident[dev] = per_dev;
      cu_count[dev] = cus;
    }
  }
  // Workgroups are dispatched one per CU at a time, so with three or more
  // per CU the last `cus` of a full grid are each the youngest on their CU.
  *young_from = per_dev > 2 * cus ? per_dev - cus : per_dev;
  return (unsigned)(per_dev < items ? per_dev : items);
}

template <typename CT, int D, int BS, int MODE>
hipError_t launch_mode(const DecodeArgs& a, const MfmaParams& p, long long items) {
  // FP8 caches keep every workgroup claiming: with more vector work per
  // byte the youngest workgroup on a CU keeps a larger share (about 60% of
  // the oldest's rate, against a third with bf16 caches) and still adds
  // throughput after its first item.
  constexpr bool kStopYoung = Geometry<CT, D>::ELEM == 2;
  MfmaParams pl = p;
  // The sorted item order packs a context length into 31 - kSeqBits bits.
  if (a.S <= kMaxScanSeqs && a.max_ctx < (1 << (31 - kSeqBits))) {
    const unsigned grid = persistent_grid<CT, D, BS, true, MODE>(items, &pl.young_from);
    if (!kStopYoung) pl.young_from = (int)grid;
    hipLaunchKernelGGL((decode_mfma_kernel<CT, D, BS, true, MODE>), dim3(grid), dim3(kNW * 64), 0,
                       a.stream, pl);
  } else {
    const unsigned grid = persistent_grid<CT, D, BS, false, MODE>(items, &pl.young_from);
    if (!kStopYoung) pl.young_from = (int)grid;
    hipLaunchKernelGGL((decode_mfma_kernel<CT, D, BS, false, MODE>), dim3(grid), dim3(kNW * 64),
                       0, a.stream, pl);
  }
  return hipGetLastError();
}

template <typename CT, int D, int BS>
hipError_t launch_bs(const DecodeArgs& a) {
  MfmaParams p;
  p.q = a.q; p.kc = a.key_cache; p.vc = a.value_cache; p.ks = a.key_scale; p.vs = a.value_scale;
  p.tables = a.tables; p.lens = a.lens; p.out = a.out;
  p.ws_m = a.ws_m; p.ws_l = a.ws_l; p.ws_acc = a.ws_acc; p.sched = a.sched;
  p.arrivals = a.arrivals;
  p.fused = a.fused ? 1 : 0;
  p.S = a.S; p.H = a.H; p.H_kv = a.H_kv; p.G = a.H / a.H_kv; p.M = a.M;
  p.chunks = (a.M * p.G + 15) / 16;
  p.max_blocks = a.max_blocks; p.P = a.P; p.NP = a.NP;
  p.max_ctx = a.max_ctx;
  p.tab_off = a.len_off / a.bs;
  p.len_off = a.len_off; p.prefix = a.prefix_rows; p.slot_off = a.slot_off;
  p.pre_chunks = (a.S * p.G + 15) / 16;
  p.pre_slots = a.prefix_rows > 0 ? a.prefix_slots : 0;
  p.pre_items = a.H_kv * p.pre_chunks * p.pre_slots;
  p.np_stride = a.np_stride > 0 ? a.np_stride : a.NP;
  p.force_partial = a.force_partial ? 1 : 0;
  // FP8 scales are [num_blocks][H_kv] floats: a block's KV heads share their
  // scale lines, which one XCD's L2 then serves to all of them (with a KV
  // head per queue every XCD fetched every line, 6% of the traffic).  The
  // split-prefix kind keeps a KV head per queue: there the heads' shared
  // prefix blocks are what the L2 serves.
  p.group_major = Geometry<CT, D>::ELEM == 1 && !(a.prefix_rows > 0 || a.len_off > 0 ||
                                                  a.force_partial);
  p.new_k = a.new_k; p.new_v = a.new_v; p.slots = a.slots; p.num_slots = a.num_slots;
  p.scale_log2 = a.scale * kLog2e;
  const long long items = (long long)a.H_kv * p.chunks * a.S * a.NP + p.pre_items;
  if (a.new_k) {  // write fused into a one-token decode: copies, so bf16 caches only
    if constexpr (Geometry<CT, D>::ELEM == 2)
      return launch_mode<CT, D, BS, kModeDecodeWrite>(a, p, items);
    return hipErrorInvalidValue;
  }
  if (a.prefix_rows > 0 || a.len_off > 0 || a.force_partial)
    return launch_mode<CT, D, BS, kModeSplitPrefix>(a, p, items);
  return a.M > 1 ? launch_mode<CT, D, BS, kModeCausal>(a, p, items)
                 : launch_mode<CT, D, BS, kModeDecode>(a, p, items);
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

// Every bf16-query decode runs here, one head per KV head included: the
// score and P V products cost the same matrix-core issue for 1..16 heads and
// the kernel stays HBM-bound.  fp32 queries keep the vector-ALU kernel.
bool decode_mfma_supported(const DecodeArgs& a) {
  return a.q_dtype == PKV_BF16 && (a.cache_dtype == PKV_BF16 || a.cache_dtype == PKV_FP8_E4M3) &&
         (a.P + a.bs - 1) / a.bs <= kMaxTable;
}

hipError_t launch_decode_mfma(const DecodeArgs& a) {
  if (a.cache_dtype == PKV_BF16) return launch_c<BF16>(a);
  return launch_c<FP8>(a);
}

}  // namespace pkv
