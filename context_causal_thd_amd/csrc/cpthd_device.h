// Device-side definitions shared by the cpthd kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpthd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kDCS = 0;      // DualChunkSwap
constexpr int kContig = 1;   // NO_LOAD_BALANCE
constexpr int kPacked = 2;   // PACKED_SUPER_SEQUENCE

// status bits (mirror the public header)
constexpr int kDevCuOrder = 1, kDevCuTotal = 2, kDevDcsDivisible = 4, kDevActual = 8, kDevPlan = 16,
              kDevIndex = 32, kDevDocBytes = 64;

// ---------------------------------------------------------------------------
// tiling constants shared by the plan and the attention kernels
// ---------------------------------------------------------------------------
#ifndef CPTHD_ROWS_PER_WG
#define CPTHD_ROWS_PER_WG 256
#endif
constexpr int kRowsPerWG = CPTHD_ROWS_PER_WG;   // query rows (token x head pairs) per fwd / dq work-group
constexpr int kQWaves = kRowsPerWG / 32;        // fwd / dq waves (one 32-row MFMA block each)
constexpr int kQMinBlocks = kQWaves >= 8 ? 1 : 8 / kQWaves;   // work-groups per CU the launch bounds ask for
// Register-budget hint: a kernel that runs as one work-group of W waves per CU
// has W/4 waves per SIMD and never more, so the scheduler may spend the whole
// 512/(W/4) registers on latency hiding instead of chasing occupancy it cannot get.
#ifndef CPTHD_WAVES_HINT
#define CPTHD_WAVES_HINT 1
#endif
#if CPTHD_WAVES_HINT
#define CPTHD_WAVES_PER_EU(n) __attribute__((amdgpu_waves_per_eu(n, n)))
#else
#define CPTHD_WAVES_PER_EU(n)
#endif
constexpr int kKeysPerWG = 128;   // keys per dk/dv work-group
constexpr int kKvStep = 64;       // keys per inner step of the fwd / dq kernels
constexpr int kQChunk = 64;       // query rows per inner step of the dk/dv kernel
constexpr int kCostBins = 2048;   // counting-sort bins for longest-first ordering
constexpr int kPlanMagic = 0x43505444;  // "CPTD"
constexpr int kPlanVersion = 3;

// Query tile: `ntok` consecutive local rows of one segment (a run of the rank's
// rows inside one document), all q heads of one kv group.  Keys [ds, kv_end),
// visited in 64-key steps [s0, s1) of that range: the whole range, or one part
// of a tile the plan split so that no work-group holds far more than its share
// of the launch.  The parts of a split tile write their partial results to
// partial slots slot .. slot + nparts - 1; a merge kernel, launched after the
// attention kernel, combines them in part order.
struct QTile {
  int32_t lrow0;   // first local row
  int32_t ntok;    // rows (tokens) in the tile
  int32_t p0;      // physical token of the first row
  int32_t ds;      // document start (physical)
  int32_t kv_end;  // one past the last key any actual row of the tile sees
  int32_t ve;      // end of the document's actual tokens
  int32_t cost;    // steps s1 - s0
  int32_t doc;
  int32_t s0, s1;  // the key steps this entry visits
  int32_t slot;    // first partial slot of the split tile, -1 when the tile is whole
  int32_t part, nparts;
  int32_t vt;      // column of key ds in the workspace's V^T rows
  int32_t pad_[2];
};
static_assert(sizeof(QTile) == 64, "query tile is 64 bytes");

// Key tile of one document: keys [k0, k0 + nkeys) (inside the document's slot),
// and of the rank's query chunks that see it, those with index [c0, c1) in the
// order the kernel visits them (all of them, or one part of a split tile, as
// for query tiles).
struct KVTile {
  int32_t k0;
  int32_t nkeys;
  int32_t doc;
  int32_t cost;    // chunks c1 - c0
  int32_t c0, c1;
  int32_t slot, part, nparts;
  int32_t pad_[3];
};
static_assert(sizeof(KVTile) == 48, "key tile is 48 bytes");

// A split tile, for the merge kernels: its first partial slot, its part count,
// and the tile's rows (query tiles: a = lrow0, b = ntok, c = p0, d = ve) or
// keys (key tiles: a = k0, b = nkeys, c = doc).
struct SplitTile {
  int32_t slot, nparts;
  int32_t a, b, c, d;
  int32_t pad_[2];
};

// The rank's rows of one document: up to two segments (DualChunkSwap chunks
// r and 2cp-1-r; contiguous: one), each `n` local rows from local row `l`
// at physical token `p`.
struct DocSeg {
  int32_t ds, ve, la, pa, na, lb, pb, nb;
};

struct PlanHeader {
  int32_t magic, version, valid;
  int32_t T, S, cp, rank, strategy, Hq, Hkv, D, G, num_docs;
  int32_t bm_tok;               // tokens per query tile
  int32_t n_qtiles, n_kvtiles;  // entries of the tile lists (parts included)
  int32_t max_qtiles, max_kvtiles, max_docs, max_parts;
  int32_t num_cu;               // compute units the split rule balanced the work over
  int32_t q_part_steps, kv_part_chunks;   // part sizes of split tiles (0: nothing split)
  int32_t n_qsplit, n_kvsplit;            // split tiles (entries of the merge lists)
  int32_t n_kvwhole;                      // key tiles before splitting (they tile the V^T columns)
  int32_t pad_[38];
};
static_assert(sizeof(PlanHeader) == 256, "plan header is 256 bytes");

// Workspace layout (byte offsets), identical on host and device.
struct PlanLayout {
  size_t qtiles, qtiles_tmp, kvtiles, kvtiles_tmp, docs, cu_copy, qsplit, kvsplit, qpart, kvpart, delta, lse2, total;
  size_t vt;          // V^T rows (when has_vt): [Hkv][D][vt_cols] bf16
  bool has_vt;
  int64_t vt_cols;    // 128 columns per key tile of the list before splitting
  int64_t max_qtiles, max_kvtiles, max_docs;
  int64_t max_parts;                     // partial slots of each tile list (its entries hold up to that many more)
  int64_t qpart_stride, kvpart_stride;   // floats per (partial slot, kv head)
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline int tokens_per_qtile(int G) { return kRowsPerWG / G; }

// The head dimension the kernels are instantiated for.
__host__ __device__ inline int padded_head_dim(int D) { return D <= 32 ? 32 : (D <= 64 ? 64 : 128); }

// Partial slots the default workspace holds: 256 / Hkv, at least 8, and at
// most one per 128 tokens of capacity (a small buffer has no long tiles to
// split).  One slot holds, per kv head, a query tile's 256 rows (output and
// softmax statistics) and a key tile's 128 keys (dK and dV) in fp32.
__host__ __device__ inline int default_split_parts(int Hkv, int64_t capacity) {
  const int n = 256 / Hkv > 8 ? 256 / Hkv : 8;
  return capacity / 128 < n ? (int)(capacity / 128) : n;
}

__host__ __device__ inline PlanLayout plan_layout(int64_t capacity, int cp, int Hq, int Hkv, int D, int max_docs,
                                                  int max_parts, bool with_vt) {
  PlanLayout L;
  const int G = Hq / Hkv;
  const int64_t S = capacity / cp;
  const int bm = tokens_per_qtile(G);
  const int64_t dp = padded_head_dim(D);
  L.max_docs = max_docs;
  L.max_parts = max_parts;
  const int64_t nq = (S + bm - 1) / bm + 2 * (int64_t)max_docs;          // whole query tiles
  const int64_t nkv = (capacity + kKeysPerWG - 1) / kKeysPerWG + (int64_t)max_docs;
  L.max_qtiles = nq + max_parts;
  L.max_kvtiles = nkv + max_parts;
  L.qpart_stride = (int64_t)kRowsPerWG * (dp + 4);   // per row: the output columns, then (max, sum) pairs
  L.kvpart_stride = (int64_t)kKeysPerWG * 2 * dp;    // per key: dK and dV columns
  size_t off = sizeof(PlanHeader);
  L.qtiles = off;       off = align_up(off + L.max_qtiles * sizeof(QTile), 256);
  L.qtiles_tmp = off;   off = align_up(off + nq * sizeof(QTile), 256);
  L.kvtiles = off;      off = align_up(off + L.max_kvtiles * sizeof(KVTile), 256);
  L.kvtiles_tmp = off;  off = align_up(off + nkv * sizeof(KVTile), 256);
  L.docs = off;         off = align_up(off + (size_t)max_docs * sizeof(DocSeg), 256);
  L.cu_copy = off;      off = align_up(off + 2 * ((size_t)max_docs + 1) * sizeof(int32_t), 256);
  L.qsplit = off;       off = align_up(off + (size_t)max_parts * sizeof(SplitTile), 256);
  L.kvsplit = off;      off = align_up(off + (size_t)max_parts * sizeof(SplitTile), 256);
  L.qpart = off;        off = align_up(off + (size_t)max_parts * Hkv * L.qpart_stride * sizeof(float), 256);
  L.kvpart = off;       off = align_up(off + (size_t)max_parts * Hkv * L.kvpart_stride * sizeof(float), 256);
  L.delta = off;        off = align_up(off + (size_t)S * Hq * sizeof(float), 256);
  L.lse2 = off;         off = align_up(off + (size_t)S * Hq * sizeof(float), 256);
  // V^T of the forward: one row per (kv head, head-dim column), the keys of
  // document i from column 128 * (its first key tile) on, each document's
  // columns padded to a multiple of 128 with zeros
  L.vt_cols = nkv * kKeysPerWG;
  L.has_vt = with_vt;
  L.vt = off;
  if (with_vt) off = align_up(off + (size_t)Hkv * D * L.vt_cols * 2, 256);
  L.total = off;
  return L;
}

// Whether the forward reads V^T rows written by a pass of its own instead of
// reading V through the transpose LDS read: only in builds with CPTHD_FWD_VT=1
// (measured slower: the V^T pass costs 2-6% of the forward and the forward
// itself does not gain), for head dim 64 or 128 (the V^T tile needs whole wave
// loads), with a kv head's rows inside one 32-bit buffer range.
#ifndef CPTHD_FWD_VT
#define CPTHD_FWD_VT 0
#endif
__host__ __device__ inline bool vt_wanted(int D, int64_t vt_cols) {
  return CPTHD_FWD_VT && D >= 64 && (int64_t)D * vt_cols * 2 < ((int64_t)1 << 31);
}

// The layout of a call with a workspace of ws_bytes: the V^T rows when they
// fit beside the plan, then the most partial slots, up to the default, that
// the rest holds (none when it holds only the plan itself).
inline PlanLayout call_layout(int64_t capacity, int cp, int Hq, int Hkv, int D, int max_docs, size_t ws_bytes) {
  const PlanLayout v0 = plan_layout(capacity, cp, Hq, Hkv, D, max_docs, 0, true);
  const bool vt = v0.total <= ws_bytes && vt_wanted(D, v0.vt_cols);
  int lo = 0, hi = default_split_parts(Hkv, capacity);
  if (plan_layout(capacity, cp, Hq, Hkv, D, max_docs, hi, vt).total > ws_bytes) {
    while (lo < hi) {   // the layout grows with the slot count
      const int mid = (lo + hi + 1) / 2;
      if (plan_layout(capacity, cp, Hq, Hkv, D, max_docs, mid, vt).total <= ws_bytes) lo = mid; else hi = mid - 1;
    }
    hi = lo;
  }
  return plan_layout(capacity, cp, Hq, Hkv, D, max_docs, hi, vt);
}

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
// The work-item's wave within its work-group, as a wave-uniform (scalar) value:
// everything derived from it (LDS tile bases, M0 for direct loads, row blocks)
// then lives in scalar registers instead of being kept per lane.
__device__ inline int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Work-group barrier over LDS only: waits for this wave's LDS accesses, not for its outstanding global loads, so
// direct-to-LDS prefetches into other buffers stay in flight across it.  (__syncthreads() also waits for every
// global memory operation of the wave.)  One asm statement with a memory clobber, so the compiler moves no
// memory access across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Reductions of x with the value of the lane 32 apart, the same bits in both
// lanes.  v_permlane32_swap (a VALU op, no LDS round trip) with x as both
// operands returns, in lanes 0-31, (own, lane + 32) and in lanes 32-63,
// (lane - 32, own) -- lane layout checked on gfx950.
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite)
__device__ inline uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Largest i in [0, n] with a[i] <= x, for a non-decreasing array a[0..n] with a[0] <= x.
__device__ inline int upper_index(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace cpthd
