// Pieces shared by the attention kernels: parameters, plan access, LDS tile
// staging.  MFMA layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand: lane l holds A[i = l%32][k = 8*(l/32) .. +7]
//   B operand: lane l holds B[k = 8*(l/32) .. +7][j = l%32]
//   C result : lane l holds C[i = 8*(r/4) + 4*(l/32) + r%4][j = l%32], r = 0..15
// Score tiles are kept with the query as the lane index j, so softmax row
// statistics are per lane (plus one exchange between the two half-waves), and
// an accumulator reused as the next product's operand keeps the same
// permutation of its contraction index on both operands.
#pragma once
#include "cpthd_device.h"

namespace cpthd {

struct AttnParams {
  int T, S, cp, rank, strategy, Hq, Hkv, D, G, num_docs;
  int num_cu;         // compute units of the device (the plan's split rule balances over them)
  int qsplit;         // 1: query tiles may be split (their work-groups cannot fill the device)
  float scale;        // softmax scale
  float scale_log2;   // softmax scale * log2(e)
};

// A plan is usable iff it was built for exactly these arguments and this
// workspace layout (the plan kernel that ran before the attention kernel in
// the same call also checked the cu arrays it was built from).  Every field is
// compared (bitwise &, no short circuit), so the header is read in a few wide
// loads instead of a chain of dependent ones.
__device__ inline bool plan_matches(const PlanHeader* hp, const AttnParams& p, const PlanLayout& lay) {
  const PlanHeader h = *hp;
  return (h.valid == 1) & (h.magic == kPlanMagic) & (h.version == kPlanVersion) & (h.T == p.T) & (h.S == p.S) &
         (h.cp == p.cp) & (h.rank == p.rank) & (h.strategy == p.strategy) & (h.Hq == p.Hq) & (h.Hkv == p.Hkv) &
         (h.D == p.D) & (h.num_docs == p.num_docs) & (h.num_cu == p.num_cu) & (h.max_qtiles == (int)lay.max_qtiles) &
         (h.max_kvtiles == (int)lay.max_kvtiles) & (h.max_docs == (int)lay.max_docs) &
         (h.max_parts == (int)lay.max_parts);
}

// The part fields of a tile entry: a whole tile (slot -1, one part), or part
// `part` of `nparts` >= 2 whose partial slots lie inside the workspace's.
__device__ inline bool parts_ok(int slot, int part, int nparts, const PlanLayout& lay) {
  return ((slot == -1) & (part == 0) & (nparts == 1)) |
         ((slot >= 0) & (nparts >= 2) & (part >= 0) & (part < nparts) & (slot <= (int)lay.max_parts - nparts));
}

// A document's segments lie inside the rank's local rows and its slot inside
// [0, T); under DualChunkSwap its two chunks are equal and adjacent in local
// order, which keeps every row of the all-gathered map (AgMap) below T.
__device__ inline bool docseg_ok(const DocSeg& d, const AttnParams& p) {
  const bool base = (d.ds >= 0) & (d.ve >= d.ds) & (d.ve <= p.T) & (d.na >= 0) & (d.nb >= 0) &
                    ((d.na == 0) | ((d.la >= 0) & (d.la <= p.S - d.na))) &
                    ((d.nb == 0) | ((d.lb >= 0) & (d.lb <= p.S - d.nb)));
  const bool dcs = (p.strategy != kDCS) | ((d.nb == d.na) & (d.lb == d.la + d.na) &
                                            (d.ds <= p.T - 2 * p.cp * d.na));
  return base & dcs;
}

// Check a query tile descriptor against the tensors' extents (bitwise, so
// its fields load together).
__device__ inline bool check_qtile(const QTile& t, const AttnParams& p, const PlanLayout& lay) {
  return (t.lrow0 >= 0) & (t.ntok >= 0) & (t.lrow0 <= p.S - t.ntok) & (t.ds >= 0) & (t.ds <= p.T) &
         (t.kv_end >= t.ds) & (t.kv_end <= p.T) & (t.p0 >= 0) & (t.p0 <= p.T - t.ntok) & (t.doc >= 0) &
         (t.doc < p.num_docs) & (t.s0 >= 0) & (t.s1 >= t.s0) & parts_ok(t.slot, t.part, t.nparts, lay);
}

// The start of every attention work-group: is the plan the one built for these
// arguments, is the work-group's tile in it, and is the tile sound?  Evaluated
// without short circuits and decided by one branch, so the header and the tile
// are read in one round of loads.  A mismatched plan or an unsound tile sets the
// plan bit of the device status; a tile past the plan's count is only surplus.
__device__ inline bool tile_usable(bool plan_ok, bool in_range, bool tile_ok, int32_t* status) {
  if (plan_ok & in_range & tile_ok) return true;
  if (threadIdx.x == 0 && status && (!plan_ok || (in_range && !tile_ok))) atomicOr(status, kDevPlan);
  return false;
}

// Row of the rank-major all-gathered K/V buffer (rank 0's local rows, then
// rank 1's, ...) that holds physical token p.  A partition unit (one document
// under DualChunkSwap, the whole buffer under the packed strategy) starting at
// physical token u0 is cut into 2*cp chunks of c tokens; rank j < cp holds
// chunk j at local rows lb.., and chunk 2cp-1-j right after it at lb + c..,
// where lb is the unit's first local row (the same on every rank).  The chunk
// index comes from a float reciprocal plus one correction step: p - u0 < 2^31
// and the quotient is below 2*cp, so the estimate is off by at most one.
struct AgMap {
  int u0, c, lb, S, cp;
  float rc;
  __device__ inline int row(int p) const {
    const int pos = p - u0;
    const int j0 = (int)((float)pos * rc);
    const int o0 = pos - j0 * c;
    const int j = o0 < 0 ? j0 - 1 : (o0 >= c ? j0 + 1 : j0);
    const int off = o0 < 0 ? o0 + c : (o0 >= c ? o0 - c : o0);
    const bool first = j < cp;
    return (first ? j : 2 * cp - 1 - j) * S + lb + (first ? off : c + off);
  }
  // chunk j holding p (p >= u0) and its first token
  __device__ inline void chunk_of(int p, int& j, int& start) const {
    const int pos = p - u0;
    const int j0 = (int)((float)pos * rc);
    const int o0 = pos - j0 * c;
    j = o0 < 0 ? j0 - 1 : (o0 >= c ? j0 + 1 : j0);
    start = u0 + j * c;
  }
};

// The chunk the key steps of one tile have reached (keys only move forward).
struct AgCursor {
  int j, start;
};

// The map of a document's keys (contiguous strategy: the identity, c = S).
__device__ inline AgMap ag_map(const DocSeg& d, const AttnParams& p) {
  AgMap m;
  m.S = p.S;
  m.cp = p.cp;
  if (p.strategy == kDCS) {
    m.u0 = d.ds;
    m.c = d.na;
    m.lb = d.la;
  } else {
    m.u0 = 0;
    m.c = p.strategy == kPacked ? p.S / 2 : p.S;
    m.lb = 0;
  }
  // the map is the same for every lane: keep it (and whatever is derived from it) in scalar registers
  m.u0 = __builtin_amdgcn_readfirstlane(m.u0);
  m.c = __builtin_amdgcn_readfirstlane(m.c);
  m.lb = __builtin_amdgcn_readfirstlane(m.lb);
  m.rc = m.c > 0 ? 1.0f / (float)m.c : 0.f;
  return m;
}

// ---------------------------------------------------------------------------
// LDS tiles of 64 rows x DP bf16, staged straight from global memory
// ---------------------------------------------------------------------------
// Rows are DP + 8 elements apart (one 16-byte padding slot per row): 16
// consecutive rows of a 16-byte-per-lane read then fall on distinct banks.
// Tiles that are also read through the transpose read store logical row q at
// row rho(q) (a 4x4 transpose inside each block of 16 rows), so the 4 logical
// rows one transpose read touches sit 4 rows apart, on disjoint bank spans.
__device__ inline int rho(int q) { return (q & ~15) | ((q & 3) << 2) | ((q >> 2) & 3); }

template <int DP, bool PERM>
struct LdsTile {
  static constexpr int C = DP / 8;                 // 16-byte chunks of data per row
  static constexpr int SPR = C + 1;                // 16-byte slots per row
  static constexpr int STRIDE = DP + 8;            // elements per row
  static constexpr int ELEMS = 64 * STRIDE;
  static constexpr int NLOAD = SPR;                // 1 KiB wave loads per tile (64 * SPR slots)
  __device__ static inline int row(int q) { return PERM ? rho(q) : q; }
};

// Per-lane offsets of one work-group's direct loads of an LdsTile: of NW
// waves, wave w issues loads u = w, w + NW, ...; lane l of load u fills 16-byte
// slot 64u + l.  Padding slots, columns >= D and rows without data get an
// offset past the buffer's range, which the hardware turns into zeros.
template <int DP, bool PERM, int NW = 4>
struct TileLoader {
  using L = LdsTile<DP, PERM>;
  static constexpr int NLW = (L::NLOAD + NW - 1) / NW;   // loads per wave
  uint32_t voff[NLW];

  // rowoff(q): byte offset of logical row q from the descriptor base, or < 0 for a zero row
  template <typename RowOff>
  __device__ inline void init(int wave, int lane, int D, RowOff rowoff) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int u = wave + NW * i;
      const int slot = 64 * u + lane;
      const int R = slot / L::SPR, ch = slot - R * L::SPR;
      uint32_t off = 0x80000000u;
      if (u < L::NLOAD && ch < L::C && ch * 8 < D) {
        const int64_t ro = rowoff(PERM ? rho(R) : R);
        if (ro >= 0) off = (uint32_t)(ro + 16 * ch);
      }
      voff[i] = off;
    }
  }
  // Loads whose rows move from step to step: each load's logical row (-1 for
  // a slot without data) and column byte offset, fixed per lane; set_rows()
  // then derives the offsets from a per-step row offset function.
  int srow[NLW];
  uint32_t scol[NLW];
  __device__ inline void init_slots(int wave, int lane, int D) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int u = wave + NW * i;
      const int slot = 64 * u + lane;
      const int R = slot / L::SPR, ch = slot - R * L::SPR;
      const bool ok = u < L::NLOAD && ch < L::C && ch * 8 < D;
      srow[i] = ok ? (PERM ? rho(R) : R) : -1;
      scol[i] = 16u * (uint32_t)ch;
    }
  }
  // off(r): byte offset of logical row r >= 0 (any r: the caller selects), valid(r): row has data
  template <typename Off, typename Valid>
  __device__ inline void set_rows(Off off, Valid valid) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int r = srow[i];
      const uint32_t o = off(r < 0 ? 0 : r) + scol[i];
      voff[i] = (r >= 0 && valid(r)) ? o : 0x80000000u;
    }
  }
  // rows [0, nvalid) of a step whose rows follow each other from a scalar offset on: r * row_bytes + col;
  // rows from nvalid on read as zero
  __device__ inline void set_rows_linear(uint32_t row_bytes, uint32_t col, int nvalid) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int r = srow[i];
      voff[i] = (r >= 0 && r < nvalid) ? (uint32_t)r * row_bytes + col + scol[i] : 0x80000000u;
    }
  }
  // the same over two runs of consecutive rows: rows [0, split) from row a0 on, rows [split, nvalid) from
  // row a1 on (absolute row offsets, used with a zero scalar offset)
  __device__ inline void set_rows_two(uint32_t row_bytes, uint32_t col, int nvalid, int split, int a0, int a1) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int r = srow[i];
      const int row = r < split ? a0 + r : a1 + (r - split);
      voff[i] = (r >= 0 && r < nvalid) ? (uint32_t)row * row_bytes + col + scol[i] : 0x80000000u;
    }
  }
  __device__ inline void issue(__amdgpu_buffer_rsrc_t rsrc, uint16_t* tile, uint32_t soff, int wave) const {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int u = wave + NW * i;
      if (u < L::NLOAD)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(tile + 512 * u), 16,
                                                 voff[i], soff, 0, 0);
    }
  }
};

// Buffer descriptor over `bytes` bytes from `base` (raw, no stride); loads past
// the range read as zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 4-byte direct load per lane into LDS[base + 4*lane].
__device__ inline void lds_load_dword(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

// Wait for this wave's direct-to-LDS loads, then for the whole work-group.
__device__ inline void lds_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Operand with the contraction index along a row: lane l gets
// X[q][k0 + 8*(l/32) .. +7] of logical row q (one 16-byte LDS read).
template <int DP, bool PERM>
__device__ inline bf16x8 lds_row8(const uint16_t* tile, int q, int k0, int half) {
  using L = LdsTile<DP, PERM>;
  return *reinterpret_cast<const bf16x8*>(tile + L::row(q) * L::STRIDE + k0 + 8 * half);
}

// Operand whose lane index runs along the columns, with two gfx950 transpose
// reads (ds_read_b64_tr_b16): lane l gets X[q0 + s][c0 + l%32] in slots
// s = 0..3 and X[q1 + s][c0 + l%32] in slots 4..7 (q0, q1 multiples of 4).
// Within each 16-lane group the hardware hands output lane j, slot s, element
// j%4 of the 8 bytes addressed by lane 4s + j/4, so lane i addresses logical
// row q + i/4, columns c + 4*(i%4) .. +3.
template <int DP, bool PERM>
__device__ inline bf16x8 lds_tr8(const uint16_t* tile, int q0, int q1, int c0) {
  using L = LdsTile<DP, PERM>;
  const int l = threadIdx.x & 63, sub = l & 15;
  const int col = c0 + 16 * ((l >> 4) & 1) + 4 * (sub & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + L::row(q0 + (sub >> 2)) * L::STRIDE + col));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + L::row(q1 + (sub >> 2)) * L::STRIDE + col));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Scheduling hint for a run of N MFMAs that consume R LDS reads each, in
// order: keep the reads of AHEAD products in flight ahead of the products, so
// a product waits for reads issued AHEAD products earlier rather than for the
// ones just issued.  EXTRA further reads (operands read once, such as an
// accumulator's start values) go with the first group.  Place it after the
// run's code.
template <int N, int AHEAD, int R = 1, int EXTRA = 0>
__device__ inline void pipeline_reads_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * R + EXTRA, 0);   // LDS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Eight accumulator entries r0..r0+7 of a 32x32 result as a bf16 operand.
__device__ inline bf16x8 acc_to_bf16(const f32x16& a, int r0) {
  u32x4 v;
  v.x = pack_bf16x2(a[r0 + 0], a[r0 + 1]);
  v.y = pack_bf16x2(a[r0 + 2], a[r0 + 3]);
  v.z = pack_bf16x2(a[r0 + 4], a[r0 + 5]);
  v.w = pack_bf16x2(a[r0 + 6], a[r0 + 7]);
  return as_bf16x8(v);
}

// Direct loads of the K and V rows of keys [kb, kb + 64) of kv head kvh into
// one step's tiles (same rows, same lane offsets, two descriptors); keys from
// kend on read as zero.  Physical order: the descriptors start at the
// document's first key ds and the lane offsets were set once, so a step only
// moves the scalar offset.  Rank-major all-gathered order (AG): the
// descriptors cover all T rows (T * row_bytes < 2^31).  A step whose keys lie
// in one chunk of the partition reads consecutive gathered rows, from a scalar
// offset the cursor gives; a step over two chunks picks one of two scalar row
// bases per lane; only a step over more chunks (chunks under 64 keys) maps
// every lane's row through the map.
template <bool AG, int DP, int NW, bool WITH_V = true>
__device__ inline void issue_kv_step(TileLoader<DP, true, NW>& ld, __amdgpu_buffer_rsrc_t krs,
                                     __amdgpu_buffer_rsrc_t vrs, const AgMap& agm, AgCursor& cur, int kb, int ds,
                                     int kend, uint32_t row_bytes, int kvh, int D, int wave, int lane, uint16_t* Kn,
                                     uint16_t* Vn) {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer-resource builtins: device pass only
  if constexpr (AG) {
    const uint32_t col = (uint32_t)kvh * D * 2;
    const int nvalid = min(kKvStep, kend - kb);
    // move the cursor to the chunk holding kb (at most 2cp chunks in a unit)
    for (int g = 0; g < 2 * agm.cp && kb >= cur.start + agm.c; ++g) {
      cur.start += agm.c;
      ++cur.j;
    }
    // gathered row of the first token of chunk j
    auto chunk_row = [&](int j) __attribute__((always_inline)) {
      const bool first = j < agm.cp;
      return (first ? j : 2 * agm.cp - 1 - j) * agm.S + agm.lb + (first ? 0 : agm.c);
    };
    if (kb >= cur.start && kb + nvalid <= cur.start + agm.c) {
      // the step's keys lie in one chunk, so they are consecutive rows of the gathered buffer
      const int row0 = chunk_row(cur.j) + (kb - cur.start);
      ld.set_rows_linear(row_bytes, col, nvalid);
      ld.issue(krs, Kn, (uint32_t)row0 * row_bytes, wave);
      if constexpr (WITH_V) ld.issue(vrs, Vn, (uint32_t)row0 * row_bytes, wave);
    } else if (kb >= cur.start && kb + nvalid <= cur.start + 2 * agm.c && cur.j + 1 < 2 * agm.cp) {
      // two chunks: two runs of consecutive gathered rows
      const int split = cur.start + agm.c - kb;
      ld.set_rows_two(row_bytes, col, nvalid, split, chunk_row(cur.j) + (kb - cur.start), chunk_row(cur.j + 1));
      ld.issue(krs, Kn, 0, wave);
      if constexpr (WITH_V) ld.issue(vrs, Vn, 0, wave);
    } else {
      const int last = kend - 1;
      ld.set_rows([&](int r) __attribute__((always_inline)) { return (uint32_t)agm.row(min(kb + r, last)) * row_bytes + col; },
                  [&](int r) __attribute__((always_inline)) { return kb + r < kend; });
      ld.issue(krs, Kn, 0, wave);
      if constexpr (WITH_V) ld.issue(vrs, Vn, 0, wave);
    }
  } else {
    const uint32_t soff = (uint32_t)(kb - ds) * row_bytes;
    ld.issue(krs, Kn, soff, wave);
    if constexpr (WITH_V) ld.issue(vrs, Vn, soff, wave);
  }
#endif
}

// ---------------------------------------------------------------------------
// V^T tiles of the forward: DP rows (head-dim columns) x 64 keys
// ---------------------------------------------------------------------------
// The workspace's V^T rows hold each 16-key group of a row in the order
// 0-3, 8-11, 4-7, 12-15, which is the order of the contraction index in the
// forward's P^T operand (the scores' accumulator layout): half-wave h then
// reads its 8 keys of a 16-key slice as one 16-byte row read at column 8h.
// Rows are 64 + 8 elements apart, so 8 consecutive rows of a 16-byte read fall
// on distinct banks.
template <int DP>
struct LdsTileVT {
  static constexpr int SPR = 9;                    // 16-byte slots per row: 8 of keys, 1 of padding
  static constexpr int STRIDE = 72;                // elements per row
  static constexpr int ELEMS = DP * STRIDE;
  static constexpr int NLOAD = DP * SPR / 64;      // 1 KiB wave loads per tile
  static_assert(DP * SPR % 64 == 0, "whole wave loads");
};

// Position of key k (0..15) of a 16-key group in a V^T row.
__host__ __device__ inline int vt_pos16(int k) { return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Direct loads of one step's V^T tile: lane offsets fixed per lane (row d,
// 16-byte chunk), the step's first column in the scalar offset; rows >= D and
// padding slots read as zero.
template <int DP, int NW>
struct VTLoader {
  using L = LdsTileVT<DP>;
  static constexpr int NLW = (L::NLOAD + NW - 1) / NW;
  uint32_t voff[NLW];
  __device__ inline void init(int wave, int lane, int D, uint32_t row_bytes) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int u = wave + NW * i;
      const int slot = 64 * u + lane;
      const int R = slot / L::SPR, ch = slot - R * L::SPR;
      voff[i] = (u < L::NLOAD && ch < 8 && R < D) ? (uint32_t)R * row_bytes + 16u * ch : 0x80000000u;
    }
  }
  __device__ inline void issue(__amdgpu_buffer_rsrc_t rsrc, uint16_t* tile, uint32_t soff, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int u = wave + NW * i;
      if (u < L::NLOAD)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(tile + 512 * u), 16,
                                                 voff[i], soff, 0, 0);
    }
#endif
  }
};

// Host helpers shared by the plan, forward and backward entry points.
int check_attn_args(int64_t T, int64_t capacity, int32_t cp, int32_t rank, int32_t strategy, int32_t num_docs,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t wl, int32_t wr, const void* ws,
                    size_t ws_bytes, PlanLayout& lay, AttnParams& prm);
int64_t qtile_grid(const AttnParams& prm, const PlanLayout& lay);
int64_t kvtile_grid(const AttnParams& prm, const PlanLayout& lay);
// The compute units of the current device (cached per device), and whether
// query tiles may be split: only when the whole query tiles of the call, times
// the kv heads, are fewer work-groups than compute units.  Splitting then adds
// parallelism; on a full device the merge's launch and partial traffic cost
// more than the balance gains.
int device_cus(AttnParams& prm);
// Work-groups of a merge kernel over one list of split tiles (one per split
// tile and kv head; a split tile has at least two parts).
inline int64_t split_grid(const AttnParams& prm, const PlanLayout& lay) { return lay.max_parts / 2 * prm.Hkv; }
// Launch the plan kernel: build the plan (ensure = false), or make sure the
// workspace holds the plan of these arguments and cu arrays, rebuilding it
// only when it does not (ensure = true).  Event slot `slot` times it.
int launch_plan(const int32_t* cu_a, const int32_t* cu_p, const AttnParams& prm, char* ws, const PlanLayout& lay,
                bool ensure, int32_t* status, hipStream_t stream, hipEvent_t* ev, int nev, int slot);

}  // namespace cpthd
