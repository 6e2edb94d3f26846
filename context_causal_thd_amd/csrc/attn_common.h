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
  float scale;        // softmax scale
  float scale_log2;   // softmax scale * log2(e)
};

// A plan is usable iff it was built for exactly these arguments.
__device__ inline bool plan_matches(const PlanHeader* h, const AttnParams& p) {
  return h->valid == 1 && h->magic == kPlanMagic && h->version == kPlanVersion && h->T == p.T && h->S == p.S &&
         h->cp == p.cp && h->rank == p.rank && h->strategy == p.strategy && h->Hq == p.Hq && h->Hkv == p.Hkv &&
         h->D == p.D && h->num_docs == p.num_docs;
}

// Load a query tile descriptor and clamp it to the tensors' extents.
__device__ inline bool load_qtile(const char* ws, const PlanLayout& lay, int idx, const AttnParams& p, QTile& t) {
  t = reinterpret_cast<const QTile*>(ws + lay.qtiles)[idx];
  if (t.lrow0 < 0 || t.ntok < 0 || t.lrow0 > p.S - t.ntok) return false;
  if (t.ds < 0 || t.ds > p.T || t.kv_end < t.ds || t.kv_end > p.T || t.p0 < 0 || t.p0 > p.T - t.ntok) return false;
  return true;
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

// Eight accumulator entries r0..r0+7 of a 32x32 result as a bf16 operand.
__device__ inline bf16x8 acc_to_bf16(const f32x16& a, int r0) {
  u32x4 v;
  v.x = pack_bf16x2(a[r0 + 0], a[r0 + 1]);
  v.y = pack_bf16x2(a[r0 + 2], a[r0 + 3]);
  v.z = pack_bf16x2(a[r0 + 4], a[r0 + 5]);
  v.w = pack_bf16x2(a[r0 + 6], a[r0 + 7]);
  return as_bf16x8(v);
}

// Host helpers shared by the forward and backward entry points.
int check_attn_args(int64_t T, int64_t capacity, int32_t cp, int32_t rank, int32_t strategy, int32_t num_docs,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t wl, int32_t wr, const void* ws,
                    size_t ws_bytes, PlanLayout& lay, AttnParams& prm);
unsigned qtile_grid(const AttnParams& prm);

}  // namespace cpthd
