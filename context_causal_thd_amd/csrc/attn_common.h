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

// LDS row strides (in bf16 elements) of natural [row][DP] tiles.  kNat keeps
// 16 consecutive rows of a 16-byte-per-lane read on distinct banks; kTr puts
// the 4 rows that one transpose read touches on disjoint 16-bank spans.
template <int DP> struct Lds {
  static constexpr int kNat = DP + 8;
  static constexpr int kTr = DP + (DP == 32 ? 0 : 32);
};

// Per-thread register staging of an [NR rows x DP] bf16 tile: NPF 16-byte
// chunks per thread, chunk c = tid + 256*u -> row c / (DP/8), column 8*(c % (DP/8)).
template <int DP, int NR>
struct TileRegs {
  static constexpr int CH = DP / 8;
  static constexpr int NPF = (NR * CH + 255) / 256;
  u32x4 v[NPF];

  // row_of(r) -> global row index (element offset / D) or -1 for a zero row
  template <typename RowFn>
  __device__ inline void load(const uint16_t* __restrict__ src, int D, RowFn row_of) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int c = threadIdx.x + 256 * u;
      const int r = c / CH, ch = c - r * CH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < NR) {
        const int64_t g = row_of(r);
        if (g >= 0 && ch * 8 < D) x = *reinterpret_cast<const u32x4*>(src + g * D + ch * 8);
      }
      v[u] = x;
    }
  }
  __device__ inline void store(uint16_t* lds, int stride) const {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int c = threadIdx.x + 256 * u;
      const int r = c / CH, ch = c - r * CH;
      if (r < NR) *reinterpret_cast<u32x4*>(lds + r * stride + ch * 8) = v[u];
    }
  }
};

// Operand with the contraction index along a tile's rows' contiguous dimension:
// lane l gets X[row][k0 + 8*(l/32) .. +7] (one 16-byte LDS read).
__device__ inline bf16x8 lds_row8(const uint16_t* tile, int stride, int row, int k0, int half) {
  return *reinterpret_cast<const bf16x8*>(tile + row * stride + k0 + 8 * half);
}

// Operand whose lane index runs along a tile's contiguous (column) dimension,
// read from a natural [row][col] LDS tile with two gfx950 transpose reads
// (ds_read_b64_tr_b16): lane l gets X[r0 + s][c0 + l%32] in slots s = 0..3 and
// X[r1 + s][c0 + l%32] in slots 4..7.  Within each 16-lane group the hardware
// hands output lane j, slot s, element j%4 of the 8 bytes addressed by lane
// 4s + j/4, so lane i addresses row r + i/4, columns c + 4*(i%4) .. +3.
__device__ inline bf16x8 lds_tr8(const uint16_t* tile, int stride, int r0, int r1, int c0) {
  const int l = threadIdx.x & 63, sub = l & 15;
  const int col = c0 + 16 * ((l >> 4) & 1) + 4 * (sub & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + (r0 + (sub >> 2)) * stride + col));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + (r1 + (sub >> 2)) * stride + col));
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
