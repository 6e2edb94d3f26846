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

// Stage `nrows` rows (starting at global row index row(r) of `src`, D valid
// bf16 per row, zero beyond D or beyond nvalid) into LDS, natural layout
// nat[r][DP + 8] and / or transposed trn[d][NR + 8].
template <int DP, int NR, bool NAT, bool TRN, typename RowFn>
__device__ inline void stage_rows(const uint16_t* __restrict__ src, int D, RowFn row_of, uint16_t* nat,
                                  uint16_t* trn) {
  constexpr int CH = DP / 8;
  for (int c = threadIdx.x; c < NR * CH; c += blockDim.x) {
    const int r = c / CH, ch = c - r * CH;
    const int64_t g = row_of(r);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (g >= 0 && ch * 8 < D) val = *reinterpret_cast<const u32x4*>(src + g * D + ch * 8);
    if (NAT) *reinterpret_cast<u32x4*>(nat + r * (DP + 8) + ch * 8) = val;
    if (TRN) {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
      for (int i = 0; i < 8; ++i) trn[(ch * 8 + i) * (NR + 8) + r] = e[i];
    }
  }
}

// A operand (32 rows x 16 k) from a natural LDS tile: row 32*blk + l%32, k = 16*s + 8*(l/32).
template <int DP>
__device__ inline bf16x8 lds_a_nat(const uint16_t* nat, int row, int s, int half) {
  return *reinterpret_cast<const bf16x8*>(nat + row * (DP + 8) + 16 * s + 8 * half);
}

// A operand from a transposed LDS tile trn[d][NR+8] whose contraction index
// follows the accumulator permutation: k-step `ks` of 16 covers entries
// 16*ks + {4h..4h+3, 8+4h..8+4h+3} (h = l/32).
template <int NR>
__device__ inline bf16x8 lds_a_trn(const uint16_t* trn, int drow, int ks, int half) {
  const uint16_t* p = trn + drow * (NR + 8) + 16 * ks + 4 * half;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  u32x4 v = {lo.x, lo.y, hi.x, hi.y};
  return as_bf16x8(v);
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
