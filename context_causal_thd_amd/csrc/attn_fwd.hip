// Causal THD attention forward for one CP rank's query rows (gfx950).
//
// TransformerEngine PR #3221, "Scope and constraints": THD self-attention,
// causal without a sliding window (window_size = (-1, 0)); per the review
// thread the packed documents are kept apart by the cu_seqlens metadata alone.
// A local row at physical token p of document d attends to the actual keys of
// d at positions <= p's position.
//
// One work-group = one query tile of the plan (<= 256/G tokens of one segment
// times the G q heads of one kv head: 256 rows, 8 waves of one 32-row MFMA
// block each) against its key range [document start, last actual token of the
// tile], 64 keys per step:
//   S^T = K Q^T (bf16 MFMA 32x32x16; K operands read by rows from LDS, all of
//   a 32-key block's ahead of its products; Q in registers),
//   online softmax in fp32 / exp2 with the query as the lane index and a
//   rescale of the running output only when a row maximum grows by more than
//   2^8 (the exponentials stay <= 256, the final normalisation is exact),
//   O^T += V^T P^T (V^T operand straight from the natural V tile through the
//   transpose LDS read; P^T straight from the score registers).
// The next step's K/V rows go straight from global memory into the other half
// of double-buffered LDS tiles (buffer loads with an LDS destination) while the
// current step computes.  K/V rows are in physical order, or, for the
// all-gathered entry point, in rank-major order and read through the inverse
// of the partition.  Key steps past the causal diagonal are never visited;
// only steps that straddle it apply the per-element mask.
#include <mutex>

#include "attn_common.h"
#include "cpthd_host.h"

namespace cpthd {

constexpr float kRescaleThreshold = 8.0f;   // log2 units
#ifndef CPTHD_FWD_ROW_BLOCKS
#define CPTHD_FWD_ROW_BLOCKS 1   // 32-row blocks per wave (1: 8 waves, 2: 4 waves)
#endif
constexpr int kFwdRowBlocks = CPTHD_FWD_ROW_BLOCKS;
#ifndef CPTHD_FWD_PREFETCH
#define CPTHD_FWD_PREFETCH 1     // K operands of a 32-key block read ahead of its products
#endif

template <int DP, int QB, bool AG, bool VTR>
__global__ __launch_bounds__(64 * (kQWaves / QB), kQMinBlocks) CPTHD_WAVES_PER_EU(kQWaves / QB * kQMinBlocks / 4) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, const char* __restrict__ ws,
                                                          PlanLayout lay, AttnParams prm, int32_t* status) {
  constexpr int NW = kQWaves / QB;  // waves, QB 32-row blocks each
  // K: read by rows (S^T operand).  V^T operand: with VTR, rows of the
  // workspace's V^T tile, read at the row rate; else the natural V tile
  // through the transpose read, in K's row order (one loader fills both).
  using KT = LdsTile<DP, true>;
  constexpr int V_ELEMS = VTR ? LdsTileVT<VTR ? DP : 64>::ELEMS : LdsTile<DP, true>::ELEMS;
  // two separate buffers per tensor (not one 2-D array): with the step loop
  // unrolled by two, every LDS access names its buffer statically, so the
  // in-flight direct loads into the other buffer need no wait before it
  __shared__ __align__(16) uint16_t K0[KT::ELEMS], K1[KT::ELEMS];
  __shared__ __align__(16) uint16_t V0[V_ELEMS], V1[V_ELEMS];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  const int tile = blockIdx.x / prm.Hkv, kvh = blockIdx.x - (blockIdx.x / prm.Hkv) * prm.Hkv;
  // the tile is read beside the header (the workspace holds a tile slot for
  // every work-group the launch can have); it is used only once both check out
  const QTile t = reinterpret_cast<const QTile*>(ws + lay.qtiles)[tile];
  if (!tile_usable(plan_matches(hdr, prm, lay), tile < hdr->n_qtiles, check_qtile(t, prm, lay), status)) return;

  const int tid = threadIdx.x, wave = wave_index(), lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv;
  const int bm = kRowsPerWG / G;

  // K/V rows [ds, kv_end) of kv head kvh; rows past kv_end read as zero.
  // Physical order: one descriptor over the document's rows, a scalar offset
  // per step.  All-gathered order: a descriptor over all T rows and per-step
  // row offsets through the map.
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
  const int kend = t.kv_end;
  // this entry's steps [s0, s1) of the tile's (a whole tile: all of them)
  const int s0 = t.s0, s1 = min(t.s1, (kend - t.ds + kKvStep - 1) / kKvStep);
  const int64_t kv0 = AG ? 0 : (int64_t)t.ds * Hkv * D;
  const uint32_t kv_bytes = AG ? (uint32_t)prm.T * row_bytes : (uint32_t)(kend - t.ds) * row_bytes;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + kv0, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + kv0, kv_bytes);
  TileLoader<DP, true, NW> kvld;
  AgMap agm;
  AgCursor cur{0, 0};
  if constexpr (AG) {
    agm = ag_map(reinterpret_cast<const DocSeg*>(ws + lay.docs)[t.doc], prm);
    agm.chunk_of(t.ds + s0 * kKvStep, cur.j, cur.start);
  }
  // V^T rows of kv head kvh: the tile's keys from column t.vt on (the
  // document's columns, zero past its actual tokens)
  VTLoader<VTR ? DP : 64, NW> vtld;   // (unused without VTR; 64 keeps the type valid for head dim 32)
  __amdgpu_buffer_rsrc_t vtrs;
  if constexpr (VTR) {
    const uint32_t vt_row_bytes = (uint32_t)lay.vt_cols * 2;
    vtrs = make_rsrc(reinterpret_cast<const uint16_t*>(ws + lay.vt) + (int64_t)kvh * D * lay.vt_cols,
                     (uint32_t)D * vt_row_bytes);
    vtld.init(wave, lane, D, vt_row_bytes);
  }
  auto issue_kv = [&](int kb, uint16_t* Kn, uint16_t* Vn) __attribute__((always_inline)) {
    issue_kv_step<AG, DP, NW, !VTR>(kvld, krs, vrs, agm, cur, kb, t.ds, kend, row_bytes, kvh, D, wave, lane, Kn, Vn);
    if constexpr (VTR) vtld.issue(vtrs, Vn, (uint32_t)(t.vt + (kb - t.ds)) * 2u, wave);
  };
  if constexpr (AG) {
    kvld.init_slots(wave, lane, D);
  } else {
    auto rowoff = [&](int r) __attribute__((always_inline)) -> int64_t { return (int64_t)r * row_bytes + (int64_t)kvh * D * 2; };
    kvld.init(wave, lane, D, rowoff);
  }
  if (s1 > s0) issue_kv(t.ds + s0 * kKvStep, K0, V0);

  // the lane's query row in each of the wave's 32-row blocks
  bool row_in[QB], valid[QB];
  int p_q[QB];
  int64_t qrow[QB];
  bf16x8 qf[QB][DP / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = wave * 32 * QB + 32 * qb + l32;
    const int tt = m / G, g = m - tt * G;
    row_in[qb] = m < bm * G && tt < t.ntok;
    p_q[qb] = t.p0 + tt;
    valid[qb] = row_in[qb] && p_q[qb] < t.ve;
    qrow[qb] = (int64_t)(t.lrow0 + tt) * Hq + kvh * G + g;
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) {
      u32x4 val = {0u, 0u, 0u, 0u};
      const int d = 16 * s + 8 * h;
      if (row_in[qb] && d < D) val = *reinterpret_cast<const u32x4*>(q + qrow[qb] * D + d);
      qf[qb][s] = as_bf16x8(val);
    }
  }

  // Steps this wave computes: up to the one holding the key of its last actual
  // token.  Later steps of the tile are masked for every row of the wave (and
  // a wave without an actual row, the tail of a segment's last tile, has none):
  // it only loads its share of those tiles and meets the barriers, so its SIMD
  // runs the other wave alone.  The outputs do not change.
  int nsteps_w = 0;
  {
    const int m_lo = wave * 32 * QB, m_hi = min(m_lo + 32 * QB, bm * G) - 1;
    if (m_lo <= m_hi && m_lo / G < t.ntok && t.p0 + m_lo / G < t.ve) {
      const int p_hi = min(t.p0 + min(m_hi / G, t.ntok - 1), t.ve - 1);
      nsteps_w = (p_hi + 1 - t.ds + kKvStep - 1) / kKvStep;
    }
  }

  float m_i[QB], l_i[QB];
  f32x16 acc[QB][DP / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_i[qb] = -INFINITY;
    l_i[qb] = 0.f;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) acc[qb][db] = f32x16{};

  lds_loads_barrier();

  const float sl2 = prm.scale_log2;
  f32x16 sc[QB][2];   // scores of one step (key as the VGPR index, query as the lane)
  // S^T of a step's 64 keys against the wave's rows
  auto s_products = [&](const uint16_t* Kt) __attribute__((always_inline)) {
#if CPTHD_FWD_PREFETCH
    // all K operands of key block 0 first, then block 1's reads overlap block 0's products
    bf16x8 ka[DP / 16], kb1[DP / 16];
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) ka[s] = lds_row8<DP, true>(Kt, l32, 16 * s, h);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sc[qb][0] = sc[qb][1] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) {
      kb1[s] = lds_row8<DP, true>(Kt, 32 + l32, 16 * s, h);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb][0] = mfma32(ka[s], qf[qb][s], sc[qb][0]);
    }
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);  // then the products of one operand
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < DP / 16; ++s)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb][1] = mfma32(kb1[s], qf[qb][s], sc[qb][1]);
#else
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb][b] = f32x16{};
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        const bf16x8 a = lds_row8<DP, true>(Kt, 32 * b + l32, 16 * s, h);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb][b] = mfma32(a, qf[qb][s], sc[qb][b]);
      }
    }
#endif
  };
  // online softmax of the step from key kb on: P (bf16 operands) and the running max / sum
  auto softmax = [&](int kb, bf16x8 (&pb)[QB][4]) __attribute__((always_inline)) {
    const bool need_mask = kb + kKvStep - 1 > t.p0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (need_mask) {
        // key kb + 32b + 8(r/4) + 4h + r%4 is allowed iff it is <= the row's token
        const int lim = p_q[qb] - kb - 4 * h;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * b + 8 * (r >> 2) + (r & 3) > lim) sc[qb][b][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qb][b][r]);
      mx = max_xor32(mx) * sl2;
      if (__any(mx > m_i[qb] + kRescaleThreshold)) {
        const float m_new = fmaxf(m_i[qb], mx);
        const float alpha = exp2_fast(m_i[qb] - (m_new == -INFINITY ? 0.f : m_new));
        l_i[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DP / 32; ++db) acc[qb][db] *= alpha;
        m_i[qb] = m_new;
      }
      const float m_use = m_i[qb] == -INFINITY ? 0.f : m_i[qb];
      float rs = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_fast(fmaf(sc[qb][b][r], sl2, -m_use));
          sc[qb][b][r] = pv;
          rs += pv;
        }
      l_i[qb] += rs;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pb[qb][ks] = acc_to_bf16(sc[qb][ks >> 1], 8 * (ks & 1));
    }
  };
  // O^T += V^T P^T
  auto pv_products = [&](const uint16_t* Vt, const bf16x8 (&pb)[QB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 a;
        if constexpr (VTR)   // keys 16ks + 4h + 0..3 and 16ks + 8 + 4h + 0..3, stored together at column 16ks + 8h
          a = *reinterpret_cast<const bf16x8*>(Vt + (32 * db + l32) * LdsTileVT<64>::STRIDE + 16 * ks + 8 * h);
        else
          a = lds_tr8<DP, true>(Vt, 16 * ks + 4 * h, 16 * ks + 8 + 4 * h, 32 * db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32(a, pb[qb][ks], acc[qb][db]);
      }
  };
  auto step = [&](int it, const uint16_t* Kt, const uint16_t* Vt, uint16_t* Kn, uint16_t* Vn) __attribute__((always_inline)) {
    const int kb = t.ds + it * kKvStep;
    if (it + 1 < s1) issue_kv(kb + kKvStep, Kn, Vn);
    bf16x8 pb[QB][4];
    s_products(Kt);
    softmax(kb, pb);
    pv_products(Vt, pb);
    lds_loads_barrier();
  };
  // step s0 + j uses buffer j % 2
  const int n_all = max(s1 - s0, 0), n_w = max(min(nsteps_w, s1) - s0, 0);
  for (int j = 0; j < n_w; j += 2) {
    step(s0 + j, K0, V0, K1, V1);
    if (j + 1 < n_w) step(s0 + j + 1, K1, V1, K0, V0);
  }
  // the rest of the entry's steps: the same loads and barriers, no products
  for (int j = n_w; j < n_all; ++j) {
    if (j + 1 < n_all) issue_kv(t.ds + (s0 + j + 1) * kKvStep, (j & 1) ? K0 : K1, (j & 1) ? V0 : V1);
    lds_loads_barrier();
  }

  if (t.slot >= 0) {
    // One part of a split tile: its unnormalised output and its softmax
    // statistics (the running maximum, in log2 units, and the sum relative to
    // it) go to its partial slot, in the lanes' own order; the merge kernel
    // combines the parts.
    float* slot = reinterpret_cast<float*>(const_cast<char*>(ws) + lay.qpart) +
                  ((int64_t)(t.slot + t.part) * Hkv + kvh) * lay.qpart_stride;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int blk = wave * QB + qb;
#pragma unroll
      for (int db = 0; db < DP / 32; ++db)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
          reinterpret_cast<f32x4*>(slot)[((blk * (DP / 32) + db) * 4 + gi) * 64 + lane] =
              f32x4{acc[qb][db][4 * gi], acc[qb][db][4 * gi + 1], acc[qb][db][4 * gi + 2], acc[qb][db][4 * gi + 3]};
      reinterpret_cast<float2*>(slot + kRowsPerWG * DP)[blk * 64 + lane] = float2{m_i[qb], sum_xor32(l_i[qb])};
    }
    return;
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_xor32(l_i[qb]);
    if (!row_in[qb]) continue;
    const float inv = (valid[qb] && l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d0 = 32 * db + 8 * gi + 4 * h;
        if (d0 < D) {
          u32x2 w;
          w.x = pack_bf16x2(acc[qb][db][4 * gi + 0] * inv, acc[qb][db][4 * gi + 1] * inv);
          w.y = pack_bf16x2(acc[qb][db][4 * gi + 2] * inv, acc[qb][db][4 * gi + 3] * inv);
          *reinterpret_cast<u32x2*>(o + qrow[qb] * D + d0) = w;
        }
      }
    if (h == 0)
      lse[qrow[qb]] = valid[qb] ? (m_i[qb] + log2_fast(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

// Merge of split query tiles: one wave per (split tile, kv head, 32-row
// block), each lane reading the partial values the attention kernel's lane of
// that block held.  With m_p the parts' running maxima and l_p their sums,
// M = max m_p, w_p = 2^(m_p - M), O = sum w_p O_p / sum w_p l_p and
// LSE = (M + log2 sum w_p l_p) ln 2, summed in part order.
template <int DP>
__global__ __launch_bounds__(64) void attn_fwd_merge_kernel(uint16_t* __restrict__ o, float* __restrict__ lse,
                                                            const char* __restrict__ ws, PlanLayout lay,
                                                            AttnParams prm, int32_t* status) {
  constexpr int NBLK = kRowsPerWG / 32;
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  const int Hkv = prm.Hkv;
  const int blk = blockIdx.x % NBLK, pair = blockIdx.x / NBLK;
  const int si = pair / Hkv, kvh = pair - si * Hkv;
  const SplitTile sp = reinterpret_cast<const SplitTile*>(ws + lay.qsplit)[si];
  const bool ok = (sp.slot >= 0) & (sp.nparts >= 2) & (sp.slot <= (int)lay.max_parts - sp.nparts) & (sp.a >= 0) &
                  (sp.b >= 0) & (sp.a <= prm.S - sp.b) & (sp.c >= 0) & (sp.c <= prm.T - sp.b);
  if (!tile_usable(plan_matches(hdr, prm, lay), si < hdr->n_qsplit, ok, status)) return;
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq;
  const int m = 32 * blk + l32, tt = m / G, g = m - tt * G;
  const bool row_in = m < (kRowsPerWG / G) * G && tt < sp.b;
  const bool valid = row_in && sp.c + tt < sp.d;
  const float* part0 = reinterpret_cast<const float*>(ws + lay.qpart) + ((int64_t)sp.slot * Hkv + kvh) * lay.qpart_stride;
  const int64_t pstride = (int64_t)Hkv * lay.qpart_stride;   // floats from one part's slot to the next
  float mx = -INFINITY;
  for (int p = 0; p < sp.nparts; ++p)
    mx = fmaxf(mx, reinterpret_cast<const float2*>(part0 + p * pstride + kRowsPerWG * DP)[blk * 64 + lane].x);
  float l_tot = 0.f;
  f32x16 acc[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) acc[db] = f32x16{};
  for (int p = 0; p < sp.nparts; ++p) {
    const float* src = part0 + p * pstride;
    const float2 st = reinterpret_cast<const float2*>(src + kRowsPerWG * DP)[blk * 64 + lane];
    const float w = st.x == -INFINITY ? 0.f : exp2_fast(st.x - mx);
    l_tot = fmaf(w, st.y, l_tot);
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 x = reinterpret_cast<const f32x4*>(src)[((blk * (DP / 32) + db) * 4 + gi) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * gi + e] = fmaf(w, x[e], acc[db][4 * gi + e]);
      }
  }
  if (!row_in) return;
  const int64_t qrow = (int64_t)(sp.a + tt) * Hq + kvh * G + g;
  const float inv = (valid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int d0 = 32 * db + 8 * gi + 4 * h;
      if (d0 < D) {
        u32x2 w;
        w.x = pack_bf16x2(acc[db][4 * gi + 0] * inv, acc[db][4 * gi + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * gi + 2] * inv, acc[db][4 * gi + 3] * inv);
        *reinterpret_cast<u32x2*>(o + qrow * D + d0) = w;
      }
    }
  if (h == 0) lse[qrow] = (valid && l_tot > 0.f) ? (mx + log2_fast(l_tot)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
// V^T of the forward, written once per call
// ---------------------------------------------------------------------------
// One work-group per (key tile of the plan's list before splitting, kv head):
// the tile's 128 keys of V go through LDS and out as 128-column pieces of the
// D rows of V^T, each 16-key group in the order the forward's operand wants
// (vt_pos16).  Keys past the tile's end or at or past the document's actual
// end are written as zeros, so every column a forward step loads is finite.
template <bool AG>
__global__ __launch_bounds__(256) void attn_vt_kernel(const uint16_t* __restrict__ v, char* __restrict__ ws,
                                                     PlanLayout lay, AttnParams prm, int32_t* status) {
  __shared__ __align__(16) uint16_t sv[kKeysPerWG * (128 + 8)];   // [key][d], rows D + 8 apart
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  const int Hkv = prm.Hkv, D = prm.D, tid = threadIdx.x;
  const int t = blockIdx.x / Hkv, kvh = blockIdx.x - t * Hkv;
  const KVTile kt = reinterpret_cast<const KVTile*>(ws + lay.kvtiles_tmp)[t];
  const bool kt_ok = (kt.doc >= 0) & (kt.doc < prm.num_docs) & (kt.k0 >= 0) & (kt.nkeys >= 0) &
                     (kt.nkeys <= kKeysPerWG) & (kt.k0 <= prm.T - kt.nkeys);
  if (!tile_usable(plan_matches(hdr, prm, lay), t < hdr->n_kvwhole, kt_ok, status)) return;
  const DocSeg d = reinterpret_cast<const DocSeg*>(ws + lay.docs)[kt.doc];
  AgMap agm;
  if constexpr (AG) {
    const bool ds_ok = docseg_ok(d, prm) & ((prm.strategy != kDCS) |
                                            ((kt.k0 >= d.ds) & (kt.k0 - d.ds <= 2 * prm.cp * d.na - kt.nkeys)));
    if (!tile_usable(true, true, ds_ok, status)) return;
    agm = ag_map(d, prm);
  }
  const int stride = D + 8, cpr = D / 8;   // LDS row stride; 16-byte chunks per key row
  // keys [k0, k0 + 128) of kv head kvh into LDS, zeros past the tile or the document's actual tokens
  for (int c = tid; c < kKeysPerWG * cpr; c += 256) {
    const int key = c / cpr, ch = c - key * cpr, p = kt.k0 + key;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < kt.nkeys && p < d.ve) {
      const int64_t row = (AG ? (int64_t)agm.row(p) : (int64_t)p) * Hkv + kvh;
      val = *reinterpret_cast<const u32x4*>(v + row * D + 8 * ch);
    }
    *reinterpret_cast<u32x4*>(sv + key * stride + 8 * ch) = val;
  }
  __syncthreads();
  // row dd of V^T, columns 128 t .. +127: 16 chunks of 8 positions
  uint16_t* out = reinterpret_cast<uint16_t*>(ws + lay.vt) + (int64_t)kvh * D * lay.vt_cols + (int64_t)t * kKeysPerWG;
  for (int c = tid; c < D * 16; c += 256) {
    const int dd = c >> 4, cc = c & 15;
    uint16_t e[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int pos = 8 * cc + s;
      e[s] = sv[((pos & ~15) | vt_pos16(pos & 15)) * stride + dd];
    }
    u32x4 w;
    w.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    w.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    w.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    w.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<u32x4*>(out + (int64_t)dd * lay.vt_cols + 8 * cc) = w;
  }
}

template <int DP, bool AG>
static int launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const char* ws,
                      const PlanLayout& lay, const AttnParams& prm, int32_t* status, unsigned grid,
                      hipStream_t stream, hipEvent_t* ev, int nev) {
  constexpr int QB = kFwdRowBlocks;
  int e;
  if (DP >= 64 && lay.has_vt) {   // (call_layout gives V^T rows only where vt_wanted)
    // V^T rows first (event pair 3), then the forward reading them at the row rate
    const int64_t gvt = ((int64_t)(prm.T + kKeysPerWG - 1) / kKeysPerWG + prm.num_docs) * prm.Hkv;
    e = launch(attn_vt_kernel<AG>, dim3((unsigned)gvt), dim3(256), 0, stream, ev, nev, 3, (const uint16_t*)v,
               const_cast<char*>(ws), lay, prm, status);
    if (e) return e;
    e = launch(attn_fwd_kernel<DP, QB, AG, (DP >= 64)>, dim3(grid), dim3(64 * (kQWaves / QB)), 0, stream, ev, nev, 1,
               (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, ws, lay, prm, status);
  } else {
    if ((e = skip_launch(ev, nev, 3, stream))) return e;
    e = launch(attn_fwd_kernel<DP, QB, AG, false>, dim3(grid), dim3(64 * (kQWaves / QB)), 0, stream, ev, nev, 1,
               (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, ws, lay, prm, status);
  }
  if (e) return e;
  if (lay.max_parts < 2 || !prm.qsplit) return skip_launch(ev, nev, 2, stream);   // no split query tile possible
  return launch(attn_fwd_merge_kernel<DP>, dim3((unsigned)(split_grid(prm, lay) * (kRowsPerWG / 32))), dim3(64), 0,
                stream, ev, nev, 2, (uint16_t*)o, lse, ws, lay, prm, status);
}

template <bool AG>
static int dispatch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const char* ws,
                        const PlanLayout& lay, const AttnParams& prm, int32_t* status, unsigned grid,
                        hipStream_t stream, hipEvent_t* ev, int nev) {
  switch (prm.D) {
    case 16:
    case 32: return launch_fwd<32, AG>(q, k, v, o, lse, ws, lay, prm, status, grid, stream, ev, nev);
    case 64: return launch_fwd<64, AG>(q, k, v, o, lse, ws, lay, prm, status, grid, stream, ev, nev);
    default: return launch_fwd<128, AG>(q, k, v, o, lse, ws, lay, prm, status, grid, stream, ev, nev);
  }
}

int check_attn_args(int64_t T, int64_t capacity, int32_t cp, int32_t rank, int32_t strategy, int32_t num_docs,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t wl, int32_t wr, const void* ws,
                    size_t ws_bytes, PlanLayout& lay, AttnParams& prm) {
  if (cp < 1 || rank < 0 || rank >= cp) return CPTHD_ERR_RANK;
  if (int e = check_strategy(strategy)) return e;
  if (int e = check_tokens(T, capacity, cp, num_docs)) return e;
  if (int e = check_strategy_tokens(strategy, T, cp)) return e;
  if (int e = check_heads(Hq, Hkv, D)) return e;
  if (causal != 1 || wl != -1 || wr != 0) return CPTHD_ERR_MASK;
  lay = call_layout(capacity, cp, Hq, Hkv, D, num_docs, ws_bytes);
  if (!ws || ws_bytes < lay.total || reinterpret_cast<uintptr_t>(ws) % 256) return CPTHD_ERR_WORKSPACE;
  prm.T = (int)T;
  prm.S = (int)(T / cp);
  prm.cp = cp;
  prm.rank = rank;
  prm.strategy = strategy;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.D = D;
  prm.G = Hq / Hkv;
  prm.num_docs = num_docs;
  prm.num_cu = 0;
  prm.qsplit = 0;
  return CPTHD_OK;
}

// Work-groups for the query tiles: an upper bound from the active S, plus the
// parts split tiles may add (the plan holds the exact count; surplus
// work-groups exit at once).
int64_t qtile_grid(const AttnParams& prm, const PlanLayout& lay) {
  const int64_t bm = tokens_per_qtile(prm.G);
  const int64_t seg = (prm.strategy == CPTHD_NO_LOAD_BALANCE ? 1 : 2) * (int64_t)prm.num_docs;
  return ((prm.S + bm - 1) / bm + seg + lay.max_parts) * prm.Hkv;
}

// The same for the key tiles: 128-key tiles of the active T, one more per document, plus the parts.
int64_t kvtile_grid(const AttnParams& prm, const PlanLayout& lay) {
  return (((int64_t)prm.T + kKeysPerWG - 1) / kKeysPerWG + prm.num_docs + lay.max_parts) * prm.Hkv;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_cu_mutex;
int g_cus[kMaxDevices];   // compute units per device, read once
}  // namespace

int device_cus(AttnParams& prm) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CPTHD_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return CPTHD_ERR_LAUNCH;
    g_cus[dev] = n;
  }
  prm.num_cu = g_cus[dev];
  const int64_t bm = tokens_per_qtile(prm.G);
  const int64_t seg = (prm.strategy == CPTHD_NO_LOAD_BALANCE ? 1 : 2) * (int64_t)prm.num_docs;
  prm.qsplit = ((prm.S + bm - 1) / bm + seg) * prm.Hkv < prm.num_cu ? 1 : 0;
  return CPTHD_OK;
}

}  // namespace cpthd

using namespace cpthd;

static int attn_fwd_entry(const void* q_local, const void* k, const void* v, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                          int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                          int32_t causal, int32_t window_left, int32_t window_right, void* o_local, float* lse_local,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream,
                          hipEvent_t* events, int32_t n_events, bool allgathered) {
  if (!q_local || !k || !v || !o_local || !lse_local || !cu_seqlens || !cu_seqlens_padded) return CPTHD_ERR_NULL;
  PlanLayout lay;
  AttnParams prm;
  if (int e = check_attn_args(total_tokens, capacity_tokens, cp_size, rank, strategy, num_docs, num_q_heads,
                              num_kv_heads, head_dim, causal, window_left, window_right, workspace,
                              workspace_bytes, lay, prm))
    return e;
  // the gathered order differs from the physical one unless ownership is contiguous
  const bool ag = allgathered && strategy != CPTHD_NO_LOAD_BALANCE;
  if (ag) {
    if (int e = check_allgathered_bytes(total_tokens, num_kv_heads, head_dim)) return e;
  }
  prm.scale = softmax_scale;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  const int64_t grid = qtile_grid(prm, lay);
  if (grid > INT32_MAX) return CPTHD_ERR_TOKENS;   // more work-groups than one launch takes
  if (int e = device_cus(prm)) return e;
  char* ws = (char*)workspace;
  if (int e = launch_plan(cu_seqlens, cu_seqlens_padded, prm, ws, lay, true, dev_status, stream, events, n_events, 0))
    return e;
  return ag ? dispatch_fwd<true>(q_local, k, v, o_local, lse_local, ws, lay, prm, dev_status, grid, stream, events,
                                 n_events)
            : dispatch_fwd<false>(q_local, k, v, o_local, lse_local, ws, lay, prm, dev_status, grid, stream, events,
                                  n_events);
}

#define CPTHD_FWD_ARGS                                                                                              \
  const void *q_local, const void *k, const void *v, const int32_t *cu_seqlens, const int32_t *cu_seqlens_padded, \
      int32_t num_docs, int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t rank,             \
      int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,        \
      int32_t causal, int32_t window_left, int32_t window_right, void *o_local, float *lse_local, void *workspace, \
      size_t workspace_bytes, int32_t *dev_status, hipStream_t stream
#define CPTHD_FWD_PASS                                                                                              \
  q_local, k, v, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size, rank, strategy, \
      num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, o_local, lse_local,  \
      workspace, workspace_bytes, dev_status, stream

extern "C" int cpthd_attn_fwd(CPTHD_FWD_ARGS) {
  return attn_fwd_entry(CPTHD_FWD_PASS, nullptr, 0, false);
}

extern "C" int cpthd_attn_fwd_allgathered(CPTHD_FWD_ARGS) {
  return attn_fwd_entry(CPTHD_FWD_PASS, nullptr, 0, true);
}

extern "C" int cpthd_attn_fwd_timed(CPTHD_FWD_ARGS, int32_t kv_allgathered, hipEvent_t* events, int32_t n_events) {
  return attn_fwd_entry(CPTHD_FWD_PASS, events, n_events, kv_allgathered != 0);
}
