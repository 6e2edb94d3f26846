// Causal THD attention backward for one CP rank (gfx950).
//
// TransformerEngine PR #3221: forward captures the strategy so backward uses
// the same token layout ("What changed"); in the sequence diagram backward
// restores that strategy and uses its step layout and K/V order to return
// dQ/dK/dV.  With P = softmax of the scores, dP = dO V^T and
// delta = rowsum(dO * O) = rowsum(P * dP):
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// dK/dV here are the rank's partial gradients (its query rows only) over all
// T physical rows; a reduce-scatter over the ranks would sum them.
//
// Two passes, no atomics, deterministic:
//   1. query tiles (the forward's tiles, 32 rows per wave): delta from O and
//      dO, then per 64-key step S^T = K Q^T, P^T = exp2(S^T - LSE),
//      dP^T = V dO^T, dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (the K^T
//      operand comes from the natural K tile through the transpose LDS read);
//   2. key tiles (128 keys of one document; 8 waves, each pair of waves
//      sharing 32 keys and splitting the dK/dV columns): for every query row
//      of the rank that sees the tile, 64 rows per step, last rows first,
//      S = Q K^T and dP = dO V^T with the key as the lane index,
//      dS = P (dP - delta), dV += P^T dO and dK += dS^T Q (dO^T and Q^T
//      operands through the transpose read of the natural tiles).
// Both passes load the next step's rows straight into the other half of
// double-buffered LDS tiles while computing the current one.  K/V (and dK/dV)
// rows are in physical order, or in rank-major all-gathered order for the
// all-gathered entry point.
#include <algorithm>
#include <mutex>

#include "attn_common.h"
#include "cpthd_host.h"

namespace cpthd {

#ifndef CPTHD_DQ_ROW_BLOCKS
#define CPTHD_DQ_ROW_BLOCKS 1
#endif
constexpr int kDqRowBlocks = CPTHD_DQ_ROW_BLOCKS;   // 32-row blocks per wave (1: 8 waves, 2: 4 waves)
#ifndef CPTHD_DKDV_SPLIT
#define CPTHD_DKDV_SPLIT 2
#endif
constexpr int kDkdvSplit = CPTHD_DKDV_SPLIT;   // 1: 4 waves; 2: 8 waves, key-group pairs splitting dK/dV columns
#ifndef CPTHD_DQ_SPLIT
#define CPTHD_DQ_SPLIT 2   // work-groups per query tile in the dQ pass (two 4-wave groups per CU)
#endif
constexpr int kDqSplit = CPTHD_DQ_SPLIT;
#ifndef CPTHD_DQ_PIPE
#define CPTHD_DQ_PIPE 1   // read-ahead scheduling hints in the dQ pass
#endif
#ifndef CPTHD_DKDV_ACC_PIPE
#define CPTHD_DKDV_ACC_PIPE 2   // dK/dV products: transpose-read pairs kept this many ahead (0: no hint)
#endif
#ifndef CPTHD_DKDV_PIPE
#define CPTHD_DKDV_PIPE 2   // dK/dV score products: row reads kept this many ahead (0: no hint)
#endif
#ifndef CPTHD_DKDV_REVERSE
#define CPTHD_DKDV_REVERSE 1   // dK/dV: visit a key tile's query chunks last first
#endif

// ---------------------------------------------------------------------------
// pass 1: delta and dQ over the query tiles
// ---------------------------------------------------------------------------
template <int DP, int QB, bool AG>
__global__ __launch_bounds__(64 * (kQWaves / QB / kDqSplit), kQMinBlocks * kDqSplit)
    CPTHD_WAVES_PER_EU(kQWaves / QB * kQMinBlocks / 4) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dq, char* __restrict__ ws, PlanLayout lay, AttnParams prm, int32_t* status) {
  constexpr int NW = kQWaves / QB / kDqSplit;  // waves, QB 32-row blocks each
  using KT = LdsTile<DP, true>;    // K: read by rows (S^T operand) and transposed (K^T operand of dQ^T)
  using VT = LdsTile<DP, true>;    // V: read by rows (dP^T operand), in K's row order (one loader for both)
  __shared__ __align__(16) uint16_t K0[KT::ELEMS], K1[KT::ELEMS];
  __shared__ __align__(16) uint16_t V0[VT::ELEMS], V1[VT::ELEMS];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  // kDqSplit work-groups per query tile, each with kRowsPerWG / kDqSplit of its rows; the kv head stays
  // blockIdx mod Hkv
  const int kvh = blockIdx.x - (blockIdx.x / prm.Hkv) * prm.Hkv;
  const int tile = blockIdx.x / (prm.Hkv * kDqSplit), half = (blockIdx.x / prm.Hkv) % kDqSplit;
  // the tile is read beside the header (the workspace holds a tile slot for
  // every query tile the launch can have); it is used only once both check out
  const QTile t = reinterpret_cast<const QTile*>(ws + lay.qtiles)[tile];
  if (!tile_usable(plan_matches(hdr, prm, lay), tile < hdr->n_qtiles, check_qtile(t, prm, lay), status)) return;
  float* ndelta = reinterpret_cast<float*>(ws + lay.delta);   // -delta per row, for the key-tile pass
  float* lse2w = reinterpret_cast<float*>(ws + lay.lse2);

  const int tid = threadIdx.x, wave = wave_index(), lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv;
  const int bm = kRowsPerWG / G;
  // a work-group holding none of the tile's rows (the tile has at most
  // half * kRowsPerWG / kDqSplit of them) has nothing to write: it leaves
  // before issuing any load
  const int m_first = half * (kRowsPerWG / kDqSplit);
  if (m_first >= bm * G || m_first / G >= t.ntok) return;

  // K/V rows [ds, kv_end) as in the forward (physical or all-gathered order)
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
  auto issue_kv = [&](int kb, uint16_t* Kn, uint16_t* Vn) __attribute__((always_inline)) {
    issue_kv_step<AG>(kvld, krs, vrs, agm, cur, kb, t.ds, kend, row_bytes, kvh, D, wave, lane, Kn, Vn);
  };
  if constexpr (AG) {
    kvld.init_slots(wave, lane, D);
  } else {
    auto rowoff = [&](int r) __attribute__((always_inline)) -> int64_t { return (int64_t)r * row_bytes + (int64_t)kvh * D * 2; };
    kvld.init(wave, lane, D, rowoff);
  }
  if (s1 > s0) issue_kv(t.ds + s0 * kKvStep, K0, V0);

  bool row_in[QB], valid[QB];
  int p_q[QB];
  int64_t qrow[QB];
  float dlt[QB], lse2[QB];
  bf16x8 qf[QB][DP / 16], df[QB][DP / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = half * (kRowsPerWG / kDqSplit) + wave * 32 * QB + 32 * qb + l32;
    const int tt = m / G, g = m - tt * G;
    row_in[qb] = m < bm * G && tt < t.ntok;
    p_q[qb] = t.p0 + tt;
    valid[qb] = row_in[qb] && p_q[qb] < t.ve;
    qrow[qb] = (int64_t)(t.lrow0 + tt) * Hq + kvh * G + g;
    float dpart = 0.f;
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) {
      u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = {0u, 0u, 0u, 0u}, ov = {0u, 0u, 0u, 0u};
      const int d = 16 * s + 8 * h;
      if (valid[qb] && d < D) {
        qv = *reinterpret_cast<const u32x4*>(q + qrow[qb] * D + d);
        dv4 = *reinterpret_cast<const u32x4*>(dout + qrow[qb] * D + d);
        ov = *reinterpret_cast<const u32x4*>(o + qrow[qb] * D + d);
      }
      qf[qb][s] = as_bf16x8(qv);
      df[qb][s] = as_bf16x8(dv4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = dv4[i], b = ov[i];
        dpart += __uint_as_float(a << 16) * __uint_as_float(b << 16) +
                 __uint_as_float(a & 0xFFFF0000u) * __uint_as_float(b & 0xFFFF0000u);
      }
    }
    dlt[qb] = sum_xor32(dpart);
    lse2[qb] = valid[qb] ? lse[qrow[qb]] * 1.4426950408889634f : INFINITY;
    // (every part of a split tile writes the same values)
    if (row_in[qb] && h == 0) {
      ndelta[qrow[qb]] = valid[qb] ? -dlt[qb] : 0.f;
      lse2w[qrow[qb]] = valid[qb] ? lse2[qb] : 0.f;
    }
  }

  // a wave none of whose rows is an actual token (the tail of a segment's last
  // tile, or pads) skips the products and only helps load the tiles: its SIMD
  // then runs the other wave alone (its rows' dQ stays zero, as it must).  The
  // all-gathered instantiation keeps every wave computing: it sits at the
  // register limit, and the second loop made it spill.
  bool any_valid = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) any_valid = any_valid || valid[qb];
  const bool wave_active = AG || __any(any_valid);

  f32x16 acc[QB][DP / 32], ndl[QB];   // ndl: -delta in every entry, the start of each dP^T product
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) acc[qb][db] = f32x16{};
#pragma unroll
    for (int r = 0; r < 16; ++r) ndl[qb][r] = -dlt[qb];
  }

  lds_loads_barrier();

  const float sl2 = prm.scale_log2;
  auto step = [&](int it, const uint16_t* Kt, const uint16_t* Vt, uint16_t* Kn, uint16_t* Vn) __attribute__((always_inline)) {
    const int kb = t.ds + it * kKvStep;
    if (it + 1 < s1) issue_kv(kb + kKvStep, Kn, Vn);
    const bool need_mask = kb + kKvStep - 1 > t.p0;
    bf16x8 dsb[QB][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 sc[QB], dp[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        sc[qb] = f32x16{};
        dp[qb] = ndl[qb];   // dP^T - delta accumulates in place
      }
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        const bf16x8 ka = lds_row8<DP, true>(Kt, 32 * b + l32, 16 * s, h);
        const bf16x8 va = lds_row8<DP, true>(Vt, 32 * b + l32, 16 * s, h);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sc[qb] = mfma32(ka, qf[qb][s], sc[qb]);
          dp[qb] = mfma32(va, df[qb][s], dp[qb]);
        }
      }
#if CPTHD_DQ_PIPE
      if constexpr (QB == 1) pipeline_reads_mfma<2 * (DP / 16), 4>();
#endif
      // dS = P (dP - delta); the causal test only on steps that reach the diagonal (a uniform branch)
      auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lim = p_q[qb] - kb - 32 * b - 4 * h;   // key offset 8(r/4) + r%4 allowed iff <= lim
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float pv = exp2_fast(fmaf(sc[qb][r], sl2, -lse2[qb]));
            if constexpr (decltype(masked)::value)
              if (8 * (r >> 2) + (r & 3) > lim) pv = 0.f;
            sc[qb][r] = pv * dp[qb][r];
          }
          dsb[qb][2 * b] = acc_to_bf16(sc[qb], 0);
          dsb[qb][2 * b + 1] = acc_to_bf16(sc[qb], 8);
        }
      };
      if (need_mask)
        probs(std::true_type{});
      else
        probs(std::false_type{});
    }
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = lds_tr8<DP, true>(Kt, 16 * ks + 4 * h, 16 * ks + 8 + 4 * h, 32 * db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32(a, dsb[qb][ks], acc[qb][db]);
      }
#if CPTHD_DQ_PIPE
    if constexpr (QB == 1) pipeline_reads_mfma<4 * (DP / 32), 2, 2>();
#endif
    lds_loads_barrier();
  };
  // step s0 + j uses buffer j % 2
  if (wave_active) {
    for (int it = s0; it < s1; it += 2) {
      step(it, K0, V0, K1, V1);
      if (it + 1 < s1) step(it + 1, K1, V1, K0, V0);
    }
  } else {
    // the same loads and barriers, no products
    for (int it = s0; it < s1; it += 2) {
      if (it + 1 < s1) issue_kv(t.ds + (it + 1) * kKvStep, K1, V1);
      lds_loads_barrier();
      if (it + 1 < s1) {
        if (it + 2 < s1) issue_kv(t.ds + (it + 2) * kKvStep, K0, V0);
        lds_loads_barrier();
      }
    }
  }

  if (t.slot >= 0) {
    // One part of a split tile: its dQ^T accumulators go to its partial slot
    // (this half's rows), in the lanes' own order; the merge kernel sums the
    // parts.
    float* slot = reinterpret_cast<float*>(ws + lay.qpart) + ((int64_t)(t.slot + t.part) * Hkv + kvh) * lay.qpart_stride;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int blk = half * (NW * QB) + wave * QB + qb;
#pragma unroll
      for (int db = 0; db < DP / 32; ++db)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
          reinterpret_cast<f32x4*>(slot)[((blk * (DP / 32) + db) * 4 + gi) * 64 + lane] =
              f32x4{acc[qb][db][4 * gi], acc[qb][db][4 * gi + 1], acc[qb][db][4 * gi + 2], acc[qb][db][4 * gi + 3]};
    }
    return;
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (!row_in[qb]) continue;
    const float sc = valid[qb] ? prm.scale : 0.f;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d0 = 32 * db + 8 * gi + 4 * h;
        if (d0 < D) {
          const f32x4 w = {acc[qb][db][4 * gi] * sc, acc[qb][db][4 * gi + 1] * sc, acc[qb][db][4 * gi + 2] * sc,
                           acc[qb][db][4 * gi + 3] * sc};
          *reinterpret_cast<f32x4*>(dq + qrow[qb] * D + d0) = w;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// pass 2: dK and dV over the key tiles
// ---------------------------------------------------------------------------
// Direct loads of one step's Q and dO rows (local rows from `base` / Hq, ntok
// tokens) and of their LSE*log2(e) and -delta values into the given buffers.
template <int DP, int NW>
__device__ inline void issue_q_chunk(const TileLoader<DP, true, NW>& qld, const uint16_t* q, const uint16_t* dout,
                                     const float* lse2w, const float* ndelta, int64_t base, int ntok,
                                     uint32_t tok_bytes, int Hq, int D, uint32_t ld_off, int wave, uint16_t* Qn,
                                     uint16_t* On, float* Ln, float* En) {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer-resource builtins: device pass only
  const uint32_t nrec = (uint32_t)ntok * tok_bytes;
  qld.issue(make_rsrc(q + base * D, nrec), Qn, 0, wave);
  qld.issue(make_rsrc(dout + base * D, nrec), On, 0, wave);
  if (wave == 0) lds_load_dword(make_rsrc(lse2w + base, (uint32_t)ntok * Hq * 4), Ln, ld_off);
  if (wave == 1) lds_load_dword(make_rsrc(ndelta + base, (uint32_t)ntok * Hq * 4), En, ld_off);
#endif
}

template <int DP, int SD, bool AG>
__global__ __launch_bounds__(256 * SD, 1) CPTHD_WAVES_PER_EU(SD) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ dk,
    float* __restrict__ dv, char* __restrict__ ws, PlanLayout lay, AttnParams prm, int32_t* status) {
  // 4 * SD waves.  Wave w owns keys k0 + 32*(w%4) .. +31.  With SD = 2 the two
  // waves of a key group split the head dimension of dK/dV: wave w computes
  // S and dP for query block w/4 of each 64-row step only, and the pair swaps
  // its bf16 P and dS operands through LDS (same lane layout, a plain copy).
  constexpr int NW = 4 * SD;
  constexpr int NDB = DP / 32 / SD;   // 32-column blocks of dK/dV per wave
  using QT = LdsTile<DP, true>;   // Q and dO: read by rows (S, dP operands) and transposed (dK, dV operands)
  __shared__ __align__(16) uint16_t Q0[QT::ELEMS], Q1[QT::ELEMS];
  __shared__ __align__(16) uint16_t O0[QT::ELEMS], O1[QT::ELEMS];
  __shared__ __align__(16) float L0[kQChunk], L1[kQChunk], E0[kQChunk], E1[kQChunk];   // LSE*log2(e), -delta
  __shared__ __align__(16) bf16x8 X[SD == 2 ? 4 * 2 * 4 * 64 : 1];   // [key group][query block][P0,P1,dS0,dS1][lane]

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  const int tile = blockIdx.x / prm.Hkv, kvh = blockIdx.x - (blockIdx.x / prm.Hkv) * prm.Hkv;
  // the tile is read beside the header (the workspace holds a tile slot for
  // every work-group the launch can have); it is used only once both check out
  const KVTile kt = reinterpret_cast<const KVTile*>(ws + lay.kvtiles)[tile];
  const bool kt_ok = (kt.doc >= 0) & (kt.doc < prm.num_docs) & (kt.k0 >= 0) & (kt.nkeys >= 0) &
                     (kt.nkeys <= kKeysPerWG) & (kt.k0 <= prm.T - kt.nkeys) & (kt.c0 >= 0) & (kt.c1 >= kt.c0) &
                     parts_ok(kt.slot, kt.part, kt.nparts, lay);
  if (!tile_usable(plan_matches(hdr, prm, lay), tile < hdr->n_kvtiles, kt_ok, status)) return;
  const DocSeg ds = reinterpret_cast<const DocSeg*>(ws + lay.docs)[kt.doc];
  // the document's segments and, for the all-gathered order, the tile's keys
  // inside the document's chunks: every K/V/dK/dV row the map gives is then < T
  const bool ds_ok = docseg_ok(ds, prm) &
                     (!AG | (prm.strategy != kDCS) |
                      ((kt.k0 >= ds.ds) & (kt.k0 - ds.ds <= 2 * prm.cp * ds.na - kt.nkeys)));
  if (!tile_usable(true, true, ds_ok, status)) return;
  const float* ndelta = reinterpret_cast<const float*>(ws + lay.delta);
  const float* lse2w = reinterpret_cast<const float*>(ws + lay.lse2);

  const int tid = threadIdx.x, wave = wave_index(), lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv, S = prm.S;
  const int kw = wave & 3, dh = wave >> 2;
  const int key = kt.k0 + kw * 32 + l32;            // this lane's key (B operand column)
  const bool key_in = kw * 32 + l32 < kt.nkeys;
  AgMap agm;
  if constexpr (AG) agm = ag_map(ds, prm);
  // K/V/dK/dV row of a key: physical, or its rank-major all-gathered row
  auto kv_row = [&](int p) __attribute__((always_inline)) -> int64_t {
    if constexpr (AG) return (int64_t)agm.row(p) * Hkv + kvh;
    return (int64_t)p * Hkv + kvh;
  };
  const int64_t krow = kv_row(key);

  // the rank's rows of the document that see the tile: suffixes (token >= k0)
  // of the document's segments, cut into steps of tpc tokens
  const int tpc = kQChunk / G;
  int plo[2], phi[2], sl[2], sp[2], nch[2];
#pragma unroll
  for (int si = 0; si < 2; ++si) {
    sp[si] = si == 0 ? ds.pa : ds.pb;
    const int sn = si == 0 ? ds.na : ds.nb;
    sl[si] = si == 0 ? ds.la : ds.lb;
    plo[si] = max(sp[si], kt.k0);
    phi[si] = min(sp[si] + sn, ds.ve);
    nch[si] = (phi[si] > plo[si] && sl[si] >= 0 && sl[si] + (phi[si] - sp[si]) <= S)
                  ? (phi[si] - plo[si] + tpc - 1) / tpc : 0;
  }
  const int nchunks = nch[0] + nch[1];
  // this entry's chunks [c0, c1) in visiting order (a whole tile: all of them)
  const int c_lo = min(kt.c0, nchunks), c_hi = min(kt.c1, nchunks);
  // chunk i: first token c0 and first local row l0
  auto chunk_at = [&](int i, int& c0, int& l0, int& ntok) __attribute__((always_inline)) {
#if CPTHD_DKDV_REVERSE
    // last chunk first: every key tile of a document starts on the document's
    // last rows, so concurrently running tiles share their Q / dO reads in L2
    i = nchunks - 1 - i;
#endif
    const int si = i < nch[0] ? 0 : 1;
    c0 = plo[si] + (i - (si ? nch[0] : 0)) * tpc;
    l0 = sl[si] + (c0 - sp[si]);
    ntok = min(tpc, phi[si] - c0);
  };

  // Q / dO rows of a chunk: tile row r = token r/G, head r%G; LSE / -delta: one float per row
  const uint32_t tok_bytes = (uint32_t)Hq * D * 2;
  TileLoader<DP, true, NW> qld;
  auto qrowoff = [&](int r) __attribute__((always_inline)) -> int64_t {
    const int t2 = r / G;
    return r < tpc * G ? (int64_t)t2 * tok_bytes + (int64_t)(kvh * G + r - t2 * G) * D * 2 : -1;
  };
  qld.init(wave, lane, D, qrowoff);
  const uint32_t ld_off = lane < tpc * G ? (uint32_t)((lane / G) * Hq + kvh * G + lane % G) * 4u : 0x80000000u;
  auto issue = [&](int i, uint16_t* Qn, uint16_t* On, float* Ln, float* En) __attribute__((always_inline)) {
    int c0, l0, ntok;
    chunk_at(i, c0, l0, ntok);
    issue_q_chunk<DP, NW>(qld, q, dout, lse2w, ndelta, (int64_t)l0 * Hq, ntok, tok_bytes, Hq, D, ld_off, wave, Qn,
                          On, Ln, En);
  };
  if (c_hi > c_lo) issue(c_lo, Q0, O0, L0, E0);

  bf16x8 kf[DP / 16], vf[DP / 16];
#pragma unroll
  for (int s = 0; s < DP / 16; ++s) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    const int d = 16 * s + 8 * h;
    if (key_in && d < D && c_hi > c_lo) {   // an entry no row of the rank sees only writes zeros
      a = *reinterpret_cast<const u32x4*>(k + krow * D + d);
      b = *reinterpret_cast<const u32x4*>(v + krow * D + d);
    }
    kf[s] = as_bf16x8(a);
    vf[s] = as_bf16x8(b);
  }
  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    dka[j] = f32x16{};
    dva[j] = f32x16{};
  }
  lds_loads_barrier();

  const float sl2 = prm.scale_log2;
  const int kmax = kt.k0 + kt.nkeys - 1;
  auto step = [&](int i, const uint16_t* Qt, const uint16_t* Dt, const float* Lt, const float* Et, uint16_t* Qn,
                  uint16_t* On, float* Ln, float* En) __attribute__((always_inline)) {
    int c0, l0, ntok;
    chunk_at(i, c0, l0, ntok);
    if (i + 1 < c_hi) issue(i + 1, Qn, On, Ln, En);
    // row qi (token c0 + qi/G) sees this lane's key iff qi >= (key - c0) * G
    const bool need_mask = kmax > c0;
    const int thr = (key - c0) * G - 4 * h;
    // P and dS of one 32-row query block as bf16 operands (key as the lane index)
    auto scores = [&](int qb, bf16x8 (&pd)[4]) {
      // dP starts from the rows' -delta, so it accumulates dP - delta in place
      f32x16 sc = f32x16{}, dp;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(Et + 32 * qb + 8 * g4 + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * g4 + j] = e4[j];
      }
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        sc = mfma32(lds_row8<DP, true>(Qt, 32 * qb + l32, 16 * s, h), kf[s], sc);
        dp = mfma32(lds_row8<DP, true>(Dt, 32 * qb + l32, 16 * s, h), vf[s], dp);
      }
#if CPTHD_DKDV_PIPE
      pipeline_reads_mfma<2 * (DP / 16), CPTHD_DKDV_PIPE, 1, 4>();   // + the four reads of -delta
#endif
      // P = exp2(S * scale * log2(e) - LSE * log2(e)), dS = P (dP - delta); the
      // causal test only on steps that reach the tile's diagonal (a uniform branch)
      auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q4 = 32 * qb + 8 * g4 + 4 * h;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + q4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * g4 + j;
            float pv = exp2_fast(fmaf(sc[r], sl2, -l4[j]));
            if constexpr (decltype(masked)::value)
              if (32 * qb + 8 * g4 + j < thr) pv = 0.f;
            sc[r] = pv;
            dp[r] = pv * dp[r];
          }
        }
      };
      if (need_mask)
        probs(std::true_type{});
      else
        probs(std::false_type{});
      pd[0] = acc_to_bf16(sc, 0);
      pd[1] = acc_to_bf16(sc, 8);
      pd[2] = acc_to_bf16(dp, 0);
      pd[3] = acc_to_bf16(dp, 8);
    };
    // dV += P^T dO, dK += dS^T Q for one query block over this wave's column blocks
    auto accumulate = [&](int qb, const bf16x8 (&pd)[4]) {
      const int r0 = 32 * qb + 4 * h;
#if CPTHD_DKDV_ACC_PIPE
      __builtin_amdgcn_sched_barrier(0);   // its own scheduling region, so the hint below applies to it alone
#endif
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        const int c0l = 32 * (dh * NDB + j);
        dva[j] = mfma32(pd[0], lds_tr8<DP, true>(Dt, r0, r0 + 8, c0l), dva[j]);
        dva[j] = mfma32(pd[1], lds_tr8<DP, true>(Dt, r0 + 16, r0 + 24, c0l), dva[j]);
        dka[j] = mfma32(pd[2], lds_tr8<DP, true>(Qt, r0, r0 + 8, c0l), dka[j]);
        dka[j] = mfma32(pd[3], lds_tr8<DP, true>(Qt, r0 + 16, r0 + 24, c0l), dka[j]);
      }
#if CPTHD_DKDV_ACC_PIPE
      pipeline_reads_mfma<4 * NDB, CPTHD_DKDV_ACC_PIPE, 2>();
#endif
    };
    if (SD == 1) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        bf16x8 pd[4];
        scores(qb, pd);
        accumulate(qb, pd);
      }
    } else {
      // the wave's own block first (before the exchange barrier), then the partner's:
      // only one set of operands is live at a time
      bf16x8 pd[4];
      scores(dh, pd);
#pragma unroll
      for (int j = 0; j < 4; ++j) X[((kw * 2 + dh) * 4 + j) * 64 + lane] = pd[j];
      accumulate(dh, pd);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) pd[j] = X[((kw * 2 + (dh ^ 1)) * 4 + j) * 64 + lane];
      accumulate(dh ^ 1, pd);
    }
    lds_loads_barrier();
  };
  // chunk c_lo + j uses buffer j % 2
  for (int i = c_lo; i < c_hi; i += 2) {
    step(i, Q0, O0, L0, E0, Q1, O1, L1, E1);
    if (i + 1 < c_hi) step(i + 1, Q1, O1, L1, E1, Q0, O0, L0, E0);
  }

  if (kt.slot >= 0) {
    // One part of a split tile: its dK and dV accumulators go to its partial
    // slot, in the lanes' own order; the merge kernel sums the parts.
    float* slot = reinterpret_cast<float*>(ws + lay.kvpart) +
                  ((int64_t)(kt.slot + kt.part) * Hkv + kvh) * lay.kvpart_stride;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        reinterpret_cast<f32x4*>(slot)[(((wave * NDB + j) * 2 + 0) * 4 + gi) * 64 + lane] =
            f32x4{dka[j][4 * gi], dka[j][4 * gi + 1], dka[j][4 * gi + 2], dka[j][4 * gi + 3]};
        reinterpret_cast<f32x4*>(slot)[(((wave * NDB + j) * 2 + 1) * 4 + gi) * 64 + lane] =
            f32x4{dva[j][4 * gi], dva[j][4 * gi + 1], dva[j][4 * gi + 2], dva[j][4 * gi + 3]};
      }
    return;
  }

  // dV[key][d] = C[i = key][j = d]: lane holds d = 32*(dh*NDB + j) + l32 for 16 keys of its key group
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    const int d = 32 * (dh * NDB + j) + l32;
    if (d >= D) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = kw * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kl < kt.nkeys) {
        const int64_t row = kv_row(kt.k0 + kl);
        dv[row * D + d] = dva[j][r];
        dk[row * D + d] = dka[j][r] * prm.scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge of split tiles: dQ of split query tiles, dK / dV of split key tiles
// ---------------------------------------------------------------------------
// One wave per work-group.  Work-groups [0, nq) take (split query tile, kv
// head, 32-row block) in the query-tile pass's row layout; the rest take
// (split key tile, kv head, wave role) in the key-tile pass's.  Each lane sums,
// in part order, the partial values that lane held, and writes its rows as the
// attention kernels write whole tiles.
template <int DP, int SD, bool AG>
__global__ __launch_bounds__(64) void attn_bwd_merge_kernel(float* __restrict__ dq, float* __restrict__ dk,
                                                            float* __restrict__ dv, const char* __restrict__ ws,
                                                            PlanLayout lay, AttnParams prm, int32_t* status, int nq) {
  constexpr int NBLK = kRowsPerWG / 32;
  constexpr int NW = 4 * SD;            // waves of the key-tile pass
  constexpr int NDB = DP / 32 / SD;
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv;
  if ((int)blockIdx.x < nq) {
    const int blk = blockIdx.x % NBLK, pair = blockIdx.x / NBLK;
    const int si = pair / Hkv, kvh = pair - si * Hkv;
    const SplitTile sp = reinterpret_cast<const SplitTile*>(ws + lay.qsplit)[si];
    const bool ok = (sp.slot >= 0) & (sp.nparts >= 2) & (sp.slot <= (int)lay.max_parts - sp.nparts) &
                    (sp.a >= 0) & (sp.b >= 0) & (sp.a <= prm.S - sp.b) & (sp.c >= 0) & (sp.c <= prm.T - sp.b);
    if (!tile_usable(plan_matches(hdr, prm, lay), si < hdr->n_qsplit, ok, status)) return;
    const int m = 32 * blk + l32, tt = m / G, g = m - tt * G;
    if (!(m < (kRowsPerWG / G) * G && tt < sp.b)) return;
    const float* part0 = reinterpret_cast<const float*>(ws + lay.qpart) + ((int64_t)sp.slot * Hkv + kvh) * lay.qpart_stride;
    const int64_t pstride = (int64_t)Hkv * lay.qpart_stride;
    const float sc = sp.c + tt < sp.d ? prm.scale : 0.f;
    const int64_t qrow = (int64_t)(sp.a + tt) * Hq + kvh * G + g;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) {
      f32x16 acc = f32x16{};
      for (int p = 0; p < sp.nparts; ++p)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const f32x4 x = reinterpret_cast<const f32x4*>(part0 + p * pstride)[((blk * (DP / 32) + db) * 4 + gi) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * gi + e] += x[e];
        }
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d0 = 32 * db + 8 * gi + 4 * h;
        if (d0 < D)
          *reinterpret_cast<f32x4*>(dq + qrow * D + d0) =
              f32x4{acc[4 * gi] * sc, acc[4 * gi + 1] * sc, acc[4 * gi + 2] * sc, acc[4 * gi + 3] * sc};
      }
    }
    return;
  }
  const int b = blockIdx.x - nq;
  const int wave = b % NW, pair = b / NW;
  const int si = pair / Hkv, kvh = pair - si * Hkv;
  const SplitTile sp = reinterpret_cast<const SplitTile*>(ws + lay.kvsplit)[si];
  const bool ok = (sp.slot >= 0) & (sp.nparts >= 2) & (sp.slot <= (int)lay.max_parts - sp.nparts) & (sp.a >= 0) &
                  (sp.b >= 0) & (sp.b <= kKeysPerWG) & (sp.a <= prm.T - sp.b) & (sp.c >= 0) & (sp.c < prm.num_docs);
  if (!tile_usable(plan_matches(hdr, prm, lay), si < hdr->n_kvsplit, ok, status)) return;
  AgMap agm;
  if constexpr (AG) {
    const DocSeg d = reinterpret_cast<const DocSeg*>(ws + lay.docs)[sp.c];
    const bool ds_ok = docseg_ok(d, prm) & ((prm.strategy != kDCS) |
                                            ((sp.a >= d.ds) & (sp.a - d.ds <= 2 * prm.cp * d.na - sp.b)));
    if (!tile_usable(true, true, ds_ok, status)) return;
    agm = ag_map(d, prm);
  }
  const int kw = wave & 3, dh = wave >> 2;
  const float* part0 = reinterpret_cast<const float*>(ws + lay.kvpart) + ((int64_t)sp.slot * Hkv + kvh) * lay.kvpart_stride;
  const int64_t pstride = (int64_t)Hkv * lay.kvpart_stride;
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    f32x16 ka = f32x16{}, va = f32x16{};
    for (int p = 0; p < sp.nparts; ++p)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4* src = reinterpret_cast<const f32x4*>(part0 + p * pstride);
        const f32x4 x = src[(((wave * NDB + j) * 2 + 0) * 4 + gi) * 64 + lane];
        const f32x4 y = src[(((wave * NDB + j) * 2 + 1) * 4 + gi) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ka[4 * gi + e] += x[e];
          va[4 * gi + e] += y[e];
        }
      }
    const int d = 32 * (dh * NDB + j) + l32;
    if (d >= D) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = kw * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kl < sp.b) {
        const int p = sp.a + kl;
        const int64_t row = (AG ? (int64_t)agm.row(p) : (int64_t)p) * Hkv + kvh;
        dv[row * D + d] = va[r];
        dk[row * D + d] = ka[r] * prm.scale;
      }
    }
  }
}

template <int DP, bool AG>
static int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv, char* ws, const PlanLayout& lay,
                      const AttnParams& prm, int32_t* status, unsigned grid_q, unsigned grid_kv,
                      hipStream_t stream, hipEvent_t* ev, int nev) {
  constexpr int QB = kDqRowBlocks;
  int e = launch(attn_bwd_dq_kernel<DP, QB, AG>, dim3(grid_q * kDqSplit), dim3(64 * (kQWaves / QB / kDqSplit)), 0,
                 stream, ev, nev, 1, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                 (const uint16_t*)dout, lse, dq, ws, lay, prm, status);
  if (e) return e;
  constexpr int SD = DP >= 64 ? kDkdvSplit : 1;
  e = launch(attn_bwd_dkdv_kernel<DP, SD, AG>, dim3(grid_kv), dim3(256 * SD), 0, stream, ev, nev, 2,
             (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, dk, dv, ws, lay,
             prm, status);
  if (e) return e;
  if (lay.max_parts < 2) return skip_launch(ev, nev, 3, stream);   // a workspace without partial slots: no split tile
  const int64_t nq = prm.qsplit ? split_grid(prm, lay) * (kRowsPerWG / 32) : 0, nkv = split_grid(prm, lay) * 4 * SD;
  return launch(attn_bwd_merge_kernel<DP, SD, AG>, dim3((unsigned)(nq + nkv)), dim3(64), 0, stream, ev, nev, 3, dq,
                dk, dv, (const char*)ws, lay, prm, status, (int)nq);
}

template <bool AG>
static int dispatch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, float* dq, float* dk, float* dv, char* ws, const PlanLayout& lay,
                        const AttnParams& prm, int32_t* status, unsigned gq, unsigned gkv, hipStream_t stream,
                        hipEvent_t* ev, int nev) {
  switch (prm.D) {
    case 16:
    case 32: return launch_bwd<32, AG>(q, k, v, o, dout, lse, dq, dk, dv, ws, lay, prm, status, gq, gkv, stream, ev, nev);
    case 64: return launch_bwd<64, AG>(q, k, v, o, dout, lse, dq, dk, dv, ws, lay, prm, status, gq, gkv, stream, ev, nev);
    default: return launch_bwd<128, AG>(q, k, v, o, dout, lse, dq, dk, dv, ws, lay, prm, status, gq, gkv, stream, ev, nev);
  }
}

static int attn_bwd_entry(const void* q_local, const void* k, const void* v, const void* o_local,
                          const void* do_local, const float* lse_local, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                          int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                          int32_t causal, int32_t window_left, int32_t window_right, float* dq_local, float* dk,
                          float* dv, void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream,
                          hipEvent_t* events, int32_t n_events, bool allgathered) {
  if (!q_local || !k || !v || !o_local || !do_local || !lse_local || !dq_local || !dk || !dv || !cu_seqlens ||
      !cu_seqlens_padded)
    return CPTHD_ERR_NULL;
  PlanLayout lay;
  AttnParams prm;
  if (int e = check_attn_args(total_tokens, capacity_tokens, cp_size, rank, strategy, num_docs, num_q_heads,
                              num_kv_heads, head_dim, causal, window_left, window_right, workspace,
                              workspace_bytes, lay, prm))
    return e;
  const bool ag = allgathered && strategy != CPTHD_NO_LOAD_BALANCE;
  if (ag) {
    if (int e = check_allgathered_bytes(total_tokens, num_kv_heads, head_dim)) return e;
  }
  prm.scale = softmax_scale;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  const int64_t gq = qtile_grid(prm, lay);
  const int64_t gkv = kvtile_grid(prm, lay);
  if (gq * kDqSplit > INT32_MAX || gkv > INT32_MAX) return CPTHD_ERR_TOKENS;   // more work-groups than one launch takes
  if (int e = device_cus(prm)) return e;
  char* ws = (char*)workspace;
  if (int e = launch_plan(cu_seqlens, cu_seqlens_padded, prm, ws, lay, true, dev_status, stream, events, n_events, 0))
    return e;
  return ag ? dispatch_bwd<true>(q_local, k, v, o_local, do_local, lse_local, dq_local, dk, dv, ws, lay, prm,
                                 dev_status, gq, gkv, stream, events, n_events)
            : dispatch_bwd<false>(q_local, k, v, o_local, do_local, lse_local, dq_local, dk, dv, ws, lay, prm,
                                  dev_status, gq, gkv, stream, events, n_events);
}

}  // namespace cpthd

using namespace cpthd;

#define CPTHD_BWD_ARGS                                                                                                \
  const void *q_local, const void *k, const void *v, const void *o_local, const void *do_local,                     \
      const float *lse_local, const int32_t *cu_seqlens, const int32_t *cu_seqlens_padded, int32_t num_docs,        \
      int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,              \
      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,            \
      int32_t window_left, int32_t window_right, float *dq_local, float *dk, float *dv, void *workspace,           \
      size_t workspace_bytes, int32_t *dev_status, hipStream_t stream
#define CPTHD_BWD_PASS                                                                                                \
  q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens,               \
      capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal,        \
      window_left, window_right, dq_local, dk, dv, workspace, workspace_bytes, dev_status, stream

extern "C" int cpthd_attn_bwd(CPTHD_BWD_ARGS) {
  return attn_bwd_entry(CPTHD_BWD_PASS, nullptr, 0, false);
}

extern "C" int cpthd_attn_bwd_allgathered(CPTHD_BWD_ARGS) {
  return attn_bwd_entry(CPTHD_BWD_PASS, nullptr, 0, true);
}

extern "C" int cpthd_attn_bwd_timed(CPTHD_BWD_ARGS, int32_t kv_allgathered, hipEvent_t* events, int32_t n_events) {
  return attn_bwd_entry(CPTHD_BWD_PASS, events, n_events, kv_allgathered != 0);
}

// ---------------------------------------------------------------------------
// allocation-free backward: the workspace is a fixed device array
// ---------------------------------------------------------------------------
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc).  The array lives in the library's
// code object: every GPU the library runs on holds its own copy until the
// process ends, and every call on that GPU shares it (the plan it leaves is
// checked and rebuilt like any workspace's, and the -delta / LSE rows are
// written before they are read, so nothing needs clearing).
static __device__ __align__(256) char scratch[CPTHD_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // the array's device address on each device, taken once

// The current device's copy of the array.  In host code `scratch` only names a
// host-side stand-in, so its device address comes from hipGetSymbolAddress.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CPTHD_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CPTHD_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CPTHD_OK;
}
}  // namespace

extern "C" int cpthd_attn_bwd_noalloc(const void* q_local, const void* k, const void* v, const void* o_local,
                                      const void* do_local, const float* lse_local, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                                      int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float softmax_scale, int32_t causal, int32_t window_left,
                                      int32_t window_right, float* dq_local, float* dk, float* dv,
                                      int32_t* dev_status, hipStream_t stream) {
  if (!q_local || !k || !v || !o_local || !do_local || !lse_local || !dq_local || !dk || !dv || !cu_seqlens ||
      !cu_seqlens_padded)
    return CPTHD_ERR_NULL;
  // the host checks of cpthd_attn_bwd against the array's size (a stand-in address: nothing is dereferenced),
  // so a call the array cannot hold is refused before any device is touched
  {
    PlanLayout lay;
    AttnParams prm;
    if (int e = check_attn_args(total_tokens, capacity_tokens, cp_size, rank, strategy, num_docs, num_q_heads,
                                num_kv_heads, head_dim, causal, window_left, window_right,
                                reinterpret_cast<void*>(uintptr_t(256)), CPTHD_STATIC_SCRATCH_BYTES, lay, prm))
      return e == CPTHD_ERR_WORKSPACE ? CPTHD_ERR_SCRATCH : e;
  }
  void* ws = nullptr;
  if (int e = scratch_address(&ws)) return e;
  return attn_bwd_entry(q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs,
                        total_tokens, capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim,
                        softmax_scale, causal, window_left, window_right, dq_local, dk, dv, ws,
                        CPTHD_STATIC_SCRATCH_BYTES, dev_status, stream, nullptr, 0, false);
}
