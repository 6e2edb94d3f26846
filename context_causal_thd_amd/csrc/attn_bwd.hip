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
#ifndef CPTHD_BWD_FUSED
#define CPTHD_BWD_FUSED 0   // head dim 64 / 128: one backward pass with dQ atomics instead of two passes
#endif
constexpr bool kBwdFused = CPTHD_BWD_FUSED;
#ifndef CPTHD_FUSED_KD_REGS
#define CPTHD_FUSED_KD_REGS 0   // one-pass backward: the dQ product's K operand held in registers (else read per step)
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
  const int tile = blockIdx.x / (prm.Hkv * kDqSplit), part = (blockIdx.x / prm.Hkv) % kDqSplit;
  // the tile is read beside the header (the workspace holds a tile slot for
  // every query tile the launch can have); it is used only once both check out
  const QTile t = reinterpret_cast<const QTile*>(ws + lay.qtiles)[tile];
  if (!tile_usable(plan_matches(hdr, prm, lay), tile < hdr->n_qtiles, check_qtile(t, prm), status)) return;
  float* ndelta = reinterpret_cast<float*>(ws + lay.delta);   // -delta per row, for the key-tile pass
  float* lse2w = reinterpret_cast<float*>(ws + lay.lse2);

  const int tid = threadIdx.x, wave = wave_index(), lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv;
  const int bm = kRowsPerWG / G;
  // a work-group holding none of the tile's rows (the tile has at most
  // part * kRowsPerWG / kDqSplit of them) has nothing to write: it leaves
  // before issuing any load
  const int m_first = part * (kRowsPerWG / kDqSplit);
  if (m_first >= bm * G || m_first / G >= t.ntok) return;

  // K/V rows [ds, kv_end) as in the forward (physical or all-gathered order)
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
  const int kend = t.kv_end;
  const int nsteps = (kend - t.ds + kKvStep - 1) / kKvStep;
  const int64_t kv0 = AG ? 0 : (int64_t)t.ds * Hkv * D;
  const uint32_t kv_bytes = AG ? (uint32_t)prm.T * row_bytes : (uint32_t)(kend - t.ds) * row_bytes;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + kv0, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + kv0, kv_bytes);
  TileLoader<DP, true, NW> kvld;
  AgMap agm;
  AgCursor cur{0, 0};
  if constexpr (AG) {
    agm = ag_map(reinterpret_cast<const DocSeg*>(ws + lay.docs)[t.doc], prm);
    agm.chunk_of(t.ds, cur.j, cur.start);
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
  if (nsteps > 0) issue_kv(t.ds, K0, V0);

  bool row_in[QB], valid[QB];
  int p_q[QB];
  int64_t qrow[QB];
  float dlt[QB], lse2[QB];
  bf16x8 qf[QB][DP / 16], df[QB][DP / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = part * (kRowsPerWG / kDqSplit) + wave * 32 * QB + 32 * qb + l32;
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
    if (it + 1 < nsteps) issue_kv(kb + kKvStep, Kn, Vn);
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
  if (wave_active) {
    for (int it = 0; it < nsteps; it += 2) {
      step(it, K0, V0, K1, V1);
      if (it + 1 < nsteps) step(it + 1, K1, V1, K0, V0);
    }
  } else {
    // the same loads and barriers, no products
    for (int it = 0; it < nsteps; it += 2) {
      if (it + 1 < nsteps) issue_kv(t.ds + (it + 1) * kKvStep, K1, V1);
      lds_loads_barrier();
      if (it + 1 < nsteps) {
        if (it + 2 < nsteps) issue_kv(t.ds + (it + 2) * kKvStep, K0, V0);
        lds_loads_barrier();
      }
    }
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
    float* __restrict__ dv, const char* __restrict__ ws, PlanLayout lay, AttnParams prm, int32_t* status) {
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
                     (kt.nkeys <= kKeysPerWG) & (kt.k0 <= prm.T - kt.nkeys);
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
  if (nchunks > 0) issue(0, Q0, O0, L0, E0);

  bf16x8 kf[DP / 16], vf[DP / 16];
#pragma unroll
  for (int s = 0; s < DP / 16; ++s) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    const int d = 16 * s + 8 * h;
    if (key_in && d < D && nchunks > 0) {   // a tile no row of the rank sees only writes zeros
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
    if (i + 1 < nchunks) issue(i + 1, Qn, On, Ln, En);
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
  for (int i = 0; i < nchunks; i += 2) {
    step(i, Q0, O0, L0, E0, Q1, O1, L1, E1);
    if (i + 1 < nchunks) step(i + 1, Q1, O1, L1, E1, Q0, O0, L0, E0);
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
// one-pass backward: the key-tile pass that also accumulates dQ
// ---------------------------------------------------------------------------
// The key-tile pass above holds dS for 128 keys and 64 query rows at every
// step; dQ of those rows is dS K over the tile's keys.  This variant computes it
// there, so the query-tile pass and its recompute of S and dP go away: a small
// prologue writes -delta and LSE*log2(e) per row and zeroes dQ, and every key
// tile adds its partial dQ with fp32 atomics (the order of the additions, and so
// the last bits of dQ, depend on the schedule).
//   - the tile's K rows sit in LDS: the S products read their K operand by rows
//     from it, and each wave keeps the dQ product's K operand (its 32 dQ columns
//     over the 128 keys, read once through the transpose read) in registers;
//   - the waves write P and dS of their 32 query rows as [key][query] tiles in
//     LDS: the partner wave of the key group reads its dK/dV operands from them by
//     rows, and every wave reads the dQ product's dS operand through the
//     transpose read;
//   - wave w computes dQ for query block w/4 and columns 32*(w%4) .. +31 over all
//     128 keys (8 products) and issues its 16 atomic adds per lane at the start of
//     the next step, after that step's loads, so the end-of-step wait (which
//     counts both) gives them a whole step to complete.
// Needs SD = 2 (head dim 64 or 128): eight waves, two per key group, and a power-of-two G.
// Measured, and not the default (CPTHD_BWD_FUSED=0): parity-green, but 2.3x (t32768_gqa32x8) to 4.7x
// (t131072_gqa64x8) slower than the two passes.  Each key tile adds 128 x D floats per 64-row step, 10-33 GB
// of atomic adds per step of those workloads, and the chip's L2 retires fp32 atomic adds at about 1 TB/s.
template <int DP, bool AG>
__global__ __launch_bounds__(512, 1) CPTHD_WAVES_PER_EU(2) void attn_bwd_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    const char* __restrict__ ws, PlanLayout lay, AttnParams prm, int32_t* status) {
  constexpr int NW = 8;
  constexpr int NDB = DP / 64;       // 32-column blocks of dK/dV per wave (the pair splits the head dim)
  using QT = LdsTile<DP, true>;      // Q, dO (64 rows) and the two halves of the tile's K (64 keys each)
  using PT = LdsTile<64, true>;      // P and dS: [key][query], two 64-key halves each
  __shared__ __align__(16) uint16_t Q0[QT::ELEMS], Q1[QT::ELEMS];
  __shared__ __align__(16) uint16_t O0[QT::ELEMS], O1[QT::ELEMS];
  __shared__ __align__(16) float L0[kQChunk], L1[kQChunk], E0[kQChunk], E1[kQChunk];   // LSE*log2(e), -delta
  // keys 0-63 and 64-127 of K, P and dS.  Each pair is one array (halves indexed by the key group), so every LDS
  // access has one underlying object and the compiler can tell it from the in-flight direct loads into Q / dO
  __shared__ __align__(16) uint16_t K2[2 * QT::ELEMS];
  __shared__ __align__(16) uint16_t P2[2 * PT::ELEMS], S2[2 * PT::ELEMS];
  uint16_t* const KA = K2;
  uint16_t* const KB = K2 + QT::ELEMS;
  uint16_t* const SA = S2;
  uint16_t* const SB = S2 + PT::ELEMS;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  const int tile = blockIdx.x / prm.Hkv, kvh = blockIdx.x - (blockIdx.x / prm.Hkv) * prm.Hkv;
  const KVTile kt = reinterpret_cast<const KVTile*>(ws + lay.kvtiles)[tile];
  const bool kt_ok = (kt.doc >= 0) & (kt.doc < prm.num_docs) & (kt.k0 >= 0) & (kt.nkeys >= 0) &
                     (kt.nkeys <= kKeysPerWG) & (kt.k0 <= prm.T - kt.nkeys);
  if (!tile_usable(plan_matches(hdr, prm, lay), tile < hdr->n_kvtiles, kt_ok, status)) return;
  const DocSeg ds = reinterpret_cast<const DocSeg*>(ws + lay.docs)[kt.doc];
  const bool ds_ok = docseg_ok(ds, prm) &
                     (!AG | (prm.strategy != kDCS) |
                      ((kt.k0 >= ds.ds) & (kt.k0 - ds.ds <= 2 * prm.cp * ds.na - kt.nkeys)));
  if (!tile_usable(true, true, ds_ok, status)) return;
  const float* ndelta = reinterpret_cast<const float*>(ws + lay.delta);
  const float* lse2w = reinterpret_cast<const float*>(ws + lay.lse2);

  const int tid = threadIdx.x, wave = wave_index(), lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv, S = prm.S;
  const int kw = wave & 3, dh = wave >> 2;
  const int key = kt.k0 + kw * 32 + l32;
  const bool key_in = kw * 32 + l32 < kt.nkeys;
  AgMap agm;
  if constexpr (AG) agm = ag_map(ds, prm);
  auto kv_row = [&](int p) __attribute__((always_inline)) -> int64_t {
    if constexpr (AG) return (int64_t)agm.row(p) * Hkv + kvh;
    return (int64_t)p * Hkv + kvh;
  };
  const int64_t krow = kv_row(key);

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
  auto chunk_at = [&](int i, int& c0, int& l0, int& ntok) __attribute__((always_inline)) {
    i = nchunks - 1 - i;   // last chunk first (concurrent key tiles of a document share their Q / dO reads)
    const int si = i < nch[0] ? 0 : 1;
    c0 = plo[si] + (i - (si ? nch[0] : 0)) * tpc;
    l0 = sl[si] + (c0 - sp[si]);
    ntok = min(tpc, phi[si] - c0);
  };

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
  if (nchunks > 0) issue(0, Q0, O0, L0, E0);

  // the tile's K rows into LDS (plain loads and stores; once per work-group), V of the lane's key in registers
  {
    constexpr int CPR = DP / 8;   // 16-byte pieces per row
#pragma unroll
    for (int i = 0; i < (kKeysPerWG * CPR + 511) / 512; ++i) {
      const int pc = tid + 512 * i;
      const int kk = pc / CPR, ch = pc - kk * CPR;
      if (kk < kKeysPerWG) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (kk < kt.nkeys && ch * 8 < D && nchunks > 0)
          val = *reinterpret_cast<const u32x4*>(k + kv_row(kt.k0 + kk) * D + ch * 8);
        uint16_t* Kt = kk < 64 ? KA : KB;
        *reinterpret_cast<u32x4*>(Kt + QT::row(kk & 63) * QT::STRIDE + ch * 8) = val;
      }
    }
  }
  bf16x8 vf[DP / 16];
#pragma unroll
  for (int s = 0; s < DP / 16; ++s) {
    u32x4 b = {0u, 0u, 0u, 0u};
    const int d = 16 * s + 8 * h;
    if (key_in && d < D && nchunks > 0) b = *reinterpret_cast<const u32x4*>(v + krow * D + d);
    vf[s] = as_bf16x8(b);
  }
  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    dka[j] = f32x16{};
    dva[j] = f32x16{};
  }
  lds_loads_barrier();

  // dQ of this wave: query block qbq, columns 32*dbq .. +31; its K operand over the 128 keys in registers
  const int qbq = wave >> 2, dbq = wave & 3;
  const bool dq_cols = 32 * dbq < D;
  const int dq_c0 = dq_cols ? 32 * dbq : 0;
#if CPTHD_FUSED_KD_REGS
  bf16x8 kd[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    kd[s] = lds_tr8<DP, true>(s < 4 ? KA : KB, 16 * (s & 3) + 4 * h, 16 * (s & 3) + 8 + 4 * h, dq_c0);
#endif

  const float sl2 = prm.scale_log2;
  const int kmax = kt.k0 + kt.nkeys - 1;
  const uint16_t* Kown = K2 + (kw >> 1) * QT::ELEMS;   // this wave's 32 keys: rows 32*(kw%2) .. of one half
  uint16_t* Pown = P2 + (kw >> 1) * PT::ELEMS;
  uint16_t* Sown = S2 + (kw >> 1) * PT::ELEMS;
  const int krow_lds = 32 * (kw & 1) + l32;

  // dQ atomics of one step: rows of query block qbq (row r of the step = token r / G, head r % G)
  f32x16 dqa = f32x16{};
  int pend_l0 = 0, pend_rows = 0;   // the pending step's first local row and its query rows (tokens * G)
  // G is a power of two on this path: row r of a step is token r >> lg, head r & (G - 1)
  const int lg = __builtin_ctz((unsigned)G), gm = G - 1;
  auto flush_dq = [&]() __attribute__((always_inline)) {
    if (!dq_cols) return;
    // the lane's rows are recomputed at every flush: kept across the loop, their 16 offsets would cost registers
    int hh = h;
    asm volatile("" : "+v"(hh));
    const int q0 = 32 * qbq + 4 * hh;
    float* base = dq + ((int64_t)pend_l0 * Hq + kvh * G) * D + 32 * dbq + l32;
    const float sc = prm.scale;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = q0 + 8 * (r >> 2) + (r & 3);
      if (qr < pend_rows) atomicAdd(base + ((qr >> lg) * Hq + (qr & gm)) * D, dqa[r] * sc);
    }
  };

  auto step = [&](int i, const uint16_t* Qt, const uint16_t* Dt, const float* Lt, const float* Et, uint16_t* Qn,
                  uint16_t* On, float* Ln, float* En) __attribute__((always_inline)) {
    int c0, l0, ntok;
    chunk_at(i, c0, l0, ntok);
    if (i + 1 < nchunks) issue(i + 1, Qn, On, Ln, En);
    if (i > 0) flush_dq();   // the previous step's dQ, behind this step's loads
    __builtin_amdgcn_sched_barrier(0);   // (its registers free before the score products)
    const bool need_mask = kmax > c0;
    const int thr = (key - c0) * G - 4 * h;
    // P and dS of this wave's query block dh (key as the lane index)
    bf16x8 pd[4];
    {
      f32x16 sc = f32x16{}, dp;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(Et + 32 * dh + 8 * g4 + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * g4 + j] = e4[j];
      }
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        sc = mfma32(lds_row8<DP, true>(Qt, 32 * dh + l32, 16 * s, h), lds_row8<DP, true>(Kown, krow_lds, 16 * s, h),
                    sc);
        dp = mfma32(lds_row8<DP, true>(Dt, 32 * dh + l32, 16 * s, h), vf[s], dp);
      }
      auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + 32 * dh + 8 * g4 + 4 * h);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * g4 + j;
            float pv = exp2_fast(fmaf(sc[r], sl2, -l4[j]));
            if constexpr (decltype(masked)::value)
              if (32 * dh + 8 * g4 + j < thr) pv = 0.f;
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
    }
    // P and dS as [key][query] rows: query 32*dh + 8*g4 + 4h .. +3 is one 8-byte piece of the lane's key row
    {
      const int base = PT::row(krow_lds) * PT::STRIDE + 32 * dh + 4 * h;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 p4 = __builtin_bit_cast(u32x4, pd[j]);
        const u32x4 s4 = __builtin_bit_cast(u32x4, pd[2 + j]);
        *reinterpret_cast<u32x2*>(Pown + base + 16 * j) = u32x2{p4.x, p4.y};
        *reinterpret_cast<u32x2*>(Pown + base + 16 * j + 8) = u32x2{p4.z, p4.w};
        *reinterpret_cast<u32x2*>(Sown + base + 16 * j) = u32x2{s4.x, s4.y};
        *reinterpret_cast<u32x2*>(Sown + base + 16 * j + 8) = u32x2{s4.z, s4.w};
      }
    }
    // dV += P^T dO, dK += dS^T Q for one query block over this wave's column blocks
    auto accumulate = [&](int qb, const bf16x8 (&p)[4]) __attribute__((always_inline)) {
      const int r0 = 32 * qb + 4 * h;
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        const int c0l = 32 * (dh * NDB + j);
        dva[j] = mfma32(p[0], lds_tr8<DP, true>(Dt, r0, r0 + 8, c0l), dva[j]);
        dva[j] = mfma32(p[1], lds_tr8<DP, true>(Dt, r0 + 16, r0 + 24, c0l), dva[j]);
        dka[j] = mfma32(p[2], lds_tr8<DP, true>(Qt, r0, r0 + 8, c0l), dka[j]);
        dka[j] = mfma32(p[3], lds_tr8<DP, true>(Qt, r0 + 16, r0 + 24, c0l), dka[j]);
      }
    };
    accumulate(dh, pd);
    lds_barrier();   // every wave's P and dS of the step are in LDS
    {
      // the partner's block: its P and dS rows of this lane's key
      const int base = PT::row(krow_lds) * PT::STRIDE + 32 * (dh ^ 1) + 4 * h;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(Pown + base + 16 * j);
        const u32x2 b = *reinterpret_cast<const u32x2*>(Pown + base + 16 * j + 8);
        const u32x2 c = *reinterpret_cast<const u32x2*>(Sown + base + 16 * j);
        const u32x2 e = *reinterpret_cast<const u32x2*>(Sown + base + 16 * j + 8);
        pd[j] = as_bf16x8(u32x4{a.x, a.y, b.x, b.y});
        pd[2 + j] = as_bf16x8(u32x4{c.x, c.y, e.x, e.y});
      }
      accumulate(dh ^ 1, pd);
    }
    // dQ[query][col] = sum over the 128 keys of dS[query][key] K[key][col] (scaled at the atomic add)
    dqa = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#if CPTHD_FUSED_KD_REGS
      const bf16x8 kop = kd[s];
#else
      const bf16x8 kop = lds_tr8<DP, true>(s < 4 ? KA : KB, 16 * (s & 3) + 4 * h, 16 * (s & 3) + 8 + 4 * h, dq_c0);
#endif
      dqa = mfma32(lds_tr8<64, true>(s < 4 ? SA : SB, 16 * (s & 3) + 4 * h, 16 * (s & 3) + 8 + 4 * h, 32 * qbq),
                   kop, dqa);
    }
    pend_l0 = l0;
    pend_rows = ntok * G;
    lds_loads_barrier();
  };
  for (int i = 0; i < nchunks; i += 2) {
    step(i, Q0, O0, L0, E0, Q1, O1, L1, E1);
    if (i + 1 < nchunks) step(i + 1, Q1, O1, L1, E1, Q0, O0, L0, E0);
  }
  if (nchunks > 0) flush_dq();

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

// Prologue of the one-pass backward: per local row and q head, -delta = -rowsum(dO * O) and LSE * log2(e) into the
// workspace, and that row of dQ set to zero (the key tiles add into it).  Sixteen lanes per row: 4 rows per wave.
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ lse, float* __restrict__ dq,
                                                            char* __restrict__ ws, PlanLayout lay, int64_t rows,
                                                            int D) {
  float* ndelta = reinterpret_cast<float*>(ws + lay.delta);
  float* lse2w = reinterpret_cast<float*>(ws + lay.lse2);
  const int sub = threadIdx.x & 15;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x / 16);
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x / 16) + (threadIdx.x >> 4); r < rows; r += stride) {
    float acc = 0.f;
    for (int c = 8 * sub; c < D; c += 128) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(dout + r * D + c);
      const u32x4 b = *reinterpret_cast<const u32x4*>(o + r * D + c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16) +
               __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(b[i] & 0xFFFF0000u);
      *reinterpret_cast<f32x4*>(dq + r * D + c) = f32x4{};
      *reinterpret_cast<f32x4*>(dq + r * D + c + 4) = f32x4{};
    }
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (sub == 0) {
      ndelta[r] = -acc;
      lse2w[r] = lse[r] * 1.4426950408889634f;
    }
  }
}

template <int DP, bool AG>
static int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv, char* ws, const PlanLayout& lay,
                      const AttnParams& prm, int32_t* status, unsigned grid_q, unsigned grid_kv,
                      hipStream_t stream, hipEvent_t* ev, int nev) {
  if (kBwdFused && DP >= 64 && (prm.G & (prm.G - 1)) == 0) {
    // one pass: prologue (-delta, LSE*log2(e), dQ = 0), then the key tiles with dQ atomics
    const int64_t rows = (int64_t)prm.S * prm.Hq;
    const unsigned gp = (unsigned)std::min<int64_t>((rows + 15) / 16, 4096);
    int e = launch(attn_bwd_prep_kernel, dim3(gp), dim3(256), 0, stream, ev, nev, 1, (const uint16_t*)o,
                   (const uint16_t*)dout, lse, dq, ws, lay, rows, prm.D);
    if (e) return e;
    return launch(attn_bwd_fused_kernel<(DP >= 64 ? DP : 64), AG>, dim3(grid_kv), dim3(512), 0, stream, ev, nev, 2,
                  (const uint16_t*)q,
                  (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, dq, dk, dv, (const char*)ws, lay,
                  prm, status);
  }
  constexpr int QB = kDqRowBlocks;
  int e = launch(attn_bwd_dq_kernel<DP, QB, AG>, dim3(grid_q * kDqSplit), dim3(64 * (kQWaves / QB / kDqSplit)), 0,
                 stream, ev, nev, 1, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                 (const uint16_t*)dout, lse, dq, ws, lay, prm, status);
  if (e) return e;
  constexpr int SD = DP >= 64 ? kDkdvSplit : 1;
  return launch(attn_bwd_dkdv_kernel<DP, SD, AG>, dim3(grid_kv), dim3(256 * SD), 0, stream, ev, nev, 2,
                (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, dk, dv,
                (const char*)ws, lay, prm, status);
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
  const int64_t gq = qtile_grid(prm);
  const int64_t gkv = ((total_tokens + kKeysPerWG - 1) / kKeysPerWG + num_docs) * (int64_t)num_kv_heads;
  if (gq * kDqSplit > INT32_MAX || gkv > INT32_MAX) return CPTHD_ERR_TOKENS;   // more work-groups than one launch takes
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
