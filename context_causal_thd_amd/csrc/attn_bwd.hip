// Causal THD attention backward for one CP rank (gfx950).
//
// TransformerEngine PR #3221: forward captures the strategy so backward uses
// the same token layout ("What changed"); backward restores it and "selects
// the matching step layout and K/V ordering" (sequence diagram) to return
// dQ/dK/dV.  With P = softmax of the scores, dP = dO V^T and
// delta = rowsum(dO * O) = rowsum(P * dP):
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// dK/dV here are the rank's partial gradients (its query rows only) over all
// T physical rows; a reduce-scatter over the ranks would sum them.
//
// Two passes, no atomics, deterministic:
//   1. query tiles (the forward's tiles, 64 rows per wave): delta from O and
//      dO, then per 64-key step S^T = K Q^T, P^T = exp2(S^T - LSE),
//      dP^T = V dO^T, dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (the K^T
//      operand comes from the natural K tile through the transpose LDS read);
//   2. key tiles (128 keys of one document, 32 per wave): for every query row
//      of the rank that sees the tile, 64 rows per step, S = Q K^T and
//      dP = dO V^T with the key as the lane index, dS = P (dP - delta),
//      dV += P^T dO and dK += dS^T Q (dO^T and Q^T operands through the
//      transpose read of the natural tiles).
// Both passes load the next step's rows into registers while computing the
// current one and double-buffer their LDS tiles.
#include "attn_common.h"
#include "cpthd_host.h"

namespace cpthd {

// ---------------------------------------------------------------------------
// pass 1: delta and dQ over the query tiles
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dq, char* __restrict__ ws, PlanLayout lay, AttnParams prm, int32_t* status) {
  constexpr int KS = Lds<DP>::kNat;
  __shared__ __align__(16) uint16_t Ks[2][kKvStep * KS];
  __shared__ __align__(16) uint16_t Vs[2][kKvStep * KS];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  if (!plan_matches(hdr, prm)) {
    if (threadIdx.x == 0 && status) atomicOr(status, kDevPlan);
    return;
  }
  const int tile = blockIdx.x / prm.Hkv, kvh = blockIdx.x - (blockIdx.x / prm.Hkv) * prm.Hkv;
  if (tile >= hdr->n_qtiles) return;
  QTile t;
  if (!load_qtile(ws, lay, tile, prm, t)) {
    if (threadIdx.x == 0 && status) atomicOr(status, kDevPlan);
    return;
  }
  float* delta = reinterpret_cast<float*>(ws + lay.delta);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv;
  const int bm = kRowsPerWG / G;

  bool row_in[2], valid[2];
  int p_q[2];
  int64_t qrow[2];
  float dlt[2], lse2[2];
  bf16x8 qf[2][DP / 16], df[2][DP / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int m = wave * kRowsPerWave + 32 * qb + l32;
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
    dlt[qb] = dpart + xor32(dpart);
    if (row_in[qb] && h == 0) delta[qrow[qb]] = valid[qb] ? dlt[qb] : 0.f;
    lse2[qb] = valid[qb] ? lse[qrow[qb]] * 1.4426950408889634f : INFINITY;
  }

  f32x16 acc[2][DP / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) acc[qb][db] = f32x16{};

  const int kend = t.kv_end;
  TileRegs<DP, kKvStep> kr, vr;
  auto fetch = [&](int kb) {
    auto key_row = [&](int r) -> int64_t {
      const int kabs = kb + r;
      return kabs < kend ? (int64_t)kabs * Hkv + kvh : -1;
    };
    kr.load(k, D, key_row);
    vr.load(v, D, key_row);
  };
  const int nsteps = (kend - t.ds + kKvStep - 1) / kKvStep;
  if (nsteps > 0) {
    fetch(t.ds);
    kr.store(Ks[0], KS);
    vr.store(Vs[0], KS);
  }
  __syncthreads();

  const float sl2 = prm.scale_log2;
  for (int it = 0; it < nsteps; ++it) {
    const int kb = t.ds + it * kKvStep;
    const int buf = it & 1;
    if (it + 1 < nsteps) fetch(kb + kKvStep);
    const uint16_t* Kt = Ks[buf];
    const uint16_t* Vt = Vs[buf];
    const bool need_mask = kb + kKvStep - 1 > t.p0;

    bf16x8 dsb[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        const bf16x8 ka = lds_row8(Kt, KS, 32 * b + l32, 16 * s, h);
        const bf16x8 va = lds_row8(Vt, KS, 32 * b + l32, 16 * s, h);
        sc[0] = mfma32(ka, qf[0][s], sc[0]);
        sc[1] = mfma32(ka, qf[1][s], sc[1]);
        dp[0] = mfma32(va, df[0][s], dp[0]);
        dp[1] = mfma32(va, df[1][s], dp[1]);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = exp2_fast(fmaf(sc[qb][r], sl2, -lse2[qb]));
          if (need_mask) {
            const int key = kb + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > p_q[qb]) pv = 0.f;
          }
          sc[qb][r] = pv * (dp[qb][r] - dlt[qb]);
        }
        dsb[qb][2 * b] = acc_to_bf16(sc[qb], 0);
        dsb[qb][2 * b + 1] = acc_to_bf16(sc[qb], 8);
      }
    }
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = lds_tr8(Kt, KS, 16 * ks + 4 * h, 16 * ks + 8 + 4 * h, 32 * db);
        acc[0][db] = mfma32(a, dsb[0][ks], acc[0][db]);
        acc[1][db] = mfma32(a, dsb[1][ks], acc[1][db]);
      }

    if (it + 1 < nsteps) {
      kr.store(Ks[buf ^ 1], KS);
      vr.store(Vs[buf ^ 1], KS);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
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
template <int DP>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ dk,
    float* __restrict__ dv, const char* __restrict__ ws, PlanLayout lay, AttnParams prm, int32_t* status) {
  constexpr int QS = Lds<DP>::kNat;
  __shared__ __align__(16) uint16_t Qs[2][kQChunk * QS];
  __shared__ __align__(16) uint16_t Ds[2][kQChunk * QS];
  __shared__ float s_lse2[2][kQChunk], s_delta[2][kQChunk];
  __shared__ int s_pq[2][kQChunk];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(ws);
  if (!plan_matches(hdr, prm)) {
    if (threadIdx.x == 0 && status) atomicOr(status, kDevPlan);
    return;
  }
  const int tile = blockIdx.x / prm.Hkv, kvh = blockIdx.x - (blockIdx.x / prm.Hkv) * prm.Hkv;
  if (tile >= hdr->n_kvtiles) return;
  const KVTile kt = reinterpret_cast<const KVTile*>(ws + lay.kvtiles)[tile];
  if (kt.doc < 0 || kt.doc >= prm.num_docs || kt.k0 < 0 || kt.nkeys < 0 || kt.nkeys > kKeysPerWG ||
      kt.k0 > prm.T - kt.nkeys) {
    if (threadIdx.x == 0 && status) atomicOr(status, kDevPlan);
    return;
  }
  const DocSeg ds = reinterpret_cast<const DocSeg*>(ws + lay.docs)[kt.doc];
  const float* delta = reinterpret_cast<const float*>(ws + lay.delta);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv, S = prm.S;
  const int key = kt.k0 + wave * 32 + l32;          // this lane's key (B operand column)
  const bool key_in = wave * 32 + l32 < kt.nkeys;
  const int64_t krow = (int64_t)key * Hkv + kvh;

  bf16x8 kf[DP / 16], vf[DP / 16];
#pragma unroll
  for (int s = 0; s < DP / 16; ++s) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    const int d = 16 * s + 8 * h;
    if (key_in && d < D) {
      a = *reinterpret_cast<const u32x4*>(k + krow * D + d);
      b = *reinterpret_cast<const u32x4*>(v + krow * D + d);
    }
    kf[s] = as_bf16x8(a);
    vf[s] = as_bf16x8(b);
  }
  f32x16 dka[DP / 32], dva[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

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
  auto chunk_c0 = [&](int i, int& si) {
    si = i < nch[0] ? 0 : 1;
    return plo[si] + (i - (si ? nch[0] : 0)) * tpc;
  };

  TileRegs<DP, kQChunk> qr, dr;
  float pf_lse = INFINITY, pf_delta = 0.f;
  int pf_pq = -1;
  auto fetch = [&](int i) {
    int si;
    const int c0 = chunk_c0(i, si);
    const int ntok = min(tpc, phi[si] - c0);
    const int l0 = sl[si] + (c0 - sp[si]);
    auto qrow_of = [&](int r) -> int64_t {
      const int t2 = r / G;
      return (r < tpc * G && t2 < ntok) ? (int64_t)(l0 + t2) * Hq + kvh * G + (r - t2 * G) : -1;
    };
    qr.load(q, D, qrow_of);
    dr.load(dout, D, qrow_of);
    if (tid < kQChunk) {
      const int64_t qrw = qrow_of(tid);
      pf_lse = qrw >= 0 ? lse[qrw] * 1.4426950408889634f : INFINITY;
      pf_delta = qrw >= 0 ? delta[qrw] : 0.f;
      pf_pq = qrw >= 0 ? c0 + tid / G : -1;
    }
  };
  auto stage = [&](int buf) {
    qr.store(Qs[buf], QS);
    dr.store(Ds[buf], QS);
    if (tid < kQChunk) {
      s_lse2[buf][tid] = pf_lse;
      s_delta[buf][tid] = pf_delta;
      s_pq[buf][tid] = pf_pq;
    }
  };
  if (nchunks > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();

  const float sl2 = prm.scale_log2;
  const int kmax = kt.k0 + kt.nkeys - 1;
  for (int i = 0; i < nchunks; ++i) {
    const int buf = i & 1;
    int si;
    const int c0 = chunk_c0(i, si);
    if (i + 1 < nchunks) fetch(i + 1);
    const bool need_mask = kmax > c0;   // some key of the tile lies after the step's first row
    const uint16_t* Qt = Qs[buf];
    const uint16_t* Dt = Ds[buf];
#pragma unroll
    for (int qb = 0; qb < kQChunk / 32; ++qb) {
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        sc = mfma32(lds_row8(Qt, QS, 32 * qb + l32, 16 * s, h), kf[s], sc);
        dp = mfma32(lds_row8(Dt, QS, 32 * qb + l32, 16 * s, h), vf[s], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
        float pv = exp2_fast(fmaf(sc[r], sl2, -s_lse2[buf][qi]));
        if (need_mask && key > s_pq[buf][qi]) pv = 0.f;
        sc[r] = pv;
        dp[r] = pv * (dp[r] - s_delta[buf][qi]);
      }
      const bf16x8 p0 = acc_to_bf16(sc, 0), p1 = acc_to_bf16(sc, 8);
      const bf16x8 s0 = acc_to_bf16(dp, 0), s1 = acc_to_bf16(dp, 8);
#pragma unroll
      for (int db = 0; db < DP / 32; ++db) {
        const int r0 = 32 * qb + 4 * h;
        dva[db] = mfma32(p0, lds_tr8(Dt, QS, r0, r0 + 8, 32 * db), dva[db]);
        dva[db] = mfma32(p1, lds_tr8(Dt, QS, r0 + 16, r0 + 24, 32 * db), dva[db]);
        dka[db] = mfma32(s0, lds_tr8(Qt, QS, r0, r0 + 8, 32 * db), dka[db]);
        dka[db] = mfma32(s1, lds_tr8(Qt, QS, r0 + 16, r0 + 24, 32 * db), dka[db]);
      }
    }
    if (i + 1 < nchunks) stage(buf ^ 1);
    __syncthreads();
  }

  // dV[key][d] = C[i = key][j = d]: lane holds d = 32*db + l32 for 16 keys of its wave
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) {
    const int d = 32 * db + l32;
    if (d >= D) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kl < kt.nkeys) {
        const int64_t row = (int64_t)(kt.k0 + kl) * Hkv + kvh;
        dv[row * D + d] = dva[db][r];
        dk[row * D + d] = dka[db][r] * prm.scale;
      }
    }
  }
}

template <int DP>
static int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv, char* ws, const PlanLayout& lay,
                      const AttnParams& prm, int32_t* status, unsigned grid_q, unsigned grid_kv,
                      hipStream_t stream, hipEvent_t* ev, int nev) {
  int e = launch(attn_bwd_dq_kernel<DP>, dim3(grid_q), dim3(256), 0, stream, ev, nev, 0, (const uint16_t*)q,
                 (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o, (const uint16_t*)dout, lse, dq, ws,
                 lay, prm, status);
  if (e) return e;
  return launch(attn_bwd_dkdv_kernel<DP>, dim3(grid_kv), dim3(256), 0, stream, ev, nev, 1, (const uint16_t*)q,
                (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, dk, dv, (const char*)ws, lay,
                prm, status);
}

}  // namespace cpthd

using namespace cpthd;

extern "C" int cpthd_attn_bwd(const void* q_local, const void* k, const void* v, const void* o_local,
                              const void* do_local, const float* lse_local, int64_t total_tokens,
                              int64_t capacity_tokens, int32_t num_docs, int32_t cp_size, int32_t rank,
                              int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
                              float* dq_local, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                              int32_t* dev_status, hipStream_t stream, hipEvent_t* events, int32_t n_events) {
  if (!q_local || !k || !v || !o_local || !do_local || !lse_local || !dq_local || !dk || !dv) return CPTHD_ERR_NULL;
  PlanLayout lay;
  AttnParams prm;
  if (int e = check_attn_args(total_tokens, capacity_tokens, cp_size, rank, strategy, num_docs, num_q_heads,
                              num_kv_heads, head_dim, causal, window_left, window_right, workspace,
                              workspace_bytes, lay, prm))
    return e;
  prm.scale = softmax_scale;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  const unsigned gq = qtile_grid(prm);
  const unsigned gkv = (unsigned)(((total_tokens + kKeysPerWG - 1) / kKeysPerWG + num_docs) * num_kv_heads);
  char* ws = (char*)workspace;
  switch (head_dim) {
    case 16:
    case 32:
      return launch_bwd<32>(q_local, k, v, o_local, do_local, lse_local, dq_local, dk, dv, ws, lay, prm, dev_status,
                            gq, gkv, stream, events, n_events);
    case 64:
      return launch_bwd<64>(q_local, k, v, o_local, do_local, lse_local, dq_local, dk, dv, ws, lay, prm, dev_status,
                            gq, gkv, stream, events, n_events);
    default:
      return launch_bwd<128>(q_local, k, v, o_local, do_local, lse_local, dq_local, dk, dv, ws, lay, prm,
                             dev_status, gq, gkv, stream, events, n_events);
  }
}
