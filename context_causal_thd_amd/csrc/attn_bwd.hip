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
//   1. query tiles (the forward's tiles): delta from O and dO, then
//      S^T = K Q^T, P^T = exp2(S^T - LSE), dP^T = V dO^T, dS^T, dQ^T += K^T dS^T;
//   2. key tiles (128 keys of one document, 32 per wave): for every query row of
//      the rank that sees the tile, 64 rows per step,
//      S = Q K^T, dP = dO V^T (key as the lane index), dS,
//      dV += P^T dO, dK += dS^T Q with Q and dO staged transposed in LDS.
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
  __shared__ __align__(16) uint16_t Ks[kKvStep * (DP + 8)];
  __shared__ __align__(16) uint16_t Kt[DP * (kKvStep + 8)];
  __shared__ __align__(16) uint16_t Vs[kKvStep * (DP + 8)];

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
  const int m = wave * 32 + l32;
  const int tt = m / G, g = m - tt * G;
  const bool row_in = m < bm * G && tt < t.ntok;
  const int p_q = t.p0 + tt;
  const bool valid = row_in && p_q < t.ve;
  const int64_t qrow = (int64_t)(t.lrow0 + tt) * Hq + kvh * G + g;

  bf16x8 qf[DP / 16], df[DP / 16];
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < DP / 16; ++s) {
    u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = {0u, 0u, 0u, 0u}, ov = {0u, 0u, 0u, 0u};
    const int d = 16 * s + 8 * h;
    if (valid && d < D) {
      qv = *reinterpret_cast<const u32x4*>(q + qrow * D + d);
      dv4 = *reinterpret_cast<const u32x4*>(dout + qrow * D + d);
      ov = *reinterpret_cast<const u32x4*>(o + qrow * D + d);
    }
    qf[s] = as_bf16x8(qv);
    df[s] = as_bf16x8(dv4);
    const uint16_t* a = reinterpret_cast<const uint16_t*>(&dv4);
    const uint16_t* b = reinterpret_cast<const uint16_t*>(&ov);
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart += __uint_as_float((uint32_t)a[i] << 16) * __uint_as_float((uint32_t)b[i] << 16);
  }
  const float dlt = dpart + xor32(dpart);
  if (row_in && h == 0) delta[qrow] = valid ? dlt : 0.f;
  const float lse2 = valid ? lse[qrow] * 1.4426950408889634f : INFINITY;

  f32x16 acc[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) acc[db] = f32x16{};

  const float sl2 = prm.scale_log2;
  for (int kb = t.ds; kb < t.kv_end; kb += kKvStep) {
    __syncthreads();
    const int kend = t.kv_end;
    auto key_row = [&](int r) -> int64_t {
      const int kabs = kb + r;
      return kabs < kend ? (int64_t)kabs * Hkv + kvh : -1;
    };
    stage_rows<DP, kKvStep, true, true>(k, D, key_row, Ks, Kt);
    stage_rows<DP, kKvStep, true, false>(v, D, key_row, Vs, nullptr);
    __syncthreads();

    const bool need_mask = kb + kKvStep - 1 > t.p0;
    bf16x8 dsb[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        sc = mfma32(lds_a_nat<DP>(Ks, 32 * b + l32, s, h), qf[s], sc);
        dp = mfma32(lds_a_nat<DP>(Vs, 32 * b + l32, s, h), df[s], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_fast(sc[r] * sl2 - lse2);
        if (need_mask) {
          const int key = kb + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > p_q) pv = 0.f;
        }
        sc[r] = pv * (dp[r] - dlt);
      }
      dsb[2 * b] = acc_to_bf16(sc, 0);
      dsb[2 * b + 1] = acc_to_bf16(sc, 8);
    }
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[db] = mfma32(lds_a_trn<kKvStep>(Kt, 32 * db + l32, ks, h), dsb[ks], acc[db]);
  }

  if (!row_in) return;
  const float sc = valid ? prm.scale : 0.f;
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int d0 = 32 * db + 8 * gi + 4 * h;
      if (d0 < D) {
        f32x4 w = {acc[db][4 * gi] * sc, acc[db][4 * gi + 1] * sc, acc[db][4 * gi + 2] * sc, acc[db][4 * gi + 3] * sc};
        *reinterpret_cast<f32x4*>(dq + qrow * D + d0) = w;
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
  __shared__ __align__(16) uint16_t Qs[kQChunk * (DP + 8)];
  __shared__ __align__(16) uint16_t Qt[DP * (kQChunk + 8)];
  __shared__ __align__(16) uint16_t Ds[kQChunk * (DP + 8)];
  __shared__ __align__(16) uint16_t Dt[DP * (kQChunk + 8)];
  __shared__ float s_lse2[kQChunk], s_delta[kQChunk];
  __shared__ int s_pq[kQChunk];

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

  const float sl2 = prm.scale_log2;
  const int tpc = kQChunk / G;   // tokens per step
  const int kmax = kt.k0 + kt.nkeys - 1;
  for (int segi = 0; segi < 2; ++segi) {
    const int sp = segi == 0 ? ds.pa : ds.pb, sn = segi == 0 ? ds.na : ds.nb, sl = segi == 0 ? ds.la : ds.lb;
    const int plo = max(sp, kt.k0), phi = min(sp + sn, ds.ve);
    if (phi <= plo || sl < 0 || sl + (phi - sp) > S) continue;
    for (int c0 = plo; c0 < phi; c0 += tpc) {
      const int ntok = min(tpc, phi - c0);
      const int l0 = sl + (c0 - sp);
      __syncthreads();
      auto qrow_of = [&](int r) -> int64_t {
        const int t2 = r / G;
        return (r < tpc * G && t2 < ntok) ? (int64_t)(l0 + t2) * Hq + kvh * G + (r - t2 * G) : -1;
      };
      stage_rows<DP, kQChunk, true, true>(q, D, qrow_of, Qs, Qt);
      stage_rows<DP, kQChunk, true, true>(dout, D, qrow_of, Ds, Dt);
      if (tid < kQChunk) {
        const int64_t qr = qrow_of(tid);
        s_lse2[tid] = qr >= 0 ? lse[qr] * 1.4426950408889634f : INFINITY;
        s_delta[tid] = qr >= 0 ? delta[qr] : 0.f;
        s_pq[tid] = qr >= 0 ? c0 + tid / G : -1;
      }
      __syncthreads();
      const bool need_mask = kmax > c0;   // some key of the tile lies after the chunk's first row
#pragma unroll
      for (int qb = 0; qb < kQChunk / 32; ++qb) {
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < DP / 16; ++s) {
          sc = mfma32(lds_a_nat<DP>(Qs, 32 * qb + l32, s, h), kf[s], sc);
          dp = mfma32(lds_a_nat<DP>(Ds, 32 * qb + l32, s, h), vf[s], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
          float pv = exp2_fast(sc[r] * sl2 - s_lse2[qi]);
          if (need_mask && key > s_pq[qi]) pv = 0.f;
          sc[r] = pv;
          dp[r] = pv * (dp[r] - s_delta[qi]);
        }
        const bf16x8 p0 = acc_to_bf16(sc, 0), p1 = acc_to_bf16(sc, 8);
        const bf16x8 s0 = acc_to_bf16(dp, 0), s1 = acc_to_bf16(dp, 8);
#pragma unroll
        for (int db = 0; db < DP / 32; ++db) {
          dva[db] = mfma32(p0, lds_a_trn<kQChunk>(Dt, 32 * db + l32, 2 * qb, h), dva[db]);
          dva[db] = mfma32(p1, lds_a_trn<kQChunk>(Dt, 32 * db + l32, 2 * qb + 1, h), dva[db]);
          dka[db] = mfma32(s0, lds_a_trn<kQChunk>(Qt, 32 * db + l32, 2 * qb, h), dka[db]);
          dka[db] = mfma32(s1, lds_a_trn<kQChunk>(Qt, 32 * db + l32, 2 * qb + 1, h), dka[db]);
        }
      }
    }
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
