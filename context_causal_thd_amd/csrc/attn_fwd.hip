// Causal THD attention forward for one CP rank's query rows (gfx950).
//
// TransformerEngine PR #3221, "Scope and constraints": THD self-attention,
// causal without a sliding window (window_size = (-1, 0)); documents stay
// isolated through the sequence metadata ("Logical sequences remain isolated
// by cu_seqlens", review thread).  A local row at physical token p of
// document d attends to the actual keys of d at positions <= p's position.
//
// One work-group = one query tile of the plan (<= 256/G tokens of one segment
// times the G q heads of one kv head: 256 rows, 64 per wave as two 32-row MFMA
// blocks) against its key range [document start, last actual token of the
// tile], 64 keys per step:
//   S^T = K Q^T (bf16 MFMA 32x32x16; K read from LDS once per key block and
//   used for both row blocks; Q in registers),
//   online softmax in fp32 / exp2 with the query as the lane index and a
//   rescale of the running output only when a row maximum grows by more than
//   2^8 (the exponentials stay <= 256, the final normalisation is exact),
//   O^T += V^T P^T (V^T operand straight from the natural V tile through the
//   transpose LDS read; P^T straight from the score registers).
// The next step's K/V rows are loaded into registers while the current step
// computes, then written to the other half of a double-buffered LDS tile.
// Key steps past the causal diagonal are never visited; only steps that
// straddle it apply the per-element mask.
#include "attn_common.h"
#include "cpthd_host.h"

namespace cpthd {

constexpr float kRescaleThreshold = 8.0f;   // log2 units

template <int DP>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, const char* __restrict__ ws,
                                                          PlanLayout lay, AttnParams prm, int32_t* status) {
  constexpr int KS = Lds<DP>::kNat, VS = Lds<DP>::kTr;
  __shared__ __align__(16) uint16_t Ks[2][kKvStep * KS];
  __shared__ __align__(16) uint16_t Vs[2][kKvStep * VS];

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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int G = prm.G, D = prm.D, Hq = prm.Hq, Hkv = prm.Hkv;
  const int bm = kRowsPerWG / G;

  // the lane's query row in each of the wave's two 32-row blocks
  bool row_in[2], valid[2];
  int p_q[2];
  int64_t qrow[2];
  bf16x8 qf[2][DP / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int m = wave * kRowsPerWave + 32 * qb + l32;
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

  float m_i[2] = {-INFINITY, -INFINITY}, l_i[2] = {0.f, 0.f};
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
    vr.store(Vs[0], VS);
  }
  __syncthreads();

  const float sl2 = prm.scale_log2;
  for (int it = 0; it < nsteps; ++it) {
    const int kb = t.ds + it * kKvStep;
    const int buf = it & 1;
    if (it + 1 < nsteps) fetch(kb + kKvStep);
    const uint16_t* Kt = Ks[buf];
    const uint16_t* Vt = Vs[buf];

    f32x16 sc[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[0][b] = f32x16{};
      sc[1][b] = f32x16{};
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) {
        const bf16x8 a = lds_row8(Kt, KS, 32 * b + l32, 16 * s, h);
        sc[0][b] = mfma32(a, qf[0][s], sc[0][b]);
        sc[1][b] = mfma32(a, qf[1][s], sc[1][b]);
      }
    }

    const bool need_mask = kb + kKvStep - 1 > t.p0;
    bf16x8 pb[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[qb][b][r];
          if (need_mask) {
            const int key = kb + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > p_q[qb]) x = -INFINITY;
          }
          sc[qb][b][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, xor32(mx)) * sl2;
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

#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = lds_tr8(Vt, VS, 16 * ks + 4 * h, 16 * ks + 8 + 4 * h, 32 * db);
        acc[0][db] = mfma32(a, pb[0][ks], acc[0][db]);
        acc[1][db] = mfma32(a, pb[1][ks], acc[1][db]);
      }

    if (it + 1 < nsteps) {
      kr.store(Ks[buf ^ 1], KS);
      vr.store(Vs[buf ^ 1], VS);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = l_i[qb] + xor32(l_i[qb]);
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

template <int DP>
static int launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const char* ws,
                      const PlanLayout& lay, const AttnParams& prm, int32_t* status, unsigned grid,
                      hipStream_t stream, hipEvent_t* ev, int nev) {
  return launch(attn_fwd_kernel<DP>, dim3(grid), dim3(256), 0, stream, ev, nev, 0, (const uint16_t*)q,
                (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, ws, lay, prm, status);
}

int check_attn_args(int64_t T, int64_t capacity, int32_t cp, int32_t rank, int32_t strategy, int32_t num_docs,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t wl, int32_t wr, const void* ws,
                    size_t ws_bytes, PlanLayout& lay, AttnParams& prm) {
  if (cp < 1 || rank < 0 || rank >= cp) return CPTHD_ERR_RANK;
  if (int e = check_strategy(strategy)) return e;
  if (int e = check_tokens(T, capacity, cp, num_docs)) return e;
  if (int e = check_heads(Hq, Hkv, D)) return e;
  if (causal != 1 || wl != -1 || wr != 0) return CPTHD_ERR_MASK;
  lay = plan_layout(capacity, cp, Hq, Hkv, num_docs);
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
  return CPTHD_OK;
}

// Work-groups for the query tiles: an upper bound from the active S (the plan
// holds the exact count; surplus work-groups exit at once).
unsigned qtile_grid(const AttnParams& prm) {
  const int64_t bm = tokens_per_qtile(prm.G);
  const int64_t seg = (prm.strategy == CPTHD_DUAL_CHUNK_SWAP ? 2 : 1) * (int64_t)prm.num_docs;
  return (unsigned)(((prm.S + bm - 1) / bm + seg) * prm.Hkv);
}

}  // namespace cpthd

using namespace cpthd;

extern "C" int cpthd_attn_fwd(const void* q_local, const void* k, const void* v, int64_t total_tokens,
                              int64_t capacity_tokens, int32_t num_docs, int32_t cp_size, int32_t rank,
                              int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
                              void* o_local, float* lse_local, void* workspace, size_t workspace_bytes,
                              int32_t* dev_status, hipStream_t stream, hipEvent_t* events, int32_t n_events) {
  if (!q_local || !k || !v || !o_local || !lse_local) return CPTHD_ERR_NULL;
  PlanLayout lay;
  AttnParams prm;
  if (int e = check_attn_args(total_tokens, capacity_tokens, cp_size, rank, strategy, num_docs, num_q_heads,
                              num_kv_heads, head_dim, causal, window_left, window_right, workspace,
                              workspace_bytes, lay, prm))
    return e;
  prm.scale = softmax_scale;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  const unsigned grid = qtile_grid(prm);
  const char* ws = (const char*)workspace;
  switch (head_dim) {
    case 16:
    case 32: return launch_fwd<32>(q_local, k, v, o_local, lse_local, ws, lay, prm, dev_status, grid, stream, events, n_events);
    case 64: return launch_fwd<64>(q_local, k, v, o_local, lse_local, ws, lay, prm, dev_status, grid, stream, events, n_events);
    default: return launch_fwd<128>(q_local, k, v, o_local, lse_local, ws, lay, prm, dev_status, grid, stream, events, n_events);
  }
}
