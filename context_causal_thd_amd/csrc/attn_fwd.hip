// Causal THD attention forward for one CP rank's query rows (gfx950).
//
// TransformerEngine PR #3221, "Scope and constraints": THD self-attention,
// causal without a sliding window (window_size = (-1, 0)); documents stay
// isolated through the sequence metadata ("Logical sequences remain isolated
// by cu_seqlens", review thread).  A local row at physical token p of
// document d attends to the actual keys of d at positions <= p's position.
//
// One work-group = one query tile of the plan (<= 128/G tokens of one segment
// times the G q heads of one kv head, 128 rows) against its key range
// [document start, last actual token of the tile], 64 keys per step:
//   S^T = K Q^T (bf16 MFMA 32x32x16, K from LDS, Q in registers),
//   online softmax in fp32 / exp2 with the query as the lane index,
//   O^T += V^T P^T (V staged transposed in LDS, P^T straight from registers).
// Key tiles past the causal diagonal are never visited; only steps that
// straddle the diagonal apply the per-element mask.
#include "attn_common.h"
#include "cpthd_host.h"

namespace cpthd {

template <int DP>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, const char* __restrict__ ws,
                                                          PlanLayout lay, AttnParams prm, int32_t* status) {
  __shared__ __align__(16) uint16_t Ks[kKvStep * (DP + 8)];
  __shared__ __align__(16) uint16_t Vt[DP * (kKvStep + 8)];

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
  const int m = wave * 32 + l32;          // row of the tile: token m / G, head m % G
  const int tt = m / G, g = m - tt * G;
  const bool row_in = m < bm * G && tt < t.ntok;
  const int p_q = t.p0 + tt;
  const bool valid = row_in && p_q < t.ve;
  const int64_t qrow = (int64_t)(t.lrow0 + tt) * Hq + kvh * G + g;

  bf16x8 qf[DP / 16];
#pragma unroll
  for (int s = 0; s < DP / 16; ++s) {
    u32x4 val = {0u, 0u, 0u, 0u};
    const int d = 16 * s + 8 * h;
    if (row_in && d < D) val = *reinterpret_cast<const u32x4*>(q + qrow * D + d);
    qf[s] = as_bf16x8(val);
  }

  float m_i = -INFINITY, l_i = 0.f;
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
    stage_rows<DP, kKvStep, true, false>(k, D, key_row, Ks, nullptr);
    stage_rows<DP, kKvStep, false, true>(v, D, key_row, nullptr, Vt);
    __syncthreads();

    f32x16 sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[b] = f32x16{};
#pragma unroll
      for (int s = 0; s < DP / 16; ++s) sc[b] = mfma32(lds_a_nat<DP>(Ks, 32 * b + l32, s, h), qf[s], sc[b]);
    }
    const bool need_mask = kb + kKvStep - 1 > t.p0;
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[b][r] * sl2;
        if (need_mask) {
          const int key = kb + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > p_q) x = -INFINITY;
        }
        sc[b][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_i, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_i - m_use);
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(sc[b][r] - m_use);
        sc[b][r] = pv;
        rs += pv;
      }
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) acc[db] *= alpha;

    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pb[ks] = acc_to_bf16(sc[ks >> 1], 8 * (ks & 1));
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[db] = mfma32(lds_a_trn<kKvStep>(Vt, 32 * db + l32, ks, h), pb[ks], acc[db]);
  }

  const float l_tot = l_i + xor32(l_i);
  if (!row_in) return;
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
  if (h == 0) lse[qrow] = valid ? (m_i + log2_fast(l_tot)) * 0.69314718055994531f : -INFINITY;
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
