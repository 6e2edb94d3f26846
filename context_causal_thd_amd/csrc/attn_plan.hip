// Strategy-specific attention metadata of one CP rank (gfx950).
//
// TransformerEngine PR #3221: the sequence diagram has the CP layer gather
// K/V and then build metadata specific to the strategy; "Why" gives
// DualChunkSwap two attention steps per document (chunks r and 2*cp_size-1-r)
// and NO_LOAD_BALANCE a single step over the rank's contiguous chunk; the
// commit messages reduce the packed strategy's metadata to one chunk and one
// step per rank.
//
// Here the two steps become *segments*: maximal runs of the rank's local rows
// that are consecutive physical tokens of one document.  A query tile is up to
// 256/G tokens of one segment (times the G q heads of a kv head); its causal key
// range is [document start, last actual token of the tile].  A key tile is up
// to 128 keys of one document's slot; the rank's rows that see it are the
// suffixes (physical token >= first key) of the document's segments.  Both
// lists are sorted by work, longest first, so the hardware dispatcher's
// in-order work-group launch acts as a longest-processing-time queue.
//
// One work-group of 1024 threads builds the whole plan: it validates the cu
// arrays, scans per-document tile counts in chunks of 1024 documents, emits
// the tiles in parallel, and counting-sorts them by cost.  The plan keeps a
// copy of the cu arrays it was built from and the call's arguments in its
// header.  Every attention call first runs this kernel in "ensure" mode: when
// the workspace already holds a plan built from exactly the call's arguments
// and cu arrays it returns at once, otherwise it rebuilds the plan, so an
// attention kernel never reads tiles of another micro-batch.
#include "attn_common.h"
#include "cpthd_host.h"

namespace cpthd {

constexpr int kPlanThreads = 1024;

__device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Exclusive prefix sum over the work-group; also returns the total.
__device__ inline int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[w] = x;
  __syncthreads();
  if (threadIdx.x < 64) {
    int wv = threadIdx.x < kPlanThreads / 64 ? s_wave[threadIdx.x] : 0;
    int z = wv;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int y = __shfl_up(z, o, 64);
      if (lane >= o) z += y;
    }
    if (threadIdx.x < kPlanThreads / 64) s_wave[16 + threadIdx.x] = z - wv;
    if (threadIdx.x == kPlanThreads / 64 - 1) s_wave[32] = z;
  }
  __syncthreads();
  const int res = x - v + s_wave[16 + w];
  total = s_wave[32];
  __syncthreads();
  return res;
}

__device__ inline DocSeg doc_segments(const int32_t* cu_a, const int32_t* cu_p, int i, int S, int cp, int rank,
                                      int strategy) {
  DocSeg d;
  const int ds = cu_p[i], L = cu_p[i + 1] - ds;
  d.ds = ds;
  d.ve = ds + (cu_a[i + 1] - cu_a[i]);
  if (strategy == kDCS) {
    const int c = L / (2 * cp);
    d.la = ds / cp;
    d.pa = ds + rank * c;
    d.na = c;
    d.lb = d.la + c;
    d.pb = ds + (2 * cp - 1 - rank) * c;
    d.nb = c;
  } else if (strategy == kPacked) {
    // the document's pieces inside whole-buffer chunks r and 2cp-1-r (c = T / 2cp = S / 2)
    const int c = S / 2;
    const int a0 = rank * c, b0 = (2 * cp - 1 - rank) * c;
    const int alo = max(ds, a0), ahi = min(ds + L, a0 + c);
    const int blo = max(ds, b0), bhi = min(ds + L, b0 + c);
    d.na = max(0, ahi - alo);
    d.pa = alo;
    d.la = alo - a0;
    d.nb = max(0, bhi - blo);
    d.pb = blo;
    d.lb = c + (blo - b0);
  } else {
    const int lo = max(ds, rank * S), hi = min(ds + L, rank * S + S);
    d.na = max(0, hi - lo);
    d.pa = lo;
    d.la = lo - rank * S;
    d.lb = d.la + d.na;
    d.pb = lo;
    d.nb = 0;
  }
  return d;
}

// Query chunks (kQChunk / G tokens each, the key-tile kernel's steps) the
// rank iterates for keys from k0 on.
__device__ inline int kv_tile_cost(const DocSeg& d, int k0, int G) {
  const int tpc = kQChunk / G;
  int cost = 0;
  int lo = max(d.pa, k0), hi = min(d.pa + d.na, d.ve);
  if (hi > lo) cost += cdiv(hi - lo, tpc);
  lo = max(d.pb, k0);
  hi = min(d.pb + d.nb, d.ve);
  if (hi > lo) cost += cdiv(hi - lo, tpc);
  return cost;
}

__device__ inline void set_range(QTile& e, int a, int b) {
  e.s0 = a;
  e.s1 = b;
}
__device__ inline void set_range(KVTile& e, int a, int b) {
  e.c0 = a;
  e.c1 = b;
}

// The merge-list entry of a split tile.
__device__ inline SplitTile split_entry(const QTile& e, int slot, int np) {
  return SplitTile{slot, np, e.lrow0, e.ntok, e.p0, e.ve, {0, 0}};
}
__device__ inline SplitTile split_entry(const KVTile& e, int slot, int np) {
  return SplitTile{slot, np, e.k0, e.nkeys, e.doc, 0, {0, 0}};
}

// Parts a tile of this cost becomes: tiles above the threshold `thr` are cut
// into parts of at most `P` steps; a tile that would stay one part is whole.
__device__ inline int parts_of(int cost, int thr, int P) {
  const int n = (P > 0 && cost > thr) ? (cost - 1) / P + 1 : 1;
  return n >= 2 ? n : 1;
}

constexpr int kSplitTries = 16;     // part sizes P0 * 2^j tried by the split rule
constexpr int kMinPartSteps = 16;   // no part has fewer steps (its partial results cost about as much as 16 steps' loads)
constexpr int kMaxCandidates = 256;
constexpr int kLdsCosts = 2048;     // tiles per list whose costs the plan also keeps in LDS

// Shared state of the split rule of one tile list.
struct SplitScratch {
  unsigned long long sum;
  int max_cost, n_cand, thr, P;
  int parts[kSplitTries];
  int cand[kMaxCandidates];       // tiles above the threshold (list index) ...
  int cand_cost[kMaxCandidates];  // ... their costs
  int cand_slot[kMaxCandidates];  // ... their first partial slots (-1: whole)
  int cand_split[kMaxCandidates]; // ... and merge-list entries
  int cost[kLdsCosts];            // costs of the list's first tiles (a candidate's: -1 - its index once split)
};

// The split rule of one tile list (n whole tiles, each run for Hkv heads, of
// total cost W and largest cost max_cost; C compute units): a tile whose cost
// exceeds the share W * Hkv / C of one unit is cut into parts of P steps, the
// smallest of P0 * 2^j (P0 = max(ceil(share / 2), 16)) whose parts fit the
// `max_parts` partial slots, and longest-first dispatch balances the rest.
// At most C / Hkv tiles exceed the share (their costs add up to less than W);
// they are listed in sc with the first partial slot and the merge-list entry
// of each split one; the cost histogram trades a split tile for its parts.
// Sets sc.thr and sc.P (P = 0: nothing split); returns the number of split
// tiles.
template <typename Tile>
__device__ int split_tiles(const Tile* tmp, int n, int Hkv, int num_cu, int max_parts, int* s_hist, int* s_wave,
                           SplitScratch& sc) {
  const int tid = threadIdx.x;
  const unsigned long long share =
      (sc.sum * (unsigned long long)Hkv + num_cu - 1) / (unsigned long long)max(num_cu, 1);
  const int thr = (int)min(share, (unsigned long long)INT32_MAX), max_cost = sc.max_cost;
  __syncthreads();   // (sc.sum and sc.max_cost read by every thread)
  if (tid == 0) {
    sc.thr = thr;
    sc.P = 0;
    sc.n_cand = 0;
  }
  if (max_cost <= thr || max_parts < 2) return 0;   // (uniform)
  const int P0 = max(thr / 2 + (thr & 1), kMinPartSteps);
  if (tid < kSplitTries) sc.parts[tid] = 0;
  __syncthreads();
  for (int t = tid; t < n; t += kPlanThreads) {
    const int c = t < kLdsCosts ? sc.cost[t] : tmp[t].cost;
    if (c <= thr) continue;
    const int k = atomicAdd(&sc.n_cand, 1);
    if (k < kMaxCandidates) {
      sc.cand[k] = t;
      sc.cand_cost[k] = c;
    }
    // parts at P0 * 2^j: ceil(c / (P0 2^j)) = ceil(ceil(c / P0) / 2^j)
    const int q0 = (c - 1) / P0 + 1;
#pragma unroll
    for (int j = 0; j < kSplitTries; ++j) {
      const int np = (q0 - 1) / (1 << j) + 1;
      if (np >= 2) atomicAdd(&sc.parts[j], min(np, max_parts + 1));
    }
  }
  __syncthreads();
  const int n_cand = sc.n_cand;
  int P = 0;
  if (n_cand <= kMaxCandidates) {   // (else more compute units than the list tracks: nothing split)
    for (int j = 0; j < kSplitTries && ((int64_t)P0 << j) < max_cost; ++j) {
      if (sc.parts[j] <= max_parts) {
        P = P0 << j;   // (< max_cost, so in range)
        break;
      }
    }
  }
  if (P == 0) {
    __syncthreads();
    if (tid == 0) sc.n_cand = 0;
    __syncthreads();
    return 0;
  }
  // the candidates' slots and merge-list entries from one scan of (np | 1 << 16)
  int np = 1, c = 0;
  if (tid < n_cand) {
    c = sc.cand_cost[tid];
    np = parts_of(c, thr, P);
  }
  int total;
  const int ex = block_exclusive_scan(np >= 2 ? (np | (1 << 16)) : 0, s_wave, total);
  if (tid < n_cand) {
    sc.cand_slot[tid] = np >= 2 ? (ex & 0xFFFF) : -1;
    sc.cand_split[tid] = ex >> 16;
    if (sc.cand[tid] < kLdsCosts) sc.cost[sc.cand[tid]] = -1 - tid;
    if (np >= 2) {
      const int base = c / np, rem = c - base * np;
      atomicSub(&s_hist[min(c, kCostBins - 1)], 1);
      if (rem) atomicAdd(&s_hist[min(base + 1, kCostBins - 1)], rem);
      atomicAdd(&s_hist[min(base, kCostBins - 1)], np - rem);
    }
  }
  if (tid == 0) sc.P = P;
  __syncthreads();
  return total >> 16;
}

// Bin offsets of a counting sort by cost, longest first: bin b starts after
// the entries of the bins above it.  Returns the entry count.
__device__ inline int bin_offsets(int* s_hist, int* s_wave) {
  const int hi = kCostBins - 1 - 2 * threadIdx.x;
  const int v0 = s_hist[hi], v1 = s_hist[hi - 1];
  int entries;
  const int excl = block_exclusive_scan(v0 + v1, s_wave, entries);
  s_hist[hi] = excl;
  s_hist[hi - 1] = excl + v0;
  return entries;
}

// Place tile t of a list: the whole tile, or its parts (and its merge-list
// entry) when it is split.
template <typename Tile>
__device__ inline void place_tile(Tile e, int t, Tile* out, SplitTile* splits, int* s_hist, const SplitScratch& sc) {
  const int c = e.cost;
  int slot = -1, si = 0;
  if (sc.P > 0 && c > sc.thr) {
    int k = -1;
    if (t < kLdsCosts) {
      const int v = sc.cost[t];
      k = v < 0 ? -1 - v : -1;
    } else {
      for (int j = 0; j < sc.n_cand; ++j)
        if (sc.cand[j] == t) k = j;
    }
    if (k >= 0) {
      slot = sc.cand_slot[k];
      si = sc.cand_split[k];
    }
  }
  if (slot >= 0) {
    const int np = parts_of(c, sc.thr, sc.P), base = c / np, rem = c - base * np;
    splits[si] = split_entry(e, slot, np);
    e.slot = slot;
    e.nparts = np;
    for (int p = 0; p < np; ++p) {
      const int a = p * base + min(p, rem), len = base + (p < rem ? 1 : 0);
      set_range(e, a, a + len);
      e.cost = len;
      e.part = p;
      out[atomicAdd(&s_hist[min(len, kCostBins - 1)], 1)] = e;
    }
  } else {
    set_range(e, 0, c);
    out[atomicAdd(&s_hist[min(c, kCostBins - 1)], 1)] = e;
  }
}

// The header and stored cu arrays of a plan built from exactly these arguments?
__device__ inline bool plan_current(const char* ws, const PlanLayout& lay, const int32_t* cu_a, const int32_t* cu_p,
                                    int B, int T, int cp, int rank, int strategy, int Hq, int Hkv, int D, int num_cu,
                                    int* s_flag) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    const PlanHeader h = *reinterpret_cast<const PlanHeader*>(ws);
    *s_flag = (h.valid == 1) & (h.magic == kPlanMagic) & (h.version == kPlanVersion) & (h.T == T) &
              (h.S == T / cp) & (h.cp == cp) & (h.rank == rank) & (h.strategy == strategy) & (h.Hq == Hq) &
              (h.Hkv == Hkv) & (h.D == D) & (h.num_docs == B) & (h.num_cu == num_cu) &
              (h.max_qtiles == (int)lay.max_qtiles) & (h.max_kvtiles == (int)lay.max_kvtiles) &
              (h.max_docs == (int)lay.max_docs) & (h.max_parts == (int)lay.max_parts);
  }
  __syncthreads();
  if (!*s_flag) return false;   // uniform: every thread read the same flag
  const int32_t* cpy = reinterpret_cast<const int32_t*>(ws + lay.cu_copy);
  int diff = 0;
  for (int i = tid; i <= B; i += kPlanThreads) diff |= (cpy[i] != cu_p[i]) | (cpy[B + 1 + i] != cu_a[i]);
  return !__syncthreads_or(diff);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ cu_a,
                                                            const int32_t* __restrict__ cu_p, int B, int T, int cp,
                                                            int rank, int strategy, int Hq, int Hkv, int D,
                                                            int num_cu, int qsplit, char* __restrict__ ws,
                                                            PlanLayout lay, int32_t* status, int ensure) {
  __shared__ int s_bits;
  __shared__ int s_flag;
  __shared__ int s_wave[40];
  __shared__ int s_qoff[kPlanThreads], s_kvoff[kPlanThreads];
  __shared__ int s_hist_q[kCostBins], s_hist_kv[kCostBins];   // entries per cost bin
  __shared__ SplitScratch s_split[2];                           // query and key lists
  __shared__ DocSeg s_docs[kPlanThreads];                       // this chunk's documents
  __shared__ int s_len[kPlanThreads];                           // and their padded lengths

  PlanHeader* hdr = reinterpret_cast<PlanHeader*>(ws);
  QTile* qt = reinterpret_cast<QTile*>(ws + lay.qtiles);
  QTile* qtmp = reinterpret_cast<QTile*>(ws + lay.qtiles_tmp);
  KVTile* kvt = reinterpret_cast<KVTile*>(ws + lay.kvtiles);
  KVTile* kvtmp = reinterpret_cast<KVTile*>(ws + lay.kvtiles_tmp);
  DocSeg* docs = reinterpret_cast<DocSeg*>(ws + lay.docs);

  const int tid = threadIdx.x;
  const int S = T / cp, G = Hq / Hkv, bm = tokens_per_qtile(G);
  // ensure mode: nothing to do when the workspace holds this call's plan
  if (ensure && plan_current(ws, lay, cu_a, cu_p, B, T, cp, rank, strategy, Hq, Hkv, D, num_cu, &s_flag)) return;
  if (tid == 0) {
    s_bits = 0;
    hdr->valid = 0;
  }
  __syncthreads();

  // 1. validate the metadata
  int bits = 0;
  for (int i = tid; i < B; i += kPlanThreads) {
    const int p0 = cu_p[i], p1 = cu_p[i + 1], a0 = cu_a[i], a1 = cu_a[i + 1];
    if (p1 < p0) bits |= kDevCuOrder;
    if (a1 < a0 || a1 - a0 > p1 - p0) bits |= kDevActual;
    if (strategy == kDCS && ((p1 - p0) % (2 * cp)) != 0) bits |= kDevDcsDivisible;
    if ((int64_t)(p1 - p0) * Hkv * D * 2 >= ((int64_t)1 << 31)) bits |= kDevDocBytes;
  }
  if (tid == 0) {
    if (cu_p[0] != 0) bits |= kDevCuOrder;
    if (cu_a[0] != 0) bits |= kDevActual;
    if (cu_p[B] != T) bits |= kDevCuTotal;
  }
  if (bits) atomicOr(&s_bits, bits);
  __syncthreads();
  if (s_bits) {
    if (tid == 0) {
      if (status) atomicOr(status, s_bits);
      hdr->n_qtiles = 0;
      hdr->n_kvtiles = 0;
      hdr->n_qsplit = 0;
      hdr->n_kvsplit = 0;
      hdr->n_kvwhole = 0;
    }
    return;
  }

  // 2. documents in chunks of 1024: segments, tile counts, scan, emission of
  //    the whole tiles, their cost histograms, totals and maxima
  for (int b = tid; b < kCostBins; b += kPlanThreads) s_hist_q[b] = s_hist_kv[b] = 0;   // (the scans' barriers
                                                                                          //  order this first)
  if (tid < 2) {
    s_split[tid].sum = 0ull;
    s_split[tid].max_cost = 0;
  }
  unsigned long long sum_q = 0, sum_kv = 0;
  int max_q = 0, max_kv = 0;
  int carry_q = 0, carry_kv = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int i = base + tid;
    const int cnt = min(kPlanThreads, B - base);
    int nq = 0, nkv = 0;
    if (i < B) {
      const DocSeg d = doc_segments(cu_a, cu_p, i, S, cp, rank, strategy);
      docs[i] = d;
      s_docs[tid] = d;
      s_len[tid] = cu_p[i + 1] - d.ds;
      nq = cdiv(d.na, bm) + cdiv(d.nb, bm);
      nkv = cdiv(s_len[tid], kKeysPerWG);
    }
    int tq, tkv;
    const int oq = block_exclusive_scan(nq, s_wave, tq);
    const int okv = block_exclusive_scan(nkv, s_wave, tkv);
    s_qoff[tid] = oq;
    s_kvoff[tid] = okv;
    __threadfence_block();
    __syncthreads();
    for (int t = tid; t < tq; t += kPlanThreads) {
      int lo = 0, hi = cnt - 1;   // last document whose first tile is <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_qoff[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const DocSeg d = s_docs[lo];
      int k = t - s_qoff[lo];
      const int nA = cdiv(d.na, bm);
      QTile e;
      if (k < nA) {
        e.lrow0 = d.la + k * bm;
        e.p0 = d.pa + k * bm;
        e.ntok = min(bm, d.na - k * bm);
      } else {
        k -= nA;
        e.lrow0 = d.lb + k * bm;
        e.p0 = d.pb + k * bm;
        e.ntok = min(bm, d.nb - k * bm);
      }
      e.ds = d.ds;
      e.ve = d.ve;
      e.kv_end = e.p0 < d.ve ? min(e.p0 + e.ntok, d.ve) : d.ds;
      e.cost = cdiv(e.kv_end - d.ds, kKvStep);
      e.doc = base + lo;
      e.slot = -1;
      e.part = 0;
      e.nparts = 1;
      e.vt = (carry_kv + s_kvoff[lo]) * kKeysPerWG;   // the document's first key tile, in V^T columns
      qtmp[carry_q + t] = e;
      if (carry_q + t < kLdsCosts) s_split[0].cost[carry_q + t] = e.cost;
      atomicAdd(&s_hist_q[min(e.cost, kCostBins - 1)], 1);
      sum_q += (unsigned long long)e.cost;
      max_q = max(max_q, e.cost);
    }
    for (int t = tid; t < tkv; t += kPlanThreads) {
      int lo = 0, hi = cnt - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_kvoff[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const DocSeg d = s_docs[lo];
      const int k = t - s_kvoff[lo];
      const int L = s_len[lo];
      KVTile e;
      e.k0 = d.ds + k * kKeysPerWG;
      e.nkeys = min(kKeysPerWG, L - k * kKeysPerWG);
      e.doc = base + lo;
      e.cost = kv_tile_cost(d, e.k0, G);
      e.slot = -1;
      e.part = 0;
      e.nparts = 1;
      kvtmp[carry_kv + t] = e;
      if (carry_kv + t < kLdsCosts) s_split[1].cost[carry_kv + t] = e.cost;
      atomicAdd(&s_hist_kv[min(e.cost, kCostBins - 1)], 1);
      sum_kv += (unsigned long long)e.cost;
      max_kv = max(max_kv, e.cost);
    }
    carry_q += tq;
    carry_kv += tkv;
    __threadfence_block();
    __syncthreads();
  }

  // 3. split the tiles that exceed a compute unit's share; longest first
  // (one shared atomic per wave: 1024 on one address would serialise)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sum_q += __shfl_xor(sum_q, o, 64);
    sum_kv += __shfl_xor(sum_kv, o, 64);
    max_q = max(max_q, __shfl_xor(max_q, o, 64));
    max_kv = max(max_kv, __shfl_xor(max_kv, o, 64));
  }
  if ((tid & 63) == 0) {
    atomicAdd(&s_split[0].sum, sum_q);
    atomicMax(&s_split[0].max_cost, max_q);
    atomicAdd(&s_split[1].sum, sum_kv);
    atomicMax(&s_split[1].max_cost, max_kv);
  }
  __threadfence_block();
  __syncthreads();
  const int n_qsplit = split_tiles(qtmp, carry_q, Hkv, num_cu, qsplit ? (int)lay.max_parts : 0, s_hist_q, s_wave,
                                   s_split[0]);
  const int n_kvsplit = split_tiles(kvtmp, carry_kv, Hkv, num_cu, (int)lay.max_parts, s_hist_kv, s_wave, s_split[1]);
  const int n_q = bin_offsets(s_hist_q, s_wave);
  const int n_kv = bin_offsets(s_hist_kv, s_wave);
  __syncthreads();
  for (int t = tid; t < max(carry_q, carry_kv); t += kPlanThreads) {
    QTile eq;
    KVTile ek;
    if (t < carry_q) eq = qtmp[t];
    if (t < carry_kv) ek = kvtmp[t];
    if (t < carry_q) place_tile(eq, t, qt, reinterpret_cast<SplitTile*>(ws + lay.qsplit), s_hist_q, s_split[0]);
    if (t < carry_kv) place_tile(ek, t, kvt, reinterpret_cast<SplitTile*>(ws + lay.kvsplit), s_hist_kv, s_split[1]);
  }

  // 4. the cu arrays the plan was built from, then the header
  int32_t* cpy = reinterpret_cast<int32_t*>(ws + lay.cu_copy);
  for (int i = tid; i <= B; i += kPlanThreads) {
    cpy[i] = cu_p[i];
    cpy[B + 1 + i] = cu_a[i];
  }
  // (no device-scope fences: the plan's readers are later kernels on the stream)
  if (tid == 0) {
    hdr->magic = kPlanMagic;
    hdr->version = kPlanVersion;
    hdr->T = T;
    hdr->S = S;
    hdr->cp = cp;
    hdr->rank = rank;
    hdr->strategy = strategy;
    hdr->Hq = Hq;
    hdr->Hkv = Hkv;
    hdr->D = D;
    hdr->G = G;
    hdr->num_docs = B;
    hdr->bm_tok = bm;
    hdr->n_qtiles = n_q;
    hdr->n_kvtiles = n_kv;
    hdr->max_qtiles = (int)lay.max_qtiles;
    hdr->max_kvtiles = (int)lay.max_kvtiles;
    hdr->max_docs = (int)lay.max_docs;
    hdr->max_parts = (int)lay.max_parts;
    hdr->num_cu = num_cu;
    hdr->q_part_steps = n_qsplit ? s_split[0].P : 0;
    hdr->kv_part_chunks = n_kvsplit ? s_split[1].P : 0;
    hdr->n_qsplit = n_qsplit;
    hdr->n_kvsplit = n_kvsplit;
    hdr->n_kvwhole = carry_kv;
    hdr->valid = 1;
  }
}

}  // namespace cpthd

using namespace cpthd;

extern "C" size_t cpthd_attn_workspace_bytes(int64_t capacity_tokens, int32_t cp_size, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t max_docs) {
  if (cp_size < 1 || max_docs < 1) return 0;
  if (check_tokens(capacity_tokens, capacity_tokens, cp_size, max_docs)) return 0;
  if (check_heads(num_q_heads, num_kv_heads, head_dim)) return 0;
  // with the V^T rows of the forward where it reads them
  const PlanLayout v = plan_layout(capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs,
                                   default_split_parts(num_kv_heads, capacity_tokens), true);
  if (vt_wanted(head_dim, v.vt_cols)) return v.total;
  return plan_layout(capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs,
                     default_split_parts(num_kv_heads, capacity_tokens), false)
      .total;
}

extern "C" size_t cpthd_attn_workspace_min_bytes(int64_t capacity_tokens, int32_t cp_size, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_docs) {
  if (cp_size < 1 || max_docs < 1) return 0;
  if (check_tokens(capacity_tokens, capacity_tokens, cp_size, max_docs)) return 0;
  if (check_heads(num_q_heads, num_kv_heads, head_dim)) return 0;
  return plan_layout(capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs, 0, false).total;
}

namespace cpthd {

int launch_plan(const int32_t* cu_a, const int32_t* cu_p, const AttnParams& prm, char* ws, const PlanLayout& lay,
                bool ensure, int32_t* status, hipStream_t stream, hipEvent_t* ev, int nev, int slot) {
  return launch(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, ev, nev, slot, cu_a, cu_p, prm.num_docs, prm.T,
                prm.cp, prm.rank, prm.strategy, prm.Hq, prm.Hkv, prm.D, prm.num_cu, prm.qsplit, ws, lay, status,
                ensure ? 1 : 0);
}

}  // namespace cpthd

extern "C" int cpthd_attn_plan(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t num_docs,
                               int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t rank,
                               int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
  if (!cu_seqlens || !cu_seqlens_padded) return CPTHD_ERR_NULL;
  PlanLayout lay;
  AttnParams prm;
  // the mask arguments are those every attention call must pass
  if (int e = check_attn_args(total_tokens, capacity_tokens, cp_size, rank, strategy, num_docs, num_q_heads,
                              num_kv_heads, head_dim, 1, -1, 0, workspace, workspace_bytes, lay, prm))
    return e;
  if (int e = device_cus(prm)) return e;
  return launch_plan(cu_seqlens, cu_seqlens_padded, prm, (char*)workspace, lay, false, dev_status, stream, nullptr,
                     0, 0);
}
