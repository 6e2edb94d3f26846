// Partition indices and K/V restoration for one CP rank (gfx950).
//
// TransformerEngine PR #3221, "Why": DualChunkSwap cuts every document into
// 2*cp_size equal chunks and rank r owns the mirrored pair (r, 2*cp_size-1-r);
// NO_LOAD_BALANCE cuts the physical buffer into cp_size contiguous chunks.
// Commit messages: rank-major (contiguous) ownership needs no K/V reorder;
// review thread: the THD stream dependency follows K/V restoration.
//
// Both kernels are pure data movement (HBM bound).  Under DualChunkSwap the
// rank's local rows of document i start at local row cu_padded[i] / cp_size
// (every earlier document contributed L/cp_size rows), so an output position
// finds its document by a search over cu_seqlens_padded, without a prefix sum.
#include <algorithm>

#include "cpthd_device.h"
#include "cpthd_host.h"

namespace cpthd {

// Checks on cu_seqlens_padded shared by partition and reorder.
__device__ inline void validate_cu_padded(const int32_t* cu, int B, int64_t T, int cp, int strategy,
                                          int32_t* status) {
  if (status == nullptr) return;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int nthreads = gridDim.x * blockDim.x;
  int bits = 0;
  for (int i = gid; i < B; i += nthreads) {
    const int a = cu[i], b = cu[i + 1];
    if (b < a) bits |= kDevCuOrder;
    if (strategy == kDCS && ((b - a) % (2 * cp)) != 0) bits |= kDevDcsDivisible;
  }
  if (gid == 0) {
    if (cu[0] != 0) bits |= kDevCuOrder;
    if ((int64_t)cu[B] != T) bits |= kDevCuTotal;
  }
  if (bits) atomicOr(status, bits);
}

// Document of the wave's first output under DualChunkSwap: the largest i in
// [0, B-1] with cu[i] <= x0, found by all 64 lanes together.  Each round the
// lanes probe 64 evenly spaced offsets and one ballot keeps the piece holding
// x0, so 10,000 documents take 3 dependent loads instead of 14.
__device__ inline int wave_upper_index(const int32_t* cu, int B, int64_t x0, int lane) {
  int lo = 0, hi = B - 1;   // cu[lo] <= x0 for a valid layout
  while (hi - lo >= 64) {
    const int64_t span = hi - lo;
    const int m = lo + (int)((span * (lane + 1)) >> 6);   // lane 63 probes hi
    const int k = __popcll(__ballot((int64_t)cu[m] <= x0));   // probes are non-decreasing: lanes 0..k-1 hold
    const int m_next = lo + (int)((span * (k + 1)) >> 6);     // first probe above x0 (when k < 64)
    if (k > 0) lo = lo + (int)((span * k) >> 6);
    if (k < 64) hi = m_next - 1;
  }
  const int cand = lo + lane;
  const int k = __popcll(__ballot(cand <= hi && (int64_t)cu[cand] <= x0));
  return max(lo + k - 1, 0);   // k >= 1 unless the layout is rejected
}

// One thread writes 4 consecutive outputs j = 4*gid .. 4*gid+3 of [0, S).
__global__ __launch_bounds__(256) void partition_kernel(const int32_t* __restrict__ cu, int B, int T, int cp,
                                                        int rank, int strategy, int32_t* __restrict__ out,
                                                        int32_t* status) {
  validate_cu_padded(cu, B, T, cp, strategy, status);
  const int S = T / cp;
  const int64_t j0 = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  int32_t res[4];
  if (strategy == kContig) {
    if (j0 >= S) return;
    for (int u = 0; u < 4; ++u) res[u] = rank * S + (int)j0 + u;
  } else if (strategy == kPacked) {
    if (j0 >= S) return;
    const int c = T / (2 * cp);   // whole-buffer chunks r and 2cp-1-r
    for (int u = 0; u < 4; ++u) {
      const int j = (int)j0 + u;
      res[u] = j < c ? rank * c + j : (2 * cp - 1 - rank) * c + (j - c);
    }
  } else {
    // document of output j: cu[i] <= j*cp < cu[i+1].  The wave's 256 outputs
    // span a short run of documents: find the first with a wave search, hold
    // the next 64 offsets one per lane, and look each output up among them
    // with register shuffles.  Every lane of a live wave takes part.
    const int lane = threadIdx.x & 63;
    const int64_t jw = j0 - 4 * lane;   // the wave's first output
    if (jw >= S) return;                // the whole wave is past the end
    const int64_t x_last = (min(jw + 255, (int64_t)S - 1)) * cp;
    const int i0 = wave_upper_index(cu, B, jw * cp, lane);
    const int w = cu[min(i0 + lane, B)];   // offsets of documents i0 .. i0+63 (cu[B] = T past the end)
    // the run is held whole when the document after the wave's last output starts inside it
    const bool held = (int64_t)__shfl(w, 63) > x_last;
    for (int u = 0; u < 4; ++u) {
      const int64_t j = min(j0 + u, (int64_t)S - 1);
      const int64_t x = j * cp;
      int start, next;
      if (held) {
        int k = 0;   // largest k with w_k <= x, one bit at a time (w_0 <= x; k <= 62 when held)
#pragma unroll
        for (int b = 32; b >= 1; b >>= 1) {
          const int t = k + b;
          if ((int64_t)__shfl(w, t) <= x) k = t;
        }
        k = min(k, 62);
        start = __shfl(w, k);
        next = __shfl(w, k + 1);
      } else {
        const int i = i0 + upper_index(cu + i0, B - 1 - i0, x);
        start = cu[i];
        next = cu[i + 1];
      }
      const int c = (next - start) / (2 * cp);
      const int jj = (int)(j - start / cp);
      const int p = jj < c ? start + rank * c + jj : start + (2 * cp - 1 - rank) * c + (jj - c);
      res[u] = min(max(p, 0), T - 1);   // stays in range even for a rejected layout
    }
    if (j0 >= S) return;
  }
  if (j0 + 3 < S && (S & 3) == 0) {
    *reinterpret_cast<int4*>(out + j0) = make_int4(res[0], res[1], res[2], res[3]);
  } else {
    for (int u = 0; u < 4 && j0 + u < S; ++u) out[j0 + u] = res[u];
  }
}

// Restoration: each wave copies kReorderRowsPerWave whole token rows.  Row p of
// the output (physical order) comes from gathered row s*S + (local index of p on
// its owner s).  A lane issues the loads of kReorderChunks 16-byte pieces of
// every row before any store, so a wave keeps rows x chunks x 1 KiB in flight.
#ifndef CPTHD_REORDER_ROWS
#define CPTHD_REORDER_ROWS 2
#endif
#ifndef CPTHD_REORDER_CHUNKS
#define CPTHD_REORDER_CHUNKS 2
#endif
constexpr int kReorderRowsPerWave = CPTHD_REORDER_ROWS;
#ifndef CPTHD_REORDER_LOAD
#define CPTHD_REORDER_LOAD __builtin_nontemporal_load   // streamed once: no cache retention
#endif
#ifndef CPTHD_REORDER_STORE
#define CPTHD_REORDER_STORE __builtin_nontemporal_store
#endif
constexpr int kReorderChunks = CPTHD_REORDER_CHUNKS;

// Gathered row of physical row p; under DualChunkSwap `doc` is the document
// holding p (unused otherwise).
__device__ inline int64_t gathered_row_of(const int32_t* cu, int doc, int S, int cp, int strategy, int p) {
  if (strategy == kContig) return p;
  int start = 0, L = cp * S;                      // whole buffer as one sequence (packed strategy)
  if (strategy == kDCS) {
    start = cu[doc];
    L = cu[doc + 1] - start;
  }
  const int c = L / (2 * cp);
  if (c <= 0) return p;                           // only for a rejected layout
  const int pos = p - start;
  const int chunk = min(pos / c, 2 * cp - 1);
  const int off = pos - chunk * c;
  const int owner = chunk < cp ? chunk : 2 * cp - 1 - chunk;
  const int local = start / cp + (chunk < cp ? off : c + off);
  return (int64_t)owner * S + local;
}

__global__ __launch_bounds__(256) void reorder_kernel(const char* __restrict__ kg, const char* __restrict__ vg,
                                                      char* __restrict__ ko, char* __restrict__ vo,
                                                      int64_t row_bytes, const int32_t* __restrict__ cu, int B,
                                                      int T, int cp, int strategy, int32_t* status) {
  constexpr int R = kReorderRowsPerWave, U = kReorderChunks;
  if (blockIdx.y == 0) validate_cu_padded(cu, B, T, cp, strategy, status);
  const char* src = blockIdx.y == 0 ? kg : vg;
  char* dst = blockIdx.y == 0 ? ko : vo;
  const int S = T / cp;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * R;
  const int nrows = (int)min((int64_t)R, (int64_t)T - row0);
  if (nrows <= 0) return;
  // the document of the wave's first row, found by all lanes together; the
  // wave's other rows are at most R - 1 rows further on
  int doc = strategy == kDCS ? wave_upper_index(cu, B, row0, lane) : 0;
  int64_t g[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int64_t p = min(row0 + rr, (int64_t)T - 1);
    if (strategy == kDCS)
      while (doc < B - 1 && (int64_t)cu[doc + 1] <= p) ++doc;
    const int64_t gr = gathered_row_of(cu, doc, S, cp, strategy, (int)p);
    g[rr] = __builtin_amdgcn_readfirstlane((int)min(max(gr, (int64_t)0), (int64_t)T - 1));
  }
  const int64_t n16 = row_bytes / 16;
  for (int64_t e0 = lane; e0 < n16; e0 += 64 * U) {
    u32x4 val[R][U];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = e0 + 64 * u;
        if (rr < nrows && e < n16)
          val[rr][u] = CPTHD_REORDER_LOAD(reinterpret_cast<const u32x4*>(src + g[rr] * row_bytes) + e);
      }
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = e0 + 64 * u;
        if (rr < nrows && e < n16)
          CPTHD_REORDER_STORE(val[rr][u], reinterpret_cast<u32x4*>(dst + (row0 + rr) * row_bytes) + e);
      }
  }
}

// Row gather dst[j] = src[index[j]]: thread u moves VEC-byte piece u % PR of row u / PR
// (PR = row_bytes / VEC pieces per row), so consecutive threads read and write
// consecutive bytes of a row and consecutive rows.
template <typename V>
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ src, int64_t src_rows,
                                                          int64_t row_bytes, const int32_t* __restrict__ index,
                                                          int64_t n, char* __restrict__ dst, int32_t* status) {
  const int64_t PR = row_bytes / (int64_t)sizeof(V);
  const int64_t total = n * PR;
  bool bad = false;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = u / PR, piece = u - j * PR;
    const int64_t i = index[j];
    V val{};
    if (i >= 0 && i < src_rows)
      val = *reinterpret_cast<const V*>(src + i * row_bytes + piece * (int64_t)sizeof(V));
    else
      bad = true;
    *reinterpret_cast<V*>(dst + j * row_bytes + piece * (int64_t)sizeof(V)) = val;
  }
  if (bad && status) atomicOr(status, kDevIndex);
}

}  // namespace cpthd

using namespace cpthd;

extern "C" int cpthd_gather_rows(const void* src, int64_t src_rows, int64_t row_bytes, const int32_t* index,
                                 int64_t n, void* dst, int32_t* dev_status, hipStream_t stream) {
  if (n < 0 || src_rows < 0) return CPTHD_ERR_TOKENS;
  if (n == 0) return CPTHD_OK;
  if (!src || !index || !dst) return CPTHD_ERR_NULL;
  if (row_bytes <= 0 || row_bytes % 4) return CPTHD_ERR_ALIGN;
  const bool wide = row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (reinterpret_cast<uintptr_t>(src) % 4 || reinterpret_cast<uintptr_t>(dst) % 4) return CPTHD_ERR_ALIGN;
  const char* s0 = (const char*)src;
  const char* d0 = (const char*)dst;
  if (d0 < s0 + src_rows * row_bytes && s0 < d0 + n * row_bytes) return CPTHD_ERR_ALIAS;
  const int64_t units = n * (row_bytes / (wide ? 16 : 4));
  const unsigned grid = (unsigned)std::min<int64_t>((units + 255) / 256, 65536);
  if (wide)
    return launch(gather_rows_kernel<u32x4>, dim3(grid), dim3(256), 0, stream, nullptr, 0, 0, (const char*)src,
                  src_rows, row_bytes, index, n, (char*)dst, dev_status);
  return launch(gather_rows_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream, nullptr, 0, 0, (const char*)src,
                src_rows, row_bytes, index, n, (char*)dst, dev_status);
}

extern "C" int cpthd_partition_indices(const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                                       int32_t cp_size, int32_t rank, int32_t strategy, int32_t* out_indices,
                                       int32_t* dev_status, hipStream_t stream) {
  if (!cu_seqlens_padded || !out_indices) return CPTHD_ERR_NULL;
  if (cp_size < 1 || rank < 0 || rank >= cp_size) return CPTHD_ERR_RANK;
  if (int e = check_strategy(strategy)) return e;
  if (int e = check_tokens(total_tokens, total_tokens, cp_size, num_docs)) return e;
  if (int e = check_strategy_tokens(strategy, total_tokens, cp_size)) return e;
  const int64_t S = total_tokens / cp_size;
  const int64_t threads = (S + 3) / 4;
  dim3 grid((unsigned)((threads + 255) / 256));
  return launch(partition_kernel, grid, dim3(256), 0, stream, nullptr, 0, 0, cu_seqlens_padded, num_docs,
                (int)total_tokens, cp_size, rank, strategy, out_indices, dev_status);
}

extern "C" int cpthd_reorder_kv(const void* k_gathered, const void* v_gathered, void* k_out, void* v_out,
                                int64_t row_bytes, const int32_t* cu_seqlens_padded, int32_t num_docs,
                                int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t strategy,
                                int32_t* dev_status, hipStream_t stream) {
  if (!k_gathered || !v_gathered || !k_out || !v_out || !cu_seqlens_padded) return CPTHD_ERR_NULL;
  if (cp_size < 1) return CPTHD_ERR_RANK;
  if (int e = check_strategy(strategy)) return e;
  if (int e = check_tokens(total_tokens, capacity_tokens, cp_size, num_docs)) return e;
  if (int e = check_strategy_tokens(strategy, total_tokens, cp_size)) return e;
  if (row_bytes <= 0 || row_bytes % 16) return CPTHD_ERR_ALIGN;
  for (const void* p : {k_gathered, v_gathered, (const void*)k_out, (const void*)v_out})
    if (reinterpret_cast<uintptr_t>(p) % 16) return CPTHD_ERR_ALIGN;
  const int64_t bytes = total_tokens * row_bytes;
  auto overlap = [bytes](const void* a, const void* b) {
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return x < y + bytes && y < x + bytes;
  };
  if (strategy == CPTHD_NO_LOAD_BALANCE) {
    if (k_out == k_gathered && v_out == v_gathered) return CPTHD_OK;   // already in physical order
    if ((k_out != k_gathered && overlap(k_out, k_gathered)) || (v_out != v_gathered && overlap(v_out, v_gathered)))
      return CPTHD_ERR_ALIAS;
  } else {
    for (const void* o : {(const void*)k_out, (const void*)v_out})
      for (const void* i : {k_gathered, v_gathered})
        if (overlap(o, i)) return CPTHD_ERR_ALIAS;
  }
  if (overlap(k_out, v_out)) return CPTHD_ERR_ALIAS;
  const int64_t rows_per_wg = 4 * kReorderRowsPerWave;
  dim3 grid((unsigned)((total_tokens + rows_per_wg - 1) / rows_per_wg), 2);
  // a NO_LOAD_BALANCE copy where only one of K/V moves copies both; same bytes result
  return launch(reorder_kernel, grid, dim3(256), 0, stream, nullptr, 0, 0, (const char*)k_gathered,
                (const char*)v_gathered, (char*)k_out, (char*)v_out, row_bytes, cu_seqlens_padded, num_docs,
                (int)total_tokens, cp_size, strategy, dev_status);
}

extern "C" const char* cpthd_status_string(int status) {
  switch (status) {
    case CPTHD_OK: return "ok";
    case CPTHD_ERR_NULL: return "a required pointer is NULL";
    case CPTHD_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
    case CPTHD_ERR_RANK: return "cp_size < 1 or rank outside [0, cp_size)";
    case CPTHD_ERR_STRATEGY: return "unknown load-balancing strategy";
    case CPTHD_ERR_TOKENS: return "bad token count (T <= 0, T > capacity, T % cp_size != 0, or num_docs < 1)";
    case CPTHD_ERR_HEADS: return "unsupported heads (Hq % Hkv != 0, Hq/Hkv > 64, or head_dim not in {16,32,64,128})";
    case CPTHD_ERR_MASK: return "only causal attention with window (-1, 0) is supported";
    case CPTHD_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case CPTHD_ERR_LAUNCH: return "HIP kernel launch failed";
    case CPTHD_ERR_ALIGN: return "row size not a multiple of 16 bytes or pointer not 16-byte aligned";
    case CPTHD_ERR_ALIAS: return "output buffer overlaps an input buffer";
    default: return "unknown status";
  }
}
