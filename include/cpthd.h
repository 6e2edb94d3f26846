/*
 * cpthd.h -- one context-parallel (CP) rank's share of causal attention over
 * THD-packed documents, on an AMD Instinct MI355X (gfx950).
 *
 * The operations follow TransformerEngine PR #3221, "[PyTorch] Add
 * no-load-balance THD all-gather CP" (sections "How to use", "What changed",
 * "Why", "Scope and constraints", its commit messages and review thread):
 *
 *   partition  which physical tokens a CP rank owns under a load-balancing
 *              strategy (DualChunkSwap or NO_LOAD_BALANCE);
 *   reorder    restoring the rank-major, all-gathered K/V buffer to physical
 *              token order ("K/V restoration"; contiguous ownership needs none);
 *   plan       the strategy-specific attention metadata of the rank (the
 *              sequence diagram builds it right after gathering K/V);
 *   fwd / bwd  causal attention with window (-1, 0), documents isolated by the
 *              sequence metadata, for the rank's query rows against the whole
 *              physical K/V buffer: O and LSE forward, dQ, dK, dV backward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense and token-major.  Q-side tensors of a rank ("local")
 *   are [S, Hq, D] with S = T / cp_size rows in the rank's local order; K/V-side
 *   tensors are [T, Hkv, D] in physical order.  LSE is [S, Hq] float.
 * - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *   never allocates, frees or retains one after the call returns.  Scratch
 *   space is the caller's workspace (size from cpthd_attn_workspace_bytes),
 *   so a buffer sized once for a token capacity serves every micro-batch.
 * - Capacity vs active T: buffers may be allocated for capacity_tokens rows;
 *   the active data is the prefix of total_tokens rows (S = T / cp_size local
 *   rows).  Kernels read only rows [0, T) / [0, S) and write every row of
 *   those ranges and nothing beyond them.
 * - cu_seqlens_padded (int32, B+1 entries, device) holds the padded slot
 *   offsets of the B documents, cu_seqlens_padded[B] == T.  cu_seqlens
 *   (int32, B+1, device) holds cumulative ACTUAL lengths; the actual tokens of
 *   document i are the prefix [cu_seqlens_padded[i], cu_seqlens_padded[i] + a_i)
 *   of its slot (a_i = cu_seqlens[i+1] - cu_seqlens[i]); the rest are pads,
 *   which neither attend nor are attended.  Without padding between documents
 *   the two arrays are equal.
 * - Rank r's local order: DualChunkSwap cuts every document into 2*cp_size
 *   equal chunks and rank r owns chunk r followed by chunk 2*cp_size-1-r of
 *   document 0, then of document 1, ...; NO_LOAD_BALANCE gives rank r the
 *   physical rows [r*S, (r+1)*S); PACKED_SUPER_SEQUENCE gives rank r the
 *   physical rows [r*c, (r+1)*c) followed by [(2*cp_size-1-r)*c,
 *   (2*cp_size-r)*c) with c = T / (2*cp_size).  In every case the local rows
 *   are increasing in physical index.
 * - Every call is asynchronous on the caller's HIP stream; there is no
 *   device or stream synchronisation inside the library.  The library holds
 *   no mutable global state; concurrent calls on different buffers are safe.
 * - Errors: the return value is a status.  0 = success; a negative value is
 *   an argument error detected on the host BEFORE anything is launched (see
 *   CPTHD_ERR_*; cpthd_status_string names it).  Violations that depend on
 *   device data (the contents of the cu arrays) are OR-ed as CPTHD_DEV_* bits
 *   into *dev_status (a device int32 the caller zeroes; NULL = unchecked).
 *   A call that raises a device bit leaves its outputs unspecified but never
 *   touches memory outside its arguments' ranges; an attention call whose cu
 *   arrays are rejected writes none of its outputs.
 * - A workspace serves one call at a time: calls that share a workspace must
 *   be ordered on one stream (or synchronised), since each may rebuild the plan
 *   in it.
 */
#ifndef CPTHD_H
#define CPTHD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Load-balancing strategy (PR #3221 "How to use": DUAL_CHUNK_SWAP is the
 * default, NO_LOAD_BALANCE the experimental contiguous strategy; the commit
 * messages' earlier packed policy, PACKED_SUPER_SEQUENCE, cuts the whole
 * physical buffer into 2*cp_size mirrored chunks as one partitioning sequence
 * and keeps documents apart only through the sequence metadata). */
#define CPTHD_DUAL_CHUNK_SWAP 0
#define CPTHD_NO_LOAD_BALANCE 1
#define CPTHD_PACKED_SUPER_SEQUENCE 2

/* Host-detected status codes (nothing was launched). */
#define CPTHD_OK 0
#define CPTHD_ERR_NULL (-1)       /* a required pointer is NULL */
#define CPTHD_ERR_RANK (-2)       /* cp_size < 1 or rank outside [0, cp_size) */
#define CPTHD_ERR_STRATEGY (-3)   /* unknown strategy */
#define CPTHD_ERR_TOKENS (-4)     /* T <= 0, T > capacity, T % cp_size (T % (2*cp_size) for PACKED_SUPER_SEQUENCE),
                                     num_docs < 1, capacity > INT32_MAX */
#define CPTHD_ERR_HEADS (-5)      /* Hq % Hkv, Hq/Hkv > 64, head_dim not in {16,32,64,128} */
#define CPTHD_ERR_MASK (-6)       /* causal != 1 or window != (-1, 0) */
#define CPTHD_ERR_WORKSPACE (-7)  /* workspace NULL / too small / misaligned */
#define CPTHD_ERR_LAUNCH (-8)     /* a HIP launch failed */
#define CPTHD_ERR_ALIGN (-9)      /* reorder rows not a multiple of 16 bytes or pointers not 16-byte aligned */
#define CPTHD_ERR_ALIAS (-10)     /* an output buffer overlaps an input buffer */
#define CPTHD_ERR_SCRATCH (-11)   /* cpthd_attn_bwd_noalloc: the call needs more than CPTHD_STATIC_SCRATCH_BYTES */

/* Device-detected status bits, OR-ed into *dev_status. */
#define CPTHD_DEV_CU_ORDER 1      /* cu_seqlens_padded not non-decreasing, or [0] != 0 */
#define CPTHD_DEV_CU_TOTAL 2      /* cu_seqlens_padded[B] != T */
#define CPTHD_DEV_DCS_DIVISIBLE 4 /* DualChunkSwap: a padded length not divisible by 2*cp_size */
#define CPTHD_DEV_ACTUAL 8        /* cu_seqlens not non-decreasing, or an actual length > padded length */
#define CPTHD_DEV_PLAN 16         /* the workspace does not hold a plan for these arguments */
#define CPTHD_DEV_INDEX 32        /* a gather index outside [0, src_rows) (that row is written as zeros) */
#define CPTHD_DEV_DOC_BYTES 64    /* a document's K/V rows (padded length * Hkv * head_dim * 2 bytes) reach 2 GiB */

/*
 * cpthd_partition_indices -- the physical token indices rank `rank` owns
 * (PR #3221 "Why": DualChunkSwap gives each rank two mirrored chunks of every
 * document; NO_LOAD_BALANCE one contiguous chunk of the physical buffer;
 * commit messages: PACKED_SUPER_SEQUENCE two mirrored chunks of the whole
 * buffer; "What changed": the native partition-index routine used for batch
 * slicing).
 *
 *   cu_seqlens_padded  device int32 [num_docs + 1]
 *   total_tokens       T (must equal cu_seqlens_padded[num_docs]; checked on device)
 *   out_indices        device int32 [T / cp_size], written in local order
 * Errors: NULL, RANK, STRATEGY, TOKENS, LAUNCH; device bits CU_ORDER,
 * CU_TOTAL, DCS_DIVISIBLE.
 */
int cpthd_partition_indices(const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                            int32_t cp_size, int32_t rank, int32_t strategy, int32_t* out_indices,
                            int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_reorder_kv -- restore the all-gathered K and V to physical order
 * (PR #3221 review thread: the THD stream wait "follows K/V restoration";
 * commit messages: rank-major ownership "needs no KV reorder").
 *
 *   k_gathered, v_gathered  device [T rows x row_bytes], rank-major: rows
 *                           [s*S, (s+1)*S) hold rank s's local rows
 *   k_out, v_out            device [T rows x row_bytes], physical order
 *   row_bytes               bytes per token row (Hkv * D * sizeof(elem));
 *                           multiple of 16, pointers 16-byte aligned
 * DualChunkSwap and PACKED_SUPER_SEQUENCE: out[idx_s[j]] = gathered[s*S + j]
 * for every rank s, j (bit-exact copy; outputs must not overlap inputs).
 * NO_LOAD_BALANCE: the
 * gathered buffer is already in physical order; the call copies it when
 * out != in and does nothing when out == in.
 * Errors: NULL, RANK (cp_size < 1), STRATEGY, TOKENS, ALIGN, ALIAS, LAUNCH;
 * device bits CU_ORDER, CU_TOTAL, DCS_DIVISIBLE.
 */
int cpthd_reorder_kv(const void* k_gathered, const void* v_gathered, void* k_out, void* v_out,
                     int64_t row_bytes, const int32_t* cu_seqlens_padded, int32_t num_docs,
                     int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t strategy,
                     int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_gather_rows -- dst[j] = src[index[j]] for j in [0, n): the rank's
 * slice of per-token tensors (PR #3221 "How to use": input_ids, labels and
 * position_ids are partitioned with the same strategy as attention, by the
 * rank's partition indices; position ids stay global positions).  Works on
 * raw rows of any element type.
 *
 *   src        device, src_rows rows of row_bytes bytes
 *   index      device int32 [n] (e.g. from cpthd_partition_indices)
 *   dst        device, n rows of row_bytes bytes; must not overlap src
 *   row_bytes  multiple of 4; pointers 4-byte aligned (16 for 16-byte rows)
 * An index outside [0, src_rows) writes a zero row and sets CPTHD_DEV_INDEX.
 * Errors: NULL, TOKENS (n < 0, src_rows < 0), ALIGN, ALIAS, LAUNCH.
 */
int cpthd_gather_rows(const void* src, int64_t src_rows, int64_t row_bytes, const int32_t* index, int64_t n,
                      void* dst, int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_attn_workspace_bytes -- workspace size for cpthd_attn_plan /
 * cpthd_attn_fwd / cpthd_attn_bwd at a token capacity and document count:
 * the plan, per-row backward scratch, partial-result slots for split tiles
 * (see cpthd_attn_plan) and, for the forward, V^T rows of the documents'
 * keys (Hkv * D rows of 128 columns per key tile; left out where a kv head's
 * rows would pass 2 GiB).  A smaller workspace is accepted down to the size of
 * the plan and row scratch alone (below it: CPTHD_ERR_WORKSPACE): it holds the
 * V^T rows only if they fit beside the plan, then as many partial slots as
 * fit, so fewer tiles are split.  The plan, and so the results, depend on the
 * workspace size only through that slot count.
 * Returns 0 for arguments no call would accept.
 */
size_t cpthd_attn_workspace_bytes(int64_t capacity_tokens, int32_t cp_size, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_docs);

/*
 * cpthd_attn_workspace_min_bytes -- the smallest workspace the attention calls
 * accept for the same arguments: the plan and row scratch without partial
 * slots, so no tile is split.  Returns 0 where cpthd_attn_workspace_bytes does.
 */
size_t cpthd_attn_workspace_min_bytes(int64_t capacity_tokens, int32_t cp_size, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t max_docs);

/*
 * cpthd_attn_plan -- build the rank's attention metadata into `workspace`
 * (PR #3221 sequence diagram: the CP layer builds metadata specific to the
 * strategy once K/V are gathered; commit messages: NO_LOAD_BALANCE has one
 * chunk and one attention step per rank, DualChunkSwap two steps).  The plan
 * lists the rank's query tiles (each inside one document, with its causal key
 * range) and the key tiles of every document with the rank's query rows that
 * see them, ordered longest first; it records the arguments and a copy of the
 * cu arrays it was built from.  A tile whose work exceeds one compute unit's
 * share of its launch (the list's work times Hkv over the device's compute
 * units) is cut into parts -- a key tile along its query chunks; a query tile
 * along its key steps, only when the call's query tiles times Hkv are fewer
 * than the compute units -- as far as the workspace's partial slots allow;
 * the parts write fp32 partial results that a merge kernel combines in part
 * order, so results do not depend on the order in which work-groups run.  Every attention call checks the workspace's
 * plan against its own arguments and cu arrays and rebuilds it when they
 * differ, so calling this first is optional: it moves the build of a
 * micro-batch's plan ahead of its first attention call.
 *
 *   cu_seqlens, cu_seqlens_padded  device int32 [num_docs + 1]
 *   workspace                      device, cpthd_attn_workspace_bytes(...) bytes
 *                                  for capacity_tokens and num_docs (or fewer, see
 *                                  there), 256-byte aligned
 * Errors: NULL, RANK, STRATEGY, TOKENS, HEADS, WORKSPACE, LAUNCH; device bits
 * CU_ORDER, CU_TOTAL, DCS_DIVISIBLE, ACTUAL, DOC_BYTES (the kernels address a
 * document's K/V rows through one 32-bit buffer range).  A layout that raises
 * a device bit leaves no plan in the workspace.
 */
int cpthd_attn_plan(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t num_docs,
                    int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t rank,
                    int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_attn_fwd -- causal attention forward for the rank's query rows
 * (PR #3221 "Scope and constraints": THD self-attention, causal without a
 * sliding window, window_size = (-1, 0), equal local Q/K/V lengths; review
 * thread: documents stay isolated through cu_seqlens).
 * For local row i at physical token p (document d, position pos) and q head
 * h (kv head h / (Hq/Hkv)): scores softmax_scale * q.k over the actual keys of
 * document d at positions <= pos;  lse = log(sum(exp(scores))) (natural log),
 * o = softmax(scores) @ v.  Pad rows: o = 0, lse = -inf.
 *
 *   q_local   device bf16 [S, Hq, D]          k, v  device bf16 [T, Hkv, D] (physical order)
 *   cu_seqlens, cu_seqlens_padded             device int32 [num_docs + 1], the micro-batch's documents
 *   o_local   device bf16 [S, Hq, D] (out)    lse_local  device float [S, Hq] (out)
 *   workspace device, cpthd_attn_workspace_bytes(capacity_tokens, ..., num_docs) bytes (or fewer, see
 *             there), 256-byte aligned; holds the plan (built or checked by this call, see
 *             cpthd_attn_plan) and the partial results of split tiles
 * Launches the plan check (a rebuild when the workspace holds another plan);
 * for head dim 64 and 128, when the workspace holds V^T rows (see
 * cpthd_attn_workspace_bytes), a pass that writes V^T of the call's documents
 * there, so the attention kernel reads its V^T operand as rows instead of
 * through the transpose LDS read; the attention kernel; and, when query tiles
 * may be split (see cpthd_attn_plan) and the workspace has partial slots, a
 * kernel that merges the parts of split tiles.  With or without V^T the
 * results are the same bits.
 * Errors: NULL, RANK, STRATEGY, TOKENS, HEADS, MASK, WORKSPACE, LAUNCH; device
 * bits as cpthd_attn_plan (then nothing is written) and PLAN.
 */
int cpthd_attn_fwd(const void* q_local, const void* k, const void* v, const int32_t* cu_seqlens,
                   const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                   int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                   int32_t window_left, int32_t window_right, void* o_local, float* lse_local, void* workspace,
                   size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_attn_bwd -- gradients of cpthd_attn_fwd for an upstream gradient dO
 * (PR #3221 "What changed": backward uses the strategy, and so the token
 * layout, captured in forward; the caller passes the same layout arguments).
 * delta = rowsum(dO * O); dS = P * (dP - delta) with dP = dO @ v^T;
 * dq = scale * dS @ k for the rank's rows; dk = scale * dS^T @ q and
 * dv = P^T @ dO summed over the rank's query rows and the Hq/Hkv q heads of
 * each kv head.  dk/dv are this rank's PARTIAL gradients over all T physical
 * rows (rows no query of the rank sees are written as 0); summing them over
 * the ranks gives the unpartitioned gradient.  Pad rows give dq = 0.
 *
 *   q_local, o_local, do_local  device bf16 [S, Hq, D]   lse_local device float [S, Hq]
 *   k, v                        device bf16 [T, Hkv, D]
 *   cu_seqlens, cu_seqlens_padded, workspace  as cpthd_attn_fwd
 *   dq_local                    device float [S, Hq, D] (out)
 *   dk, dv                      device float [T, Hkv, D] (out)
 * Launches three kernels (plan check; query-tile pass: delta and dq; key-tile
 * pass: dk, dv), then, when the workspace has partial slots, a fourth that
 * merges the parts of split tiles.  Errors as cpthd_attn_fwd.
 */
int cpthd_attn_bwd(const void* q_local, const void* k, const void* v, const void* o_local,
                   const void* do_local, const float* lse_local, const int32_t* cu_seqlens,
                   const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                   int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                   int32_t window_left, int32_t window_right, float* dq_local, float* dk, float* dv,
                   void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_attn_fwd_allgathered / cpthd_attn_bwd_allgathered -- cpthd_attn_fwd and
 * cpthd_attn_bwd with k and v (and, backward, dk and dv) in the rank-major
 * all-gathered order instead of physical order: row s*S + j holds the token
 * at local row j of rank s, which is what an all-gather of the ranks' local
 * K/V produces (PR #3221 "Why" and commit messages: contiguous, rank-major
 * ownership needs no K/V reorder; the other strategies pay a restoration).
 * The kernels read every key through the inverse of the partition, so no
 * restoration pass (cpthd_reorder_kv) and no physical-order copy of K/V are
 * needed.  dk/dv are written in the same gathered order, which is the layout
 * a reduce-scatter over the ranks splits into per-rank slices.  Results are
 * identical to cpthd_reorder_kv + cpthd_attn_fwd / cpthd_attn_bwd with dk/dv
 * permuted.  Under NO_LOAD_BALANCE the two orders coincide.
 *
 * Arguments, plan and errors as cpthd_attn_fwd / cpthd_attn_bwd, plus:
 * under DUAL_CHUNK_SWAP and PACKED_SUPER_SEQUENCE, T * Hkv * D * 2 must be
 * below 2^31 bytes (CPTHD_ERR_TOKENS otherwise).
 */
int cpthd_attn_fwd_allgathered(const void* q_local, const void* k_gathered, const void* v_gathered,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t num_docs,
                               int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t rank,
                               int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
                               void* o_local, float* lse_local, void* workspace, size_t workspace_bytes,
                               int32_t* dev_status, hipStream_t stream);
int cpthd_attn_bwd_allgathered(const void* q_local, const void* k_gathered, const void* v_gathered,
                               const void* o_local, const void* do_local, const float* lse_local,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t num_docs,
                               int64_t total_tokens, int64_t capacity_tokens, int32_t cp_size, int32_t rank,
                               int32_t strategy, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
                               float* dq_local, float* dk_gathered, float* dv_gathered, void* workspace,
                               size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * cpthd_attn_bwd_noalloc -- cpthd_attn_bwd (physical-order K/V) without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc.
 * Its scratch (the plan, -delta and LSE rows, partial slots) is a device
 * array of CPTHD_STATIC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; the call allocates and frees nothing.  It builds the
 * plan a workspace of CPTHD_STATIC_SCRATCH_BYTES bytes gets.  The array is the
 * current device's: call with the device of the buffers current.
 * Every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (different streams, or host threads without ordering) race; order them
 * on one stream.  A call whose plan and rows need more than the array holds
 * returns CPTHD_ERR_SCRATCH before launching anything.
 * Arguments, results and other errors as cpthd_attn_bwd.
 */
#define CPTHD_STATIC_SCRATCH_BYTES 16777216u /* 16 MiB */
int cpthd_attn_bwd_noalloc(const void* q_local, const void* k, const void* v, const void* o_local,
                           const void* do_local, const float* lse_local, const int32_t* cu_seqlens,
                           const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                           int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                           int32_t causal, int32_t window_left, int32_t window_right, float* dq_local, float* dk,
                           float* dv, int32_t* dev_status, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* cpthd_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* CPTHD_H */
