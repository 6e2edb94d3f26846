/*
 * cpthd_timing.h -- instrumentation variants of the attention entry points of
 * cpthd.h, for benchmarks that time each kernel a call launches.
 *
 * cpthd_attn_fwd_timed and cpthd_attn_bwd_timed compute exactly what
 * cpthd_attn_fwd and cpthd_attn_bwd compute (or, with kv_allgathered != 0,
 * cpthd_attn_fwd_allgathered and cpthd_attn_bwd_allgathered), with the same
 * arguments, checks and errors, plus:
 *
 *   kv_allgathered  0: k, v (dk, dv) in physical order; else rank-major all-gathered order
 *   events          n_events caller-created hipEvent_t handles (host array), used in
 *                   (start, stop) pairs around the kernels the call launches, in
 *                   launch order, recorded by hipExtLaunchKernel on `stream`:
 *                   forward  pair 0 plan check, pair 1 attention, pair 2 merge of
 *                            split query tiles, pair 3 the V^T pass (launched
 *                            before the attention kernel);
 *                   backward pair 0 plan check, pair 1 query-tile pass (delta, dq),
 *                            pair 2 key-tile pass (dk, dv), pair 3 merge of split
 *                            tiles (dq, dk, dv).
 *                   The merge kernels are launched when tiles may be split (see
 *                   cpthd_attn_plan, cpthd_attn_fwd and cpthd_attn_bwd); a pair
 *                   whose kernel a call leaves out is recorded back to back.
 *                   A kernel whose pair lies beyond n_events is launched untimed.
 *                   The events stay the caller's; the call only records them.
 */
#ifndef CPTHD_TIMING_H
#define CPTHD_TIMING_H

#include "cpthd.h"

#ifdef __cplusplus
extern "C" {
#endif

int cpthd_attn_fwd_timed(const void* q_local, const void* k, const void* v, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                         int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                         int32_t causal, int32_t window_left, int32_t window_right, void* o_local, float* lse_local,
                         void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream,
                         int32_t kv_allgathered, hipEvent_t* events, int32_t n_events);

int cpthd_attn_bwd_timed(const void* q_local, const void* k, const void* v, const void* o_local,
                         const void* do_local, const float* lse_local, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_padded, int32_t num_docs, int64_t total_tokens,
                         int64_t capacity_tokens, int32_t cp_size, int32_t rank, int32_t strategy,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                         int32_t causal, int32_t window_left, int32_t window_right, float* dq_local, float* dk,
                         float* dv, void* workspace, size_t workspace_bytes, int32_t* dev_status,
                         hipStream_t stream, int32_t kv_allgathered, hipEvent_t* events, int32_t n_events);

#ifdef __cplusplus
}
#endif
#endif /* CPTHD_TIMING_H */
