/*
 * psa_debug.h - read-only views of a plan's host data, for tests and tools.
 * Not needed to run attention; the layouts below may change between versions.
 */
#ifndef PSA_DEBUG_H
#define PSA_DEBUG_H

#include "psa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the plan's work list (the order the fused launch runs it in) to host
 * memory `out`: psa_plan_info.num_items units (one per workgroup) of 4 items,
 * 8 int32 per item = {kind | chunk << 8, kv_head, id, tok_begin, tok_end,
 * page_base, a, b}.  kind 0 = nothing, 1 = mat-vec over query `id`'s pages
 * (page_base indexes group pages followed by query pages; a = partials of the
 * query, b = its partial slot or -1), 2 = MFMA prefix tile over group `id`'s
 * pages for rows [a, a + b) of the plan's member array
 * (psa_plan_debug_members; the rows may span several groups whose prefixes
 * hold the same pages there; only as the first item of a unit), 3 = empty
 * partial of query `id`.
 * capacity_items must be >= 4 * num_items. */
psa_status psa_plan_debug_items(const psa_plan* plan, int32_t* out, int64_t capacity_items);

/* The plan's member array (MFMA tile rows are counted over it: row = member
 * index * Hq/Hkv + head in kv group): the queries of every group with members,
 * in query order within a group; groups whose prefixes begin with the same
 * pages are adjacent.  *count receives its length; `out` (capacity entries,
 * may be NULL when capacity is 0) receives the query ids. */
psa_status psa_plan_debug_members(const psa_plan* plan, int32_t* out, int64_t capacity, int64_t* count);

/* Per query: number of partial results merged into its output (1 = the one
 * tile writes it directly) and its first partial slot (-1 if none). */
psa_status psa_plan_debug_queries(const psa_plan* plan, int32_t* expected, int32_t* slot_off, int64_t capacity);

/* psa_decode_attention that also records, per unit (workgroup) of the fused
 * launch, 4 uint64 to device memory d_trace: start and end time of the
 * workgroup (the GPU's constant 100 MHz clock), the HW_ID register (CU, SIMD,
 * shader engine) | XCC_ID << 32, and the unit's kind (1 mat-vec, 2 MFMA
 * prefix tile, 3 empty, 0 nothing).  trace_capacity (entries) must be >=
 * 4 * num_items.  Each workgroup ends with one extra barrier; results are the
 * same as psa_decode_attention's. */
psa_status psa_decode_attention_traced(const psa_plan* plan, const void* d_q, const void* d_k_pool,
                                       const void* d_v_pool, void* d_out, float* d_out_m, float* d_out_l,
                                       void* d_workspace, size_t bytes, void* d_trace, int64_t trace_capacity,
                                       void* stream);

/* Measured ceilings for the rooflines (diagnostics; attention does not use
 * them).  Each call enqueues one launch on `stream`; time it with events.
 *
 * psa_debug_read_peak: reads `bytes` (a positive multiple of 16, at most
 * 2 GiB) of device memory d_buf once, with 16-byte non-temporal loads from
 * 2048 workgroups of 256 threads, and writes one uint32 per thread to d_sink
 * (sink_capacity >= 2048 * 256 entries) so no load is dead.  Bytes read per
 * launch = bytes.
 *
 * psa_debug_mfma_peak: 2048 workgroups of 4 waves; each wave runs `iters`
 * (a positive multiple of 8) dependent v_mfma_f32_16x16x32_bf16, and each
 * thread writes one float to d_out (out_capacity >= 2048 * 256).  Flops per
 * launch = 2048 * 4 * iters * 16384.
 *
 * Errors: NULL or non-device pointers, sizes out of range. */
psa_status psa_debug_read_peak(const void* d_buf, size_t bytes, uint32_t* d_sink, int64_t sink_capacity,
                               void* stream);
psa_status psa_debug_mfma_peak(float* d_out, int64_t out_capacity, int32_t iters, void* stream);

/* Instruction issue rates of one wave (diagnostics): 256 workgroups of 4
 * waves, one workgroup per CU, so that each SIMD holds one wave; each wave
 * times `iters` iterations of one pattern with s_memtime (core clock) and
 * writes the cycles to d_cycles[wave] (int64, capacity >= 1024 entries).
 * Per iteration, pattern
 *   0..4: 16 v_mfma_f32_16x16x32_bf16 in 16, 8, 4, 2 or 1 independent chains;
 *   5:    16 independent v_fma_f32;   6: 8 independent v_exp_f32;
 *   7:    16 MFMAs in 8 chains with 32 v_fma_f32 and 8 v_exp_f32 between
 *         them (the softmax work the MFMA prefix tile issues per MFMA).
 * Errors: NULL or non-device pointer, pattern out of range, iters <= 0,
 * capacity too small. */
psa_status psa_debug_issue_probe(int32_t pattern, int64_t* d_cycles, int64_t capacity, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PSA_DEBUG_H */
