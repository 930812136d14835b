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
 * memory `out`: 8 int32 per item = {kind, kv_head, id, tok_begin, tok_end,
 * row_begin, row_count, slot}; kind 0 = mat-vec over a query's distinct pages,
 * 1 = mat-vec over its group's prefix pages, 2 = MFMA prefix tile over rows
 * [row_begin, row_begin + row_count) of group `id` (row = member * Hq/Hkv +
 * head in kv group), 3 = empty partial of query `id`.  capacity_items must be
 * >= psa_plan_info.num_items. */
psa_status psa_plan_debug_items(const psa_plan* plan, int32_t* out, int64_t capacity_items);

/* Per query: number of partial results merged into its output (1 = the one
 * tile writes it directly) and its first partial slot (-1 if none). */
psa_status psa_plan_debug_queries(const psa_plan* plan, int32_t* expected, int32_t* slot_off, int64_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* PSA_DEBUG_H */
