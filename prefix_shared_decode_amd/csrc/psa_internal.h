// Internal structures shared by the host plan and the device kernels.
#pragma once

#include <stdint.h>

namespace psa {

// Kinds of work items in the fused launch (BatchLLM §5: the parts of the
// computation run in different workgroups, each with its own tiling).
enum ItemKind : int32_t {
  ITEM_MATVEC_DISTINCT = 0,  // one (query, kv head, distinct chunk): mat-vec tile
  ITEM_MATVEC_PREFIX = 1,    // one (query, kv head, prefix chunk) of a small group
  ITEM_PREFIX_MFMA = 2,      // one (group, kv head, row tile, prefix chunk): MFMA tile
  ITEM_EMPTY = 3,            // write the empty partial (0, -inf, 0) for all heads of a query
  ITEM_NOP = 4,              // padding (keeps per-XCD queues aligned)
};

// 32-byte work item; one per workgroup.
struct WorkItem {
  int32_t kind;
  int32_t kvh;
  int32_t id;         // query index (mat-vec, empty) or group index (MFMA)
  int32_t tok_begin;  // token range inside the segment; tok_begin is page-aligned
  int32_t tok_end;
  int32_t row_begin;  // MFMA: first row of the group (row = member * r + head_in_group)
  int32_t row_count;  // MFMA: rows in this tile (<= 128)
  int32_t slot;       // index j of this partial among the query's partials
};
static_assert(sizeof(WorkItem) == 32, "WorkItem must stay 32 bytes");

// Device image of a plan: the workspace begins with these arrays, at the
// byte offsets the plan records.  int32 everywhere on the device.
struct ImageLayout {
  int64_t items, group_page_off, group_pages, group_len, member_off, members;
  int64_t query_page_off, query_pages, query_group, query_dlen, expected, slot_off;
  int64_t counters, part_o, part_ml;
  int64_t meta_bytes;   // bytes copied by the upload (everything before part_o), counters included
  int64_t total_bytes;  // workspace size
};

// Launch arguments of the fused kernel (passed by value).
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* out_m;
  float* out_l;
  const WorkItem* items;
  const int32_t* group_page_off;
  const int32_t* group_pages;
  const int32_t* group_len;
  const int32_t* member_off;
  const int32_t* members;
  const int32_t* query_page_off;
  const int32_t* query_pages;
  const int32_t* query_group;
  const int32_t* query_dlen;
  const int32_t* expected;  // partials per query (same for every kv head)
  const int32_t* slot_off;  // first partial slot of each query
  int32_t* counters;        // [num_queries * hkv] arrivals, self-resetting
  float* part_o;            // [slots * hkv * r * d]
  float* part_ml;           // [slots * hkv * r * 2] (m natural-log, l)
  int32_t num_items;
  int32_t num_queries;
  int32_t hq;
  int32_t hkv;
  float scale_log2;         // sm_scale * log2(e)
  int32_t out_bf16;
};

}  // namespace psa
