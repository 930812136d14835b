// Internal structures shared by the host plan and the device kernels.
#pragma once

#include <stdint.h>

namespace psa {

// Kinds of work items in the fused launch (BatchLLM summary, papercache.org,
// §5: the parts of the computation run in different workgroups, each with its
// own tiling).
enum ItemKind : int32_t {
  ITEM_NOP = 0,             // nothing (padding of a unit)
  ITEM_MATVEC = 1,          // one (query, kv head, token chunk): mat-vec, one wave
  ITEM_PREFIX_MFMA = 2,     // one (group, kv head, row tile, prefix chunk): MFMA, whole workgroup
  ITEM_EMPTY = 3,           // empty partial (0, -inf, 0) of every head of a query, one wave
};

// 32-byte work item.  The fused launch runs one *unit* per workgroup; a unit
// is 4 consecutive items: either one MFMA prefix tile (items 1..3 NOP) or up
// to 4 wave-level items (mat-vec / empty), one per wave.
struct WorkItem {
  int32_t kind;       // ItemKind in bits 0..7; MFMA: prefix chunk index j in bits 8..31
  int32_t kvh;
  int32_t id;         // query (mat-vec, empty) or group (MFMA)
  int32_t tok_begin;  // token range inside the segment; tok_begin is page aligned
  int32_t tok_end;
  int32_t page_base;  // index in the page array of the page holding tok_begin
  int32_t a;          // MFMA: first row (row = (member_off[group] + member) * r + head); mat-vec: partials of the query
  int32_t b;          // MFMA: rows; mat-vec: partial slot ((slot_off + j) * hkv + kvh), -1 = write out
};
static_assert(sizeof(WorkItem) == 32, "WorkItem must stay 32 bytes");

constexpr int kUnitItems = 4;
constexpr int kMaxMatvecPages = 64;   // a mat-vec chunk holds at most 64 pages (1024 tokens)
constexpr int kMaxPrefixChunk = 2048; // tokens per MFMA prefix chunk (page ids staged in LDS)

// First 8 bytes of a workspace image: a magic word and the id of the plan
// that uploaded it.  The kernel compares them with the launching plan's id
// before it reads anything else from the workspace.
constexpr uint32_t kImageMagic = 0x31415350u;  // "PSA1"

// Device image of a plan: the workspace begins with these arrays, at the
// byte offsets the plan records (int32 everywhere on the device).
struct ImageLayout {
  int64_t header;  // {kImageMagic, plan id}
  int64_t items, pages, member_off, members, expected, slot_off;
  int64_t qlim;  // visible prefix tokens per query, -1 = no limits (every query sees its whole prefix)
  int64_t counters, part_o, part_ml;
  int64_t meta_bytes;   // bytes copied by the upload (everything before part_o), counters included
  int64_t total_bytes;  // workspace size
};

// Launch arguments of the fused kernel (passed by value).
struct DecodeParams {
  const uint32_t* header;   // workspace image header: {kImageMagic, plan_id}
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* out_m;
  float* out_l;
  const WorkItem* items;    // [num_units * 4]
  const int32_t* pages;     // group prefix pages, then query distinct pages
  const int32_t* member_off;
  const int32_t* members;
  const int32_t* expected;  // partials per query (same for every kv head)
  const int32_t* slot_off;  // first partial slot of each query, -1 if written directly
  const int32_t* qlim;      // prefix tokens each query sees, or nullptr (all of its group's)
  int32_t* counters;        // [num_queries * hkv] arrivals, self-resetting
  float* part_o;            // [slots * hkv][r][d]
  float* part_ml;           // [slots * hkv][r][2] (m in log2 units, l)
  uint32_t part_o_bytes;
  uint32_t part_ml_bytes;
  int32_t num_units;
  uint32_t plan_id;         // id of the launching plan (must match the image header)
  int32_t num_queries;
  int32_t hq;
  int32_t hkv;
  float scale_log2;         // sm_scale * log2(e)
  int32_t out_bf16;
  uint64_t* trace;          // optional, [num_units][4]: start, end (100 MHz clock), HW_ID | XCC_ID << 32, kind
};

}  // namespace psa
