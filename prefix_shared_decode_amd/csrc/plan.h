// Host-side plan object and helpers (not part of the public ABI).
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/psa.h"
#include "psa_internal.h"

struct psa_plan {
  psa_config cfg{};
  psa_plan_opts opts{};
  int32_t r = 1;
  float sm_scale = 1.f;
  psa_plan_info info{};
  psa::ImageLayout layout{};
  std::vector<uint8_t> image;          // bytes [0, layout.meta_bytes) of the workspace
  std::vector<psa::WorkItem> items;    // host copy of the work list (tests), 4 per unit
  std::vector<int32_t> members;        // member array: the queries of each group, groups in sharing order
  int64_t num_units = 0;               // workgroups of the fused launch
  int64_t num_group_pages = 0;         // query pages follow the group pages in the page array
  uint32_t part_o_bytes = 0, part_ml_bytes = 0;
  std::vector<int32_t> expected;       // per query
  std::vector<int32_t> slot_off;       // per query (-1: written directly)
  uint32_t id = 0;                     // process-unique; also in the image header
  // pinned staging buffer for the upload, allocated on first upload
  void* pinned = nullptr;
  std::mutex mu;
};

struct psa_batch_owned {
  std::vector<int32_t> group_prefix_len;
  std::vector<int64_t> group_page_off;
  std::vector<int32_t> group_pages;
  std::vector<int32_t> query_group;
  std::vector<int32_t> query_distinct_len;
  std::vector<int64_t> query_page_off;
  std::vector<int32_t> query_pages;
  int64_t saved_tokens = 0;
};

namespace psa {

// Thread-local error text.
psa_status set_error(psa_status s, const std::string& msg);

psa_status build_plan(const psa_config* cfg, const psa_batch* batch, const psa_plan_opts* opts,
                      psa_plan** out);

psa_status flatten_tree(const psa_tree* tree, int32_t page_size, psa_batch_owned** out);

// Best first-level reuse of a tree (exposed for tests through the flatten call).
int64_t maximize_reuse(const std::vector<int32_t>& parent, const std::vector<int64_t>& path_len,
                       const std::vector<int32_t>& query_node, std::vector<int32_t>& group_node);

}  // namespace psa
