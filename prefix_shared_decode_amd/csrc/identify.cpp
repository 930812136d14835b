// Prefix identification from token ids: the prefix-sharing groups of a batch
// of prompts (BatchLLM summary, papercache.org, §4.2 "explicit global KV reuse
// identification" and the prefix-identification implementation of §5: nested
// input ids in, a list of (prefix, [distinct parts]) groups out).
//
// 1. The prompts' compact prefix tree, built from the prompts sorted by their
//    token sequences: the common prefix length of neighbours in that order
//    (their LCP) gives every branching depth, and a stack over those LCPs
//    links each branching node to the next shallower one.  A node is a depth
//    at which at least two prompts still agree; a prompt hangs at the deepest
//    node it shares with a neighbour (or at the root when it shares nothing).
// 2. The dynamic program of psa_flatten_prefix_tree on that tree (maximise
//    sum over groups of prefix_len * (members - 1)).
//
// Prefixes are token-granular: a group's KV holds tokens [0, prefix_len) once
// (its last page may be partly filled) and each member's distinct part
// starts at token prefix_len in pages of its own, which psa_batch allows.
#include <algorithm>
#include <numeric>
#include <string>
#include <vector>

#include "plan.h"

struct psa_prefix_groups {
  std::vector<int32_t> group_prefix_len;
  std::vector<int32_t> group_first_request;
  std::vector<int32_t> request_group;
  int64_t saved_tokens = 0;
};

namespace psa {

psa_status identify_prefix_groups(int32_t n, const int64_t* off, const int32_t* tok, psa_prefix_groups** out) {
  if (!out) return set_error(PSA_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (n < 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "num_requests < 0");
  if (n > 0 && !off) return set_error(PSA_ERR_INVALID_ARGUMENT, "token_off is NULL");
  if (n > 0 && off[0] != 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "token_off[0] != 0");
  for (int i = 0; i < n; ++i) {
    if (off[i + 1] < off[i]) return set_error(PSA_ERR_INVALID_ARGUMENT, "token_off is not non-decreasing");
    if (off[i + 1] - off[i] > INT32_MAX)
      return set_error(PSA_ERR_UNSUPPORTED, "request " + std::to_string(i) + " is longer than 2^31 tokens");
  }
  if (n > 0 && off[n] > 0 && !tok) return set_error(PSA_ERR_INVALID_ARGUMENT, "tokens is NULL");

  auto len = [&](int i) { return off[i + 1] - off[i]; };
  auto lcp = [&](int a, int b) {
    const int64_t m = std::min(len(a), len(b));
    const int32_t* pa = tok + off[a];
    const int32_t* pb = tok + off[b];
    int64_t k = 0;
    while (k < m && pa[k] == pb[k]) ++k;
    return k;
  };

  // 1. sort by token sequence (ties by index), neighbour LCPs
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    const int32_t* pa = tok + off[a];
    const int32_t* pb = tok + off[b];
    const int64_t m = std::min(len(a), len(b));
    for (int64_t k = 0; k < m; ++k)
      if (pa[k] != pb[k]) return pa[k] < pb[k];
    if (len(a) != len(b)) return len(a) < len(b);
    return a < b;
  });
  std::vector<int64_t> nl(n > 0 ? n - 1 : 0);
  for (int k = 0; k + 1 < n; ++k) nl[k] = lcp(order[k], order[k + 1]);

  // branching nodes from the LCPs: the stack holds the open nodes on the
  // path of the current prompt, deepest last; node_of[k] = the node at depth
  // nl[k] whose prompts include sorted positions k and k + 1
  std::vector<int32_t> parent;
  std::vector<int64_t> depth;
  std::vector<int32_t> node_of(nl.size(), -1);
  std::vector<int32_t> stack;  // node ids; the virtual root (depth 0) is implicit
  auto top_depth = [&]() { return stack.empty() ? (int64_t)0 : depth[stack.back()]; };
  for (size_t k = 0; k < nl.size(); ++k) {
    const int64_t l = nl[k];
    int32_t last = -1;  // the deepest node closed by this LCP
    while (!stack.empty() && top_depth() > l) {
      const int32_t x = stack.back();
      stack.pop_back();
      if (last >= 0) parent[last] = x;
      last = x;
    }
    if (l > 0 && top_depth() < l) {
      const int32_t x = (int32_t)parent.size();
      parent.push_back(stack.empty() ? -1 : stack.back());
      depth.push_back(l);
      if (last >= 0) parent[last] = x;
      stack.push_back(x);
    } else if (last >= 0) {
      parent[last] = stack.empty() ? -1 : stack.back();
    }
    node_of[k] = l > 0 ? stack.back() : -1;
  }
  for (size_t s = stack.size(); s-- > 1;) parent[stack[s]] = stack[s - 1];
  if (!stack.empty()) parent[stack[0]] = -1;

  // each prompt hangs at the deeper of the nodes it shares with its neighbours
  std::vector<int32_t> query_node(n, -1);
  for (int k = 0; k < n; ++k) {
    const int64_t left = k > 0 ? nl[k - 1] : 0, right = k + 1 < n ? nl[k] : 0;
    if (left == 0 && right == 0) continue;
    query_node[order[k]] = left >= right ? node_of[k - 1] : node_of[k];
  }

  // 2. the DP on the tree
  std::vector<int32_t> group_node;
  auto* res = new (std::nothrow) psa_prefix_groups();
  if (!res) return set_error(PSA_ERR_ALLOC, "out of memory");
  res->saved_tokens = maximize_reuse(parent, depth, query_node, group_node);

  // groups numbered in the order of their first member
  std::vector<int32_t> gid(parent.size(), -1);
  res->request_group.assign(n, -1);
  for (int i = 0; i < n; ++i) {
    const int32_t x = group_node[i];
    if (x < 0) continue;
    if (gid[x] < 0) {
      gid[x] = (int32_t)res->group_prefix_len.size();
      res->group_prefix_len.push_back((int32_t)std::min<int64_t>(depth[x], INT32_MAX));
      res->group_first_request.push_back(i);
    }
    res->request_group[i] = gid[x];
  }
  *out = res;
  return PSA_OK;
}

}  // namespace psa

extern "C" {

psa_status psa_identify_prefix_groups(int32_t num_requests, const int64_t* token_off, const int32_t* tokens,
                                      psa_prefix_groups** out) {
  try {
    return psa::identify_prefix_groups(num_requests, token_off, tokens, out);
  } catch (const std::bad_alloc&) {
    return psa::set_error(PSA_ERR_ALLOC, "out of memory");
  }
}

psa_status psa_prefix_groups_view(const psa_prefix_groups* g, int32_t* num_groups, const int32_t** group_prefix_len,
                                  const int32_t** group_first_request, const int32_t** request_group,
                                  int64_t* saved_tokens) {
  if (!g) return psa::set_error(PSA_ERR_INVALID_ARGUMENT, "groups is NULL");
  if (num_groups) *num_groups = (int32_t)g->group_prefix_len.size();
  if (group_prefix_len) *group_prefix_len = g->group_prefix_len.data();
  if (group_first_request) *group_first_request = g->group_first_request.data();
  if (request_group) *request_group = g->request_group.data();
  if (saved_tokens) *saved_tokens = g->saved_tokens;
  return PSA_OK;
}

void psa_free_prefix_groups(psa_prefix_groups* g) { delete g; }

}  // extern "C"
