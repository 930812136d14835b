// Flattening a multi-level prefix tree to single-level prefix-sharing groups.
//
// BatchLLM summary (papercache.org) §4.2 and Fig. 4: keep one prefix level and
// choose it to maximise first-level token reuse, bottom-up on the compact
// prefix tree by dynamic programming; deeper levels are unfolded into the
// requests' distinct parts.  A group of n requests sharing a prefix of a
// tokens saves a * (n - 1) tokens (the Fig. 4 discussion: 1 token shared by 5
// prompts saves 4; 8 tokens shared by 2 saves 8); the total is the saved-token
// count of the saving rate (§3.2 Eq. 2).
//
// DP state: for node x, best[k] = the largest saving inside x's subtree when k
// of its requests are handed to x's parent still ungrouped.  Children combine
// by max-plus convolution, a request attached at x hands up itself, and x may
// then group j >= 2 of the handed-up requests at a saving of a(x) * (j - 1).
// Ties keep fewer groups.
#include <algorithm>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "plan.h"

namespace psa {
namespace {

constexpr int64_t kNeg = std::numeric_limits<int64_t>::min() / 4;

struct NodeDp {
  std::vector<int64_t> out;                // best saving per handed-up count
  std::vector<std::pair<int, int>> choice; // out index -> (count before grouping, grouped j)
  std::vector<std::vector<int>> splits;    // per child: conv split (count taken from child)
  int n_direct = 0;
};

// out[i + j] = max(h[i] + t[j]); split[i + j] = j of the winning pair.
void maxplus(const std::vector<int64_t>& h, const std::vector<int64_t>& t,
             std::vector<int64_t>& out, std::vector<int>& split) {
  out.assign(h.size() + t.size() - 1, kNeg);
  split.assign(out.size(), 0);
  for (size_t i = 0; i < h.size(); ++i) {
    if (h[i] == kNeg) continue;
    for (size_t j = 0; j < t.size(); ++j) {
      if (t[j] == kNeg) continue;
      int64_t v = h[i] + t[j];
      if (v > out[i + j]) {
        out[i + j] = v;
        split[i + j] = (int)j;
      }
    }
  }
}

}  // namespace

int64_t maximize_reuse(const std::vector<int32_t>& parent, const std::vector<int64_t>& path_len,
                       const std::vector<int32_t>& query_node, std::vector<int32_t>& group_node) {
  const int m = (int)parent.size();
  const int root = m;  // virtual root, path length 0
  std::vector<std::vector<int>> kids(m + 1), direct(m + 1);
  for (int d = 0; d < m; ++d) kids[parent[d] < 0 ? root : parent[d]].push_back(d);
  for (int i = 0; i < (int)query_node.size(); ++i)
    direct[query_node[i] < 0 ? root : query_node[i]].push_back(i);

  // post-order
  std::vector<int> order;
  order.reserve(m + 1);
  std::vector<std::pair<int, bool>> st{{root, false}};
  while (!st.empty()) {
    auto [x, done] = st.back();
    st.pop_back();
    if (done) {
      order.push_back(x);
      continue;
    }
    st.push_back({x, true});
    for (int c : kids[x]) st.push_back({c, false});
  }

  std::vector<NodeDp> dp(m + 1);
  std::vector<int64_t> tmp;
  for (int x : order) {
    NodeDp& e = dp[x];
    std::vector<int64_t> h{0};
    for (int c : kids[x]) {
      std::vector<int> sp;
      maxplus(h, dp[c].out, tmp, sp);
      h.swap(tmp);
      e.splits.push_back(std::move(sp));
    }
    // each request attached at x hands itself up: a shift by one
    e.n_direct = (int)direct[x].size();
    if (e.n_direct) h.insert(h.begin(), e.n_direct, kNeg);
    const int64_t a = x == root ? 0 : path_len[x];
    e.out = h;
    e.choice.resize(h.size());
    for (size_t k = 0; k < h.size(); ++k) e.choice[k] = {(int)k, 0};
    if (x != root && a > 0) {
      for (size_t k = 2; k < h.size(); ++k) {
        if (h[k] == kNeg) continue;
        for (size_t j = 2; j <= k; ++j) {
          int64_t v = h[k] + a * (int64_t)(j - 1);
          if (v > e.out[k - j]) {
            e.out[k - j] = v;
            e.choice[k - j] = {(int)k, (int)j};
          }
        }
      }
    }
    for (int c : kids[x]) {  // children tables are no longer needed
      std::vector<int64_t>().swap(dp[c].out);
    }
    if (x != root) {
      // keep only out (needed by the parent); choice/splits kept for backtracking
    }
  }

  const std::vector<int64_t>& rt = dp[root].out;
  int best_k = 0;
  for (int k = 1; k < (int)rt.size(); ++k)
    if (rt[k] > rt[best_k]) best_k = k;
  const int64_t best = rt[best_k];

  // backtrack: explicit stack of (node, k_out, result slot)
  group_node.assign(query_node.size(), -1);
  struct Frame {
    int x, k_out, stage;
    std::vector<int> counts;
    std::vector<int> ids;
    int k_in, j;
    size_t child;
  };
  std::vector<Frame> stack;
  std::vector<int> returned;
  stack.push_back({root, best_k, 0, {}, {}, 0, 0, 0});
  while (!stack.empty()) {
    Frame& f = stack.back();
    NodeDp& e = dp[f.x];
    if (f.stage == 0) {
      f.k_in = e.choice[f.k_out].first;
      f.j = e.choice[f.k_out].second;
      int k = f.k_in - e.n_direct;  // direct requests always hand themselves up
      f.counts.assign(kids[f.x].size(), 0);
      for (int c = (int)kids[f.x].size() - 1; c >= 0; --c) {
        int take = e.splits[c][k];
        f.counts[c] = take;
        k -= take;
      }
      f.child = 0;
      f.stage = 1;
    }
    if (f.stage == 1) {
      if (f.child < kids[f.x].size()) {
        int c = kids[f.x][f.child];
        int cnt = f.counts[f.child];
        ++f.child;
        stack.push_back({c, cnt, 0, {}, {}, 0, 0, 0});
        continue;
      }
      for (int i : direct[f.x]) f.ids.push_back(i);
      if (f.j > 0 && f.x != root) {
        for (int t = 0; t < f.j; ++t) group_node[f.ids[t]] = f.x;
        f.ids.erase(f.ids.begin(), f.ids.begin() + f.j);
      }
      std::vector<int> ids = std::move(f.ids);
      stack.pop_back();
      if (!stack.empty()) {
        Frame& p = stack.back();
        p.ids.insert(p.ids.end(), ids.begin(), ids.end());
      }
      continue;
    }
  }
  return best;
}

psa_status flatten_tree(const psa_tree* tree, int32_t page_size, psa_batch_owned** out) {
  if (!tree || !out) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: null tree or out");
  *out = nullptr;
  if (page_size != 16) return set_error(PSA_ERR_UNSUPPORTED, "flatten: page_size must be 16");
  const int m = tree->num_nodes, n = tree->num_queries;
  if (m < 0 || n < 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: negative counts");
  if ((m > 0 && (!tree->node_parent || !tree->node_len || !tree->node_page_off)) ||
      (n > 0 && (!tree->query_node || !tree->query_distinct_len || !tree->query_page_off)))
    return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: null array");
  if (m > 0 && tree->node_page_off[0] != 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: node_page_off[0] != 0");
  if (n > 0 && tree->query_page_off[0] != 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: query_page_off[0] != 0");
  std::vector<int32_t> parent(m);
  std::vector<int64_t> path(m, -1);
  for (int d = 0; d < m; ++d) {
    int p = tree->node_parent[d];
    if (p < -1 || p >= m) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: bad node_parent");
    int len = tree->node_len[d];
    if (len <= 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: node_len must be > 0");
    if (len % page_size)
      return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: node_len must be a multiple of page_size");
    int64_t a = tree->node_page_off[d], b = tree->node_page_off[d + 1];
    if (b < a) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: node_page_off not monotone");
    if (b - a != len / page_size)
      return set_error(PSA_ERR_OUT_OF_RANGE, "flatten: node page count != node_len / page_size");
    if (b > 0 && !tree->node_pages) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: null node_pages");
    parent[d] = p;
  }
  // path lengths with cycle detection
  for (int d = 0; d < m; ++d) {
    std::vector<int> chain;
    int x = d;
    while (x >= 0 && path[x] < 0) {
      chain.push_back(x);
      if ((int)chain.size() > m) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: cycle in node_parent");
      x = parent[x];
    }
    int64_t base = x < 0 ? 0 : path[x];
    for (int t = (int)chain.size() - 1; t >= 0; --t) {
      base += tree->node_len[chain[t]];
      path[chain[t]] = base;
    }
  }
  std::vector<int32_t> qn(n);
  for (int i = 0; i < n; ++i) {
    int x = tree->query_node[i];
    if (x < -1 || x >= m) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: bad query_node");
    if (tree->query_distinct_len[i] < 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: negative distinct length");
    int64_t a = tree->query_page_off[i], b = tree->query_page_off[i + 1];
    if (b < a) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: query_page_off not monotone");
    if ((int64_t)tree->query_distinct_len[i] > (b - a) * page_size)
      return set_error(PSA_ERR_OUT_OF_RANGE, "flatten: distinct length exceeds its pages");
    if (b > 0 && !tree->query_pages) return set_error(PSA_ERR_INVALID_ARGUMENT, "flatten: null query_pages");
    qn[i] = x;
  }

  std::vector<int32_t> group_node;
  auto* res = new (std::nothrow) psa_batch_owned();
  if (!res) return set_error(PSA_ERR_ALLOC, "flatten: out of memory");
  res->saved_tokens = maximize_reuse(parent, path, qn, group_node);

  // groups with >= 2 members, numbered by node id
  std::vector<int> members(m, 0);
  for (int i = 0; i < n; ++i)
    if (group_node[i] >= 0) ++members[group_node[i]];
  std::vector<int> gid(m, -1);
  auto node_pages = [&](int d, std::vector<int32_t>& dst) {
    for (int64_t t = tree->node_page_off[d]; t < tree->node_page_off[d + 1]; ++t)
      dst.push_back(tree->node_pages[t]);
  };
  auto path_nodes = [&](int d) {
    std::vector<int> p;
    while (d >= 0) {
      p.push_back(d);
      d = parent[d];
    }
    std::reverse(p.begin(), p.end());
    return p;
  };
  res->group_page_off.push_back(0);
  for (int d = 0; d < m; ++d) {
    if (members[d] < 2) continue;
    gid[d] = (int)res->group_prefix_len.size();
    for (int x : path_nodes(d)) node_pages(x, res->group_pages);
    res->group_page_off.push_back((int64_t)res->group_pages.size());
    res->group_prefix_len.push_back((int32_t)path[d]);
  }
  res->query_page_off.push_back(0);
  for (int i = 0; i < n; ++i) {
    int g = group_node[i];
    if (g >= 0 && gid[g] < 0) g = -1;
    std::vector<int> nodes = qn[i] >= 0 ? path_nodes(qn[i]) : std::vector<int>{};
    if (g >= 0) nodes.erase(nodes.begin(), std::find(nodes.begin(), nodes.end(), g) + 1);
    int64_t dl = tree->query_distinct_len[i];
    for (int x : nodes) {
      node_pages(x, res->query_pages);
      dl += tree->node_len[x];
    }
    for (int64_t t = tree->query_page_off[i]; t < tree->query_page_off[i + 1]; ++t)
      res->query_pages.push_back(tree->query_pages[t]);
    if (dl > std::numeric_limits<int32_t>::max()) {
      delete res;
      return set_error(PSA_ERR_OUT_OF_RANGE, "flatten: distinct length overflows int32");
    }
    res->query_page_off.push_back((int64_t)res->query_pages.size());
    res->query_group.push_back(g >= 0 ? gid[g] : -1);
    res->query_distinct_len.push_back((int32_t)dl);
  }
  *out = res;
  return PSA_OK;
}

}  // namespace psa
