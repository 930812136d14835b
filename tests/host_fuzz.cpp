// Host-side fuzz of the plan builder, the tree flattening and the prefix
// identification, built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitize.py (g++, no GPU code: these three sources are
// plain C++).  Random valid inputs must plan without error and satisfy cheap
// invariants; mutated inputs must come back with an error status.  Any
// out-of-bounds access, leak or undefined operation aborts the run.
//
// usage: host_fuzz SEED ITERATIONS
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "plan.h"

namespace psa {
thread_local std::string g_fuzz_err;
psa_status set_error(psa_status s, const std::string& msg) {
  g_fuzz_err = msg;
  return s;
}
}  // namespace psa

namespace {

// splitmix64 (Steele, Lea, Flood 2014)
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  int uni(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }  // [lo, hi]
  bool coin(int pct) { return uni(0, 99) < pct; }
};

int g_fail = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);        \
      std::fprintf(stderr, "\n");               \
      ++g_fail;                                 \
    }                                           \
  } while (0)

struct Batch {
  psa_config cfg{};
  std::vector<int32_t> gl, gp, qg, qd, qp, ql;
  std::vector<int64_t> go, qo;
  bool limits = false;
  psa_batch view() const {
    psa_batch b{};
    b.num_groups = (int32_t)gl.size();
    b.group_prefix_len = gl.data();
    b.group_page_off = go.data();
    b.group_pages = gp.data();
    b.num_queries = (int32_t)qg.size();
    b.query_group = qg.data();
    b.query_distinct_len = qd.data();
    b.query_page_off = qo.data();
    b.query_pages = qp.data();
    b.query_prefix_len = limits ? ql.data() : nullptr;
    return b;
  }
};

const int kHeads[][2] = {{2, 1}, {4, 1}, {32, 8}, {8, 8}, {16, 2}, {8, 1}, {40, 40}};

Batch random_batch(Rng& r) {
  Batch B;
  const auto& h = kHeads[r.uni(0, 6)];
  B.cfg.num_q_heads = h[0];
  B.cfg.num_kv_heads = h[1];
  B.cfg.head_dim = r.coin(50) ? 64 : 128;
  B.cfg.page_size = 16;
  B.cfg.num_pages = r.uni(64, 4096);
  B.cfg.kv_dtype = r.coin(80) ? PSA_BF16 : PSA_F32;
  B.cfg.out_dtype = r.coin(70) ? PSA_F32 : PSA_BF16;
  B.cfg.sm_scale = 0.125f;
  auto page = [&]() { return (int32_t)r.uni(0, B.cfg.num_pages - 1); };
  const int G = r.uni(0, 10);
  B.go.push_back(0);
  for (int g = 0; g < G; ++g) {
    const int lp = r.coin(10) ? 0 : r.uni(1, 2600);
    const int np = (lp + 15) / 16 + (r.coin(10) ? r.uni(1, 3) : 0);  // spare pages are allowed
    // consecutive groups often begin with the same pages (families)
    int shared = 0;
    if (g > 0 && r.coin(50)) {
      const int prev = (int)(B.go[g] - B.go[g - 1]);
      shared = std::min(prev, np) > 0 ? r.uni(0, std::min(prev, np)) : 0;
    }
    for (int k = 0; k < np; ++k) B.gp.push_back(k < shared ? B.gp[B.go[g - 1] + k] : page());
    B.gl.push_back(lp);
    B.go.push_back((int64_t)B.gp.size());
  }
  const int N = r.uni(0, 300);
  B.limits = G > 0 && r.coin(30);
  B.qo.push_back(0);
  for (int i = 0; i < N; ++i) {
    const int g = (G == 0 || r.coin(15)) ? -1 : r.uni(0, G - 1);
    int vis = g >= 0 ? B.gl[g] : 0;
    int lim = 0;
    if (g >= 0 && B.limits) {
      lim = r.coin(40) ? vis : r.uni(0, vis);
      vis = lim;
    }
    int ld = r.coin(15) ? 0 : r.uni(0, 1500);
    if (vis + ld == 0) ld = r.uni(1, 40);
    const int np = (ld + 15) / 16;
    for (int k = 0; k < np; ++k) B.qp.push_back(page());
    B.qg.push_back(g);
    B.qd.push_back(ld);
    B.ql.push_back(lim);
    B.qo.push_back((int64_t)B.qp.size());
  }
  return B;
}

psa_plan_opts random_opts(Rng& r, bool& use) {
  psa_plan_opts o{};
  use = r.coin(70);
  const uint32_t mode[] = {0u, PSA_PLAN_PREFIX_ONLY, PSA_PLAN_DISTINCT_ONLY};
  o.flags = mode[r.uni(0, 2)];
  for (uint32_t f : {PSA_PLAN_FORCE_MATVEC, PSA_PLAN_DEBUG_POISON, PSA_PLAN_NO_XCD_ORDER, PSA_PLAN_NO_TILE_PAIRS,
                     PSA_PLAN_NO_PAGE_SHARING})
    if (r.coin(15)) o.flags |= f;
  if (r.coin(50)) o.prefix_chunk_tokens = 16 * r.uni(1, 128);
  if (r.coin(50)) o.distinct_chunk_tokens = 16 * r.uni(1, 64);
  if (r.coin(30)) o.mfma_min_rows = r.uni(0, 64);
  if (r.coin(50)) o.mfma_tile_rows = 16 * r.uni(1, 8);
  return o;
}

// cheap invariants of a plan built from a valid batch
void check_plan(const psa_plan* p, const Batch& B, bool restricted) {
  const int N = (int)B.qg.size();
  CHECK((int64_t)p->items.size() == 4 * p->num_units, "items %zu units %lld", p->items.size(),
        (long long)p->num_units);
  CHECK(p->info.num_items == p->num_units, "info.num_items");
  CHECK((int)p->expected.size() == N && (int)p->slot_off.size() == N, "per-query arrays");
  int64_t mf = 0;
  for (const auto& it : p->items) {
    const int kind = it.kind & 0xFF;
    CHECK(kind >= 0 && kind <= 3, "item kind %d", kind);
    if (kind == 0) continue;
    CHECK(it.kvh >= 0 && it.kvh < B.cfg.num_kv_heads, "item kv head %d", it.kvh);
    if (kind == 1 || kind == 2) {
      CHECK(0 <= it.tok_begin && it.tok_begin < it.tok_end, "item tokens [%d, %d)", it.tok_begin, it.tok_end);
      CHECK(it.tok_begin % 16 == 0, "tok_begin %d not page aligned", it.tok_begin);
      CHECK(it.page_base >= 0 && it.page_base < (int64_t)(B.gp.size() + B.qp.size()), "page_base %d",
            it.page_base);
    }
    if (kind == 1 || kind == 3) CHECK(it.id >= 0 && it.id < N, "query id %d", it.id);
    if (kind == 2) {
      ++mf;
      CHECK(it.id >= 0 && it.id < (int)B.gl.size(), "group id %d", it.id);
      CHECK(it.b > 0 && it.b <= 128 && it.a >= 0, "tile rows [%d, +%d)", it.a, it.b);
    }
  }
  CHECK(mf == p->info.num_prefix_items, "prefix items %lld vs %lld", (long long)mf,
        (long long)p->info.num_prefix_items);
  for (int i = 0; i < N; ++i) {
    // 0 only when a PREFIX_ONLY / DISTINCT_ONLY plan leaves the query nothing (an empty item)
    CHECK(p->expected[i] >= (restricted ? 0 : 1), "query %d expects %d pieces", i, p->expected[i]);
    CHECK((p->expected[i] >= 2) == (p->slot_off[i] >= 0), "query %d: %d pieces, first slot %d", i, p->expected[i],
          p->slot_off[i]);
  }
  CHECK(p->layout.meta_bytes <= (int64_t)p->info.workspace_bytes, "meta beyond the workspace");
  CHECK(p->image.size() == (size_t)p->layout.meta_bytes, "image size");
  CHECK(p->info.saved_tokens == p->info.logical_tokens - p->info.processed_tokens, "saved tokens");
}

void fuzz_plans(Rng& r, int iters) {
  int ok = 0;
  for (int it = 0; it < iters; ++it) {
    Batch B = random_batch(r);
    bool use = false;
    psa_plan_opts o = random_opts(r, use);
    const psa_batch v = B.view();
    psa_plan* p = nullptr;
    const psa_status s = psa::build_plan(&B.cfg, &v, use ? &o : nullptr, &p);
    CHECK(s == PSA_OK, "valid batch rejected (iteration %d): %s", it, psa::g_fuzz_err.c_str());
    if (s == PSA_OK) {
      ++ok;
      check_plan(p, B, use && (o.flags & (PSA_PLAN_PREFIX_ONLY | PSA_PLAN_DISTINCT_ONLY)));
      delete p;
    }

    // one mutation that makes the batch invalid: an error, never a crash
    Batch M = B;
    const int G = (int)M.gl.size(), N = (int)M.qg.size();
    std::string what;
    switch (r.uni(0, 9)) {
      case 0:  // a page holding prefix tokens (spare pages past the prefix are not read)
        if (G > 0) {
          const int g = r.uni(0, G - 1);
          if (M.gl[g] > 0) {
            M.gp[M.go[g] + r.uni(0, (M.gl[g] + 15) / 16 - 1)] = r.coin(50) ? -1 : M.cfg.num_pages;
            what = "group page id";
          }
        }
        break;
      case 1:
        if (!M.qp.empty()) { M.qp[r.uni(0, (int)M.qp.size() - 1)] = r.coin(50) ? -7 : M.cfg.num_pages + 3; what = "query page id"; }
        break;
      case 2:
        if (G > 0) { M.gl[r.uni(0, G - 1)] = -1; what = "negative prefix"; }
        break;
      case 3:
        if (G > 0) { const int g = r.uni(0, G - 1); M.gl[g] = (int32_t)(M.go[g + 1] - M.go[g]) * 16 + 1; what = "prefix beyond its pages"; }
        break;
      case 4:
        if (N > 0) { M.qg[r.uni(0, N - 1)] = r.coin(50) ? G : -2; what = "group id"; }
        break;
      case 5:
        if (N > 0) { const int i = r.uni(0, N - 1); M.qd[i] = (int32_t)(M.qo[i + 1] - M.qo[i]) * 16 + 16; what = "distinct beyond its pages"; }
        break;
      case 6:
        if (N > 1) { M.qo[1] = M.qo[N] + 1; what = "query offsets not monotone"; }
        break;
      case 7:
        if (M.limits && N > 0) {
          const int i = r.uni(0, N - 1);
          if (M.qg[i] >= 0) { M.ql[i] = r.coin(50) ? -1 : M.gl[M.qg[i]] + 1; what = "prefix limit"; }
        }
        break;
      case 8:
        M.cfg.head_dim = 96;
        what = "head_dim";
        break;
      case 9:
        M.cfg.num_kv_heads = 3;
        what = "head ratio";
        break;
    }
    if (what.empty()) continue;
    const psa_batch mv = M.view();
    p = nullptr;
    const psa_status ms = psa::build_plan(&M.cfg, &mv, use ? &o : nullptr, &p);
    CHECK(ms != PSA_OK && p == nullptr, "invalid batch (%s) accepted", what.c_str());
    delete p;
  }
  std::printf("plans: %d of %d valid batches planned\n", ok, iters);
}

void fuzz_trees(Rng& r, int iters) {
  int ok = 0, rejected = 0;
  for (int it = 0; it < iters; ++it) {
    const int nodes = r.uni(0, 40);
    std::vector<int32_t> parent(nodes), len(nodes), pages;
    std::vector<int64_t> off{0};
    const int num_pages = 2048;
    for (int d = 0; d < nodes; ++d) {
      parent[d] = (d == 0 || r.coin(25)) ? -1 : r.uni(0, d - 1);
      len[d] = 16 * r.uni(1, 40);
      for (int k = 0; k < len[d] / 16; ++k) pages.push_back(r.uni(0, num_pages - 1));
      off.push_back((int64_t)pages.size());
    }
    const bool bad = r.coin(20);
    if (bad && nodes > 1) {
      switch (r.uni(0, 2)) {
        case 0: parent[0] = nodes - 1; parent[nodes - 1] = 0; break;  // cycle
        case 1: parent[r.uni(0, nodes - 1)] = nodes; break;          // out of range
        case 2: len[r.uni(0, nodes - 1)] += 3; break;                 // not page aligned
      }
    }
    const int Q = r.uni(0, 200);
    std::vector<int32_t> qn(Q), qd(Q), qp;
    std::vector<int64_t> qo{0};
    for (int i = 0; i < Q; ++i) {
      qn[i] = (nodes == 0 || r.coin(10)) ? -1 : r.uni(0, nodes - 1);
      qd[i] = r.uni(qn[i] < 0 ? 1 : 0, 300);
      for (int k = 0; k < (qd[i] + 15) / 16; ++k) qp.push_back(r.uni(0, num_pages - 1));
      qo.push_back((int64_t)qp.size());
    }
    psa_tree t{};
    t.num_nodes = nodes;
    t.node_parent = parent.data();
    t.node_len = len.data();
    t.node_page_off = off.data();
    t.node_pages = pages.data();
    t.num_queries = Q;
    t.query_node = qn.data();
    t.query_distinct_len = qd.data();
    t.query_page_off = qo.data();
    t.query_pages = qp.data();
    psa_batch_owned* o = nullptr;
    const psa_status s = psa::flatten_tree(&t, 16, &o);
    if (bad && nodes > 1) {
      if (s != PSA_OK) ++rejected;
      CHECK(s != PSA_OK || o != nullptr, "flatten: OK without a batch");
    } else {
      CHECK(s == PSA_OK, "valid tree rejected: %s", psa::g_fuzz_err.c_str());
    }
    if (s != PSA_OK) continue;
    ++ok;
    CHECK(o->saved_tokens >= 0, "negative saved tokens");
    CHECK((int)o->query_group.size() == Q, "flattened query count");
    // the flattened batch plans
    psa_batch b{};
    b.num_groups = (int32_t)o->group_prefix_len.size();
    b.group_prefix_len = o->group_prefix_len.data();
    b.group_page_off = o->group_page_off.data();
    b.group_pages = o->group_pages.data();
    b.num_queries = Q;
    b.query_group = o->query_group.data();
    b.query_distinct_len = o->query_distinct_len.data();
    b.query_page_off = o->query_page_off.data();
    b.query_pages = o->query_pages.data();
    psa_config c{32, 8, 128, 16, num_pages, PSA_BF16, PSA_F32, 0.088f};
    psa_plan* p = nullptr;
    const psa_status ps = psa::build_plan(&c, &b, nullptr, &p);
    CHECK(ps == PSA_OK, "flattened batch rejected: %s", psa::g_fuzz_err.c_str());
    if (ps == PSA_OK) CHECK(p->info.saved_tokens == o->saved_tokens, "saved tokens differ: plan %lld tree %lld",
                            (long long)p->info.saved_tokens, (long long)o->saved_tokens);
    delete p;
    delete o;
  }
  std::printf("trees: %d flattened, %d malformed rejected\n", ok, rejected);
}

void fuzz_identify(Rng& r, int iters) {
  for (int it = 0; it < iters; ++it) {
    // prompts drawn from a random trie of token runs, with repeats and empties
    const int n = r.uni(0, 120);
    std::vector<std::vector<int32_t>> prompts;
    for (int i = 0; i < n; ++i) {
      std::vector<int32_t> t;
      if (!prompts.empty() && r.coin(70)) {
        const auto& base = prompts[r.uni(0, (int)prompts.size() - 1)];
        t.assign(base.begin(), base.begin() + r.uni(0, (int)base.size()));
      }
      const int extra = r.coin(10) ? 0 : r.uni(0, 60);
      for (int k = 0; k < extra; ++k) t.push_back(r.uni(0, r.coin(50) ? 3 : 50000));
      prompts.push_back(t);
    }
    std::vector<int64_t> off{0};
    std::vector<int32_t> tok;
    for (const auto& p : prompts) {
      tok.insert(tok.end(), p.begin(), p.end());
      off.push_back((int64_t)tok.size());
    }
    psa_prefix_groups* g = nullptr;
    const psa_status s = psa_identify_prefix_groups(n, off.data(), tok.empty() ? nullptr : tok.data(), &g);
    CHECK(s == PSA_OK, "identify rejected valid prompts: %s", psa::g_fuzz_err.c_str());
    if (s != PSA_OK) continue;
    int32_t ng = 0;
    const int32_t *glen = nullptr, *gfirst = nullptr, *rg = nullptr;
    int64_t saved = 0;
    CHECK(psa_prefix_groups_view(g, &ng, &glen, &gfirst, &rg, &saved) == PSA_OK, "view");
    std::vector<int> members(ng, 0);
    int64_t sum = 0;
    for (int i = 0; i < n; ++i) {
      const int x = rg[i];
      CHECK(x >= -1 && x < ng, "request group %d", x);
      if (x < 0) continue;
      ++members[x];
      const auto& a = prompts[i];
      const auto& f = prompts[gfirst[x]];
      // every member holds the group's prefix tokens, equal to the first member's
      CHECK((int)a.size() >= glen[x] && (int)f.size() >= glen[x], "member shorter than its prefix");
      if ((int)a.size() >= glen[x] && (int)f.size() >= glen[x])
        CHECK(std::memcmp(a.data(), f.data(), sizeof(int32_t) * glen[x]) == 0, "member prefix differs");
    }
    for (int x = 0; x < ng; ++x) {
      CHECK(members[x] >= 1 && glen[x] >= 1, "group %d: %d members, prefix %d", x, members[x], glen[x]);
      CHECK(rg[gfirst[x]] == x, "group %d's first request is not in it", x);
      CHECK(x == 0 || gfirst[x] > gfirst[x - 1], "groups not numbered by first member");
      sum += (int64_t)glen[x] * (members[x] - 1);
    }
    CHECK(sum == saved, "saved %lld vs sum %lld", (long long)saved, (long long)sum);
    psa_free_prefix_groups(g);
  }
  // malformed offsets
  const int64_t bad_off[] = {0, 5, 3};
  const int32_t toks[] = {1, 2, 3, 4, 5};
  psa_prefix_groups* g = nullptr;
  CHECK(psa_identify_prefix_groups(2, bad_off, toks, &g) != PSA_OK && g == nullptr, "decreasing offsets accepted");
  const int64_t bad0[] = {1, 5};
  CHECK(psa_identify_prefix_groups(1, bad0, toks, &g) != PSA_OK && g == nullptr, "offset 0 != 0 accepted");
  std::printf("identify: %d prompt sets\n", iters);
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 0;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 200;
  Rng r{seed * 0x2545F4914F6CDD1Dull + 1};
  fuzz_plans(r, iters);
  fuzz_trees(r, iters);
  fuzz_identify(r, iters);
  if (g_fail) {
    std::printf("%d failures\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
