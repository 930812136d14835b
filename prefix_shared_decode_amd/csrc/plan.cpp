// Host plan: validate -> chunk -> classify -> order -> lay out the workspace.
//
// BatchLLM summary (papercache.org):
//  * §4.3.1 / §5: the prefix-sharing group is the unit of work; the input is a
//    list of (prefix, [distinct ...]) groups.
//  * §5 "horizontal fusion": prefix and distinct work run in different
//    workgroups of ONE launch, each part with its own tiling.
//  * §2.2: the shared-prefix part becomes a matrix multiply (all queries of a
//    group against one K/V); the distinct part stays a mat-vec.
//  * §6.3.3: when many requests share a prefix much longer than their
//    distinct parts, split the long KV range (split-K) so the work balances.
//  * §3.2 Eq. 2: saved tokens = logical - processed.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <string>
#include <vector>

#include "plan.h"

namespace psa {
namespace {

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Process-unique plan ids (never 0), written into each plan's workspace image.
uint32_t next_plan_id() {
  static std::atomic<uint32_t> counter{0};
  uint32_t id;
  do id = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  while (id == 0);
  return id;
}
int64_t ceil_div(int64_t x, int64_t a) { return (x + a - 1) / a; }

psa_status check_segment(const char* what, int64_t idx, int64_t len, int64_t off_a, int64_t off_b,
                         const int32_t* pages, int32_t P, int32_t num_pages) {
  if (len < 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(what) + " " + std::to_string(idx) + ": negative length");
  if (off_b < off_a)
    return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(what) + " page offsets not monotone at " + std::to_string(idx));
  if (len > (off_b - off_a) * P)
    return set_error(PSA_ERR_OUT_OF_RANGE, std::string(what) + " " + std::to_string(idx) +
                                               ": length exceeds its pages * page_size");
  const int64_t need = ceil_div(len, P);
  for (int64_t t = off_a; t < off_a + need; ++t) {
    if (pages[t] < 0 || pages[t] >= num_pages)
      return set_error(PSA_ERR_OUT_OF_RANGE, std::string(what) + " " + std::to_string(idx) + ": page id " +
                                                 std::to_string(pages[t]) + " outside [0, num_pages)");
  }
  return PSA_OK;
}

}  // namespace

psa_status build_plan(const psa_config* cfg, const psa_batch* b, const psa_plan_opts* opts_in,
                      psa_plan** out) {
  if (!out) return set_error(PSA_ERR_INVALID_ARGUMENT, "build_plan: out is NULL");
  *out = nullptr;
  if (!cfg || !b) return set_error(PSA_ERR_INVALID_ARGUMENT, "build_plan: cfg or batch is NULL");
  const psa_config c = *cfg;
  if (c.num_q_heads <= 0 || c.num_kv_heads <= 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "head counts must be positive");
  if (c.num_q_heads % c.num_kv_heads)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "num_q_heads must be a multiple of num_kv_heads");
  const int r = c.num_q_heads / c.num_kv_heads;
  if (r != 1 && r != 2 && r != 4 && r != 8)
    return set_error(PSA_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads must be 1, 2, 4 or 8");
  if (c.head_dim != 64 && c.head_dim != 128) return set_error(PSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c.page_size != 16) return set_error(PSA_ERR_UNSUPPORTED, "page_size must be 16");
  if (c.num_pages <= 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "num_pages must be positive");
  if ((c.kv_dtype != PSA_BF16 && c.kv_dtype != PSA_F32) || (c.out_dtype != PSA_BF16 && c.out_dtype != PSA_F32))
    return set_error(PSA_ERR_UNSUPPORTED, "dtypes must be PSA_BF16 or PSA_F32");
  if (!(std::isfinite(c.sm_scale))) return set_error(PSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");

  psa_plan_opts o{};
  if (opts_in) o = *opts_in;
  const uint32_t known = PSA_PLAN_PREFIX_ONLY | PSA_PLAN_DISTINCT_ONLY | PSA_PLAN_FORCE_MATVEC |
                         PSA_PLAN_DEBUG_POISON | PSA_PLAN_NO_XCD_ORDER | PSA_PLAN_NO_TILE_PAIRS |
                         PSA_PLAN_NO_PAGE_SHARING;
  if (o.flags & ~known) return set_error(PSA_ERR_INVALID_ARGUMENT, "unknown plan flag");
  if ((o.flags & PSA_PLAN_PREFIX_ONLY) && (o.flags & PSA_PLAN_DISTINCT_ONLY))
    return set_error(PSA_ERR_INVALID_ARGUMENT, "PREFIX_ONLY and DISTINCT_ONLY are exclusive");
  if (o.prefix_chunk_tokens == 0) o.prefix_chunk_tokens = 2048;
  if (o.distinct_chunk_tokens == 0) o.distinct_chunk_tokens = 1024;
  if (o.mfma_min_rows == 0) o.mfma_min_rows = 16;
  if (o.mfma_tile_rows == 0) o.mfma_tile_rows = 128;
  if (o.prefix_chunk_tokens < 0 || o.prefix_chunk_tokens % c.page_size || o.distinct_chunk_tokens < 0 ||
      o.distinct_chunk_tokens % c.page_size)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "chunk sizes must be positive multiples of page_size");
  if (o.prefix_chunk_tokens > kMaxPrefixChunk || o.distinct_chunk_tokens > kMaxMatvecPages * 16)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "chunk sizes are limited to 2048 (prefix) and 1024 (distinct) tokens");
  if (o.mfma_min_rows < 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "mfma_min_rows must be >= 0");
  if (o.mfma_tile_rows < 16 || o.mfma_tile_rows > 128 || o.mfma_tile_rows % 16)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "mfma_tile_rows must be a multiple of 16 in [16, 128]");
  const bool use_prefix = !(o.flags & PSA_PLAN_DISTINCT_ONLY);
  const bool use_distinct = !(o.flags & PSA_PLAN_PREFIX_ONLY);
  const bool restricted = (o.flags & (PSA_PLAN_PREFIX_ONLY | PSA_PLAN_DISTINCT_ONLY)) != 0;

  const int G = b->num_groups, N = b->num_queries;
  if (G < 0 || N < 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "negative group or query count");
  if (G > 0 && (!b->group_prefix_len || !b->group_page_off))
    return set_error(PSA_ERR_INVALID_ARGUMENT, "group arrays are NULL");
  if (N > 0 && (!b->query_group || !b->query_distinct_len || !b->query_page_off))
    return set_error(PSA_ERR_INVALID_ARGUMENT, "query arrays are NULL");
  if (G > 0 && b->group_page_off[0] != 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "group_page_off[0] != 0");
  if (N > 0 && b->query_page_off[0] != 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "query_page_off[0] != 0");
  const int64_t n_gpages = G > 0 ? b->group_page_off[G] : 0;
  const int64_t n_qpages = N > 0 ? b->query_page_off[N] : 0;
  if (n_gpages > 0 && !b->group_pages) return set_error(PSA_ERR_INVALID_ARGUMENT, "group_pages is NULL");
  if (n_qpages > 0 && !b->query_pages) return set_error(PSA_ERR_INVALID_ARGUMENT, "query_pages is NULL");
  if (n_gpages + n_qpages > INT32_MAX)
    return set_error(PSA_ERR_UNSUPPORTED, "page tables longer than 2^31 entries");
  for (int g = 0; g < G; ++g) {
    psa_status s = check_segment("group", g, b->group_prefix_len[g], b->group_page_off[g], b->group_page_off[g + 1],
                                 b->group_pages, c.page_size, c.num_pages);
    if (s != PSA_OK) return s;
  }
  for (int i = 0; i < N; ++i) {
    const int g = b->query_group[i];
    if (g < -1 || g >= G)
      return set_error(PSA_ERR_INVALID_ARGUMENT, "query " + std::to_string(i) + ": group id out of range");
    psa_status s = check_segment("query", i, b->query_distinct_len[i], b->query_page_off[i], b->query_page_off[i + 1],
                                 b->query_pages, c.page_size, c.num_pages);
    if (s != PSA_OK) return s;
    int64_t lp = g >= 0 ? b->group_prefix_len[g] : 0;
    if (b->query_prefix_len && g >= 0) {
      const int64_t v = b->query_prefix_len[i];
      if (v < 0 || v > lp)
        return set_error(PSA_ERR_INVALID_ARGUMENT,
                         "query " + std::to_string(i) + ": query_prefix_len outside [0, group prefix_len]");
      lp = v;
    }
    if (lp + b->query_distinct_len[i] == 0 && !restricted)
      return set_error(PSA_ERR_INVALID_ARGUMENT, "query " + std::to_string(i) + ": empty context");
  }
  // prefix tokens each query sees (the whole group prefix unless limited)
  auto visible = [&](int i) -> int64_t {
    const int g = b->query_group[i];
    if (g < 0) return 0;
    return b->query_prefix_len ? (int64_t)b->query_prefix_len[i] : (int64_t)b->group_prefix_len[g];
  };
  const bool limited = b->query_prefix_len != nullptr && N > 0;

  auto* plan = new (std::nothrow) psa_plan();
  if (!plan) return set_error(PSA_ERR_ALLOC, "out of memory");
  plan->cfg = c;
  plan->opts = o;
  plan->r = r;
  plan->sm_scale = c.sm_scale > 0 ? c.sm_scale : 1.0f / std::sqrt((float)c.head_dim);
  const int hkv = c.num_kv_heads, d = c.head_dim, P = c.page_size;
  const bool bf16 = c.kv_dtype == PSA_BF16;
  const int e = bf16 ? 2 : 4;

  // Sharing of leading prefix pages between groups (BatchLLM summary §4.2:
  // flattening a multi-level tree gives every group its own copy of the
  // pages above it).  Groups whose prefixes begin with the same page ids are
  // made adjacent in the member array (groups sorted by their leading page
  // ids), so that every set of groups sharing leading pages is one
  // contiguous run of MFMA rows, whatever their numbering.
  const bool sharing = use_prefix && bf16 && !limited && !(o.flags & (PSA_PLAN_FORCE_MATVEC | PSA_PLAN_NO_PAGE_SHARING));
  std::vector<int32_t> nmem(G, 0), gorder(G);
  for (int i = 0; i < N; ++i)
    if (b->query_group[i] >= 0) ++nmem[b->query_group[i]];
  std::iota(gorder.begin(), gorder.end(), 0);
  auto whole_pages = [&](int g) { return (int64_t)b->group_prefix_len[g] / P; };
  auto gpages = [&](int g) { return b->group_pages + b->group_page_off[g]; };
  if (sharing)
    std::stable_sort(gorder.begin(), gorder.end(), [&](int x, int y) {
      const int64_t nx = whole_pages(x), ny = whole_pages(y), n = std::min(nx, ny);
      const int32_t *px = gpages(x), *py = gpages(y);
      for (int64_t k = 0; k < n; ++k)
        if (px[k] != py[k]) return px[k] < py[k];
      return nx < ny;
    });
  // members of each group, in query order, groups in gorder (rows of the MFMA tile)
  std::vector<int32_t> mstart(G, 0), members;
  {
    int64_t cur = 0;
    for (int g : gorder) {
      mstart[g] = (int32_t)cur;
      cur += nmem[g];
    }
    members.resize((size_t)cur);
    std::vector<int32_t> fill(mstart);
    for (int i = 0; i < N; ++i)
      if (b->query_group[i] >= 0) members[fill[b->query_group[i]]++] = i;
  }
  auto mend = [&](int g) { return mstart[g] + nmem[g]; };

  // prefix tiling per group: MFMA tiles (bf16, enough rows) take chunks of
  // up to prefix_chunk_tokens; small groups fall back to per-query mat-vec
  // tiles whose chunks hold at most kMaxMatvecPages pages
  const int64_t Cp = o.prefix_chunk_tokens, Cd = o.distinct_chunk_tokens;
  std::vector<char> group_mfma(G, 0);
  std::vector<int64_t> group_chunk(G, Cp);
  for (int g = 0; g < G; ++g) {
    const int64_t rows = (int64_t)nmem[g] * r;
    group_mfma[g] = bf16 && !(o.flags & PSA_PLAN_FORCE_MATVEC) && rows >= o.mfma_min_rows;
    if (!group_mfma[g]) group_chunk[g] = std::min<int64_t>(Cp, kMaxMatvecPages * 16);
  }
  // Shared nodes: over the groups with members, in gorder, the common
  // leading whole pages of neighbours (lcp) define a tree of intervals (the
  // LCP-interval tree): the groups of an interval all begin with its shared
  // length L of tokens.  A node covers the tokens [A, L) its groups share
  // beyond its nearest covering ancestor (A), once, with MFMA tiles whose
  // rows span all of its groups' members; a node is kept only if it adds at
  // least one 64-token block and has enough rows for MFMA tiles (otherwise
  // its children cover those tokens).  Each group then covers its own
  // tokens [A_g, Lp) as before, A_g being the level of its deepest node.
  // Partial indices of a query: its nodes' chunks root first, then its
  // group's own chunks, then its distinct chunks.
  struct Node {
    int lo, hi;      // range of seq (groups with members, in gorder)
    int64_t A, L;    // tokens [A, L), whole pages
    int64_t j0;      // partial index of its first chunk
  };
  std::vector<Node> nodes;
  std::vector<int64_t> own_from(G, 0), own_j0(G, 0);
  constexpr int64_t kMinShared = 64;  // at least one 64-token MFMA block
  if (sharing) {
    std::vector<int32_t> seq;
    for (int g : gorder)
      if (nmem[g] > 0) seq.push_back(g);
    const int n = (int)seq.size();
    std::vector<int64_t> lcp(n, 0);  // lcp[k]: leading whole pages (in tokens) seq[k-1] and seq[k] share
    for (int k = 1; k < n; ++k) {
      const int64_t m = std::min(whole_pages(seq[k - 1]), whole_pages(seq[k]));
      const int32_t *pa = gpages(seq[k - 1]), *pb = gpages(seq[k]);
      int64_t t = 0;
      while (t < m && pa[t] == pb[t]) ++t;
      lcp[k] = t * P;
    }
    struct Range {
      int lo, hi;
      int64_t A, j0;
    };
    std::vector<Range> todo{{0, n - 1, 0, 0}};
    while (!todo.empty() && n > 0) {
      const Range R = todo.back();
      todo.pop_back();
      if (R.lo == R.hi) {
        own_from[seq[R.lo]] = R.A;
        own_j0[seq[R.lo]] = R.j0;
        continue;
      }
      int64_t m = lcp[R.lo + 1];
      for (int k = R.lo + 2; k <= R.hi; ++k) m = std::min(m, lcp[k]);
      const int64_t rows = (int64_t)(mend(seq[R.hi]) - mstart[seq[R.lo]]) * r;
      int64_t A = R.A, j0 = R.j0;
      if (m - R.A >= kMinShared && rows >= o.mfma_min_rows) {
        nodes.push_back({R.lo, R.hi, R.A, m, R.j0});
        A = m;
        j0 = R.j0 + ceil_div(m - R.A, Cp);
      }
      int start = R.lo;
      for (int k = R.lo + 1; k <= R.hi; ++k)
        if (lcp[k] == m) {
          todo.push_back({start, k - 1, A, j0});
          start = k;
        }
      todo.push_back({start, R.hi, A, j0});
    }
    // node tiles read the pages of the run's first group (every group of the run holds them)
    for (Node& nd : nodes) nd.lo = seq[nd.lo], nd.hi = seq[nd.hi];
  }

  // partial counts per query: prefix chunks first (shared ones, then the
  // group's own), then distinct chunks
  std::vector<int32_t> n_pc(N, 0), expected(N, 0), slot_off(N, -1);
  int64_t slots = 0;
  for (int i = 0; i < N; ++i) {
    const int g = b->query_group[i];
    const int64_t lp = visible(i);  // (families form only without limits: lp is the whole prefix there)
    n_pc[i] = use_prefix && g >= 0 ? (int32_t)(own_j0[g] + ceil_div(lp - own_from[g], group_chunk[g])) : 0;
    const int64_t n_dc = use_distinct ? ceil_div(b->query_distinct_len[i], Cd) : 0;
    expected[i] = n_pc[i] + (int32_t)n_dc;
    if (expected[i] >= 2) {
      slot_off[i] = (int32_t)slots;
      slots += expected[i];
    }
  }
  if (slots * hkv > INT32_MAX) {
    delete plan;
    return set_error(PSA_ERR_UNSUPPORTED, "too many partial slots");
  }

  // ---- work items with a cost estimate (arbitrary time units) ----
  // MFMA tiles fill a whole workgroup; mat-vec and empty items are wave-level
  // and are packed four to a workgroup (unit).
  struct Cand {
    WorkItem it;
    double cost;
    bool shared = false;  // MFMA tile of a shared node
  };
  std::vector<Cand> mfma, waves;
  std::vector<int64_t> mfma_set;
  const double bw_wave = 8.0e3 / 2048.0;          // bytes per ns per resident wave (HBM share)
  const double mfma_slot = 2.5e6 / 512.0 * 0.5;   // flop per ns per workgroup slot at half rate
  const double fixed = 300.0;                     // per-item overhead, ns
  int64_t n_prefix_items = 0, n_matvec_items = 0;
  const int64_t tile_max = o.mfma_tile_rows;
  int64_t next_set_id = 0;  // one id per (prefix chunk, kv head): its tiles re-read the same pages
  // MFMA tiles over rows [row0, row0 + rows) of the member array (a = first
  // row counted over the whole member array, so a tile finds its queries
  // without reading a group offset first) for tokens [tb, te) of group g's
  // pages; j = the chunk's partial index for every query of those rows
  auto mfma_tiles = [&](int g, int64_t row0, int64_t rows, int32_t tb, int32_t te_chunk, int64_t j, bool shared) {
    const int32_t pbase = (int32_t)(b->group_page_off[g] + tb / P);
    const int64_t ntiles = ceil_div(rows, tile_max);
    const int64_t per = round_up(ceil_div(rows, ntiles), 16);
    for (int kvh = 0; kvh < hkv; ++kvh) {
      const int64_t set = next_set_id++;
      for (int64_t rb = 0; rb < rows; rb += per) {
        const int64_t rc = std::min(per, rows - rb);
        int32_t te = te_chunk;
        if (limited) {  // no tile for rows that all stop before this chunk; none past their last limit
          int64_t vmax = 0;
          for (int64_t m = (row0 + rb) / r; m <= (row0 + rb + rc - 1) / r; ++m)
            vmax = std::max(vmax, visible(members[m]));
          if (vmax <= tb) continue;
          te = (int32_t)std::min<int64_t>(te, vmax);
        }
        const double kv_bytes = (double)round_up(te - tb, P) * d * e * 2;
        WorkItem it{(int32_t)(ITEM_PREFIX_MFMA | (j << 8)), kvh, g, tb, te, pbase, (int32_t)(row0 + rb), (int32_t)rc};
        const double fl = (double)round_up(te - tb, 64) * round_up(rc, 16) * d * 4;
        mfma.push_back({it, fixed + std::max(fl / mfma_slot, 4.0 * kv_bytes / bw_wave), shared});
        mfma_set.push_back(set);
        ++n_prefix_items;
      }
    }
  };
  for (const Node& nd : nodes) {  // shared nodes: tokens [A, L) of every group of the run, once
    const int64_t rows = (int64_t)(mend(nd.hi) - mstart[nd.lo]) * r;
    for (int64_t ch = 0; ch < ceil_div(nd.L - nd.A, Cp); ++ch)
      mfma_tiles(nd.lo, (int64_t)mstart[nd.lo] * r, rows, (int32_t)(nd.A + ch * Cp),
                 (int32_t)std::min(nd.L, nd.A + (ch + 1) * Cp), nd.j0 + ch, true);
  }
  for (int g = 0; g < G && use_prefix; ++g) {  // each group's own tokens
    int64_t lp = b->group_prefix_len[g];
    const int nm = nmem[g];
    if (limited) {  // tokens past every member's limit need no tiles
      int64_t vmax = 0;
      for (int t = mstart[g]; t < mend(g); ++t) vmax = std::max(vmax, visible(members[t]));
      lp = vmax;
    }
    const int64_t S = own_from[g], j0 = own_j0[g];
    if (lp <= S || nm == 0) continue;
    const int64_t rows = (int64_t)nm * r;
    const bool mf = group_mfma[g];
    const int64_t C = group_chunk[g];
    const int64_t nchunks = ceil_div(lp - S, C);
    for (int64_t ch = 0; ch < nchunks; ++ch) {
      const int32_t tb = (int32_t)(S + ch * C), te = (int32_t)std::min(lp, S + (ch + 1) * C);
      const int64_t j = j0 + ch;
      if (mf) {
        mfma_tiles(g, (int64_t)mstart[g] * r, rows, tb, te, j, false);
      } else {
        const int32_t pbase = (int32_t)(b->group_page_off[g] + tb / P);
        const double kv_bytes = (double)round_up(te - tb, P) * d * e * 2;
        for (int t = mstart[g]; t < mend(g); ++t) {
          const int qi = members[t];
          const int64_t vis = visible(qi);
          if (vis <= tb) continue;  // this query's prefix ends before the chunk
          const int32_t tq = (int32_t)std::min<int64_t>(te, vis);
          for (int kvh = 0; kvh < hkv; ++kvh) {
            const int32_t slot = expected[qi] >= 2 ? (int32_t)(((int64_t)slot_off[qi] + j) * hkv + kvh) : -1;
            WorkItem it{ITEM_MATVEC, kvh, qi, tb, tq, pbase, expected[qi], slot};
            waves.push_back({it, fixed + kv_bytes / bw_wave});
            ++n_matvec_items;
          }
        }
      }
    }
  }
  for (int i = 0; i < N && use_distinct; ++i) {
    const int64_t ld = b->query_distinct_len[i];
    const int64_t nchunks = ceil_div(ld, Cd);
    for (int64_t ch = 0; ch < nchunks; ++ch) {
      const int32_t tb = (int32_t)(ch * Cd), te = (int32_t)std::min(ld, (ch + 1) * Cd);
      const int32_t pbase = (int32_t)(n_gpages + b->query_page_off[i] + tb / P);
      const double kv_bytes = (double)round_up(te - tb, P) * d * e * 2;
      for (int kvh = 0; kvh < hkv; ++kvh) {
        const int32_t slot =
            expected[i] >= 2 ? (int32_t)(((int64_t)slot_off[i] + n_pc[i] + ch) * hkv + kvh) : -1;
        WorkItem it{ITEM_MATVEC, kvh, i, tb, te, pbase, expected[i], slot};
        waves.push_back({it, fixed + kv_bytes / bw_wave});
        ++n_matvec_items;
      }
    }
  }
  for (int i = 0; i < N; ++i) {
    if (expected[i] == 0) {  // only under PREFIX_ONLY / DISTINCT_ONLY
      WorkItem it{ITEM_EMPTY, 0, i, 0, 0, 0, 0, -1};
      waves.push_back({it, 1.0});
    }
  }

  // ---- units: one MFMA tile, or four wave items of similar cost ----
  struct Unit {
    WorkItem it[kUnitItems];
    double cost;
    int64_t set;  // units of one set re-read one prefix chunk: same XCD
    bool shared;  // an MFMA tile of a shared node
  };
  std::vector<Unit> units;
  const WorkItem nop{ITEM_NOP, 0, 0, 0, 0, 0, 0, -1};
  for (size_t t = 0; t < mfma.size(); ++t) {
    Unit u{{mfma[t].it, nop, nop, nop}, mfma[t].cost, mfma_set[t], mfma[t].shared};
    units.push_back(u);
  }
  std::stable_sort(waves.begin(), waves.end(), [](const Cand& a, const Cand& b2) { return a.cost > b2.cost; });
  int64_t next_set = (int64_t)mfma.size() + 1 + (mfma_set.empty() ? 0 : *std::max_element(mfma_set.begin(), mfma_set.end()));
  for (size_t t = 0; t < waves.size(); t += kUnitItems) {
    Unit u{{nop, nop, nop, nop}, 0.0, next_set++, false};
    for (int w = 0; w < kUnitItems && t + w < waves.size(); ++w) {
      u.it[w] = waves[t + w].it;
      u.cost = std::max(u.cost, waves[t + w].cost);
    }
    units.push_back(u);
  }

  // ---- ordering: longest first; sets spread over 8 XCD queues (workgroup
  // i runs on XCD i % 8), so tiles re-reading one prefix chunk share an L2 ----
  std::vector<Unit> ordered;
  ordered.reserve(units.size());
  if (o.flags & PSA_PLAN_NO_XCD_ORDER) {
    std::stable_sort(units.begin(), units.end(), [](const Unit& a, const Unit& b2) { return a.cost > b2.cost; });
    ordered = units;
  } else {
    std::vector<int64_t> order(units.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b2) {
      if (units[a].set != units[b2].set) return units[a].set < units[b2].set;
      return a < b2;
    });
    struct Set {
      int64_t begin, end;
      double cost;
    };
    std::vector<Set> sets;
    for (size_t t = 0; t < order.size();) {
      size_t u = t;
      double cs = 0;
      while (u < order.size() && units[order[u]].set == units[order[t]].set) cs += units[order[u++]].cost;
      sets.push_back({(int64_t)t, (int64_t)u, cs});
      t = u;
    }
    std::stable_sort(sets.begin(), sets.end(), [](const Set& a, const Set& b2) { return a.cost > b2.cost; });
    constexpr int kXcd = 8;
    std::vector<std::vector<int64_t>> q(kXcd);
    double load[kXcd] = {0};
    for (const Set& s : sets) {
      int best = 0;
      for (int x = 1; x < kXcd; ++x)
        if (load[x] < load[best]) best = x;
      for (int64_t t = s.begin; t < s.end; ++t) q[best].push_back(order[t]);
      load[best] += s.cost;
    }
    // Longest first.  A queue of MFMA tiles alone (a PREFIX_ONLY plan) puts
    // family tiles first instead: they pair with the groups' own, longer
    // tiles on the CUs (flattened 4x16x16 prefix-only: 0.126 ms against
    // 0.140 ms longest first).
    auto family = [&](int64_t u) { return units[u].shared; };
    for (auto& qq : q) {
      const bool tiles_only = std::all_of(qq.begin(), qq.end(), [&](int64_t u) {
        return units[u].it[0].kind % 256 == ITEM_PREFIX_MFMA;
      });
      std::stable_sort(qq.begin(), qq.end(), [&](int64_t a, int64_t b2) {
        if (tiles_only && family(a) != family(b2)) return family(a);
        return units[a].cost > units[b2].cost;
      });
    }
    // Tile pairs: when the launch starts, an XCD's units k and k + 32 land on
    // the same compute unit (its 32 CUs are filled in one fixed order, twice:
    // two workgroups fit per CU).  Placing an XCD's first MFMA tiles at
    // positions [0, h) and [32, 32 + h') starts them two to a CU: no mat-vec
    // unit shares those CUs' load path with the tiles' copies, and the tiles'
    // two waves per SIMD hide each other's latencies.
    constexpr int kCusPerXcd = 32;
    std::vector<int32_t> set_size(next_set + 1, 0);  // units per set (an MFMA set: row tiles of one chunk)
    for (const Unit& u : units) ++set_size[u.set];
    if (!(o.flags & PSA_PLAN_NO_TILE_PAIRS)) {
      for (auto& qq : q) {
        size_t np = 0;
        while (np < qq.size() && units[qq[np]].it[0].kind % 256 == ITEM_PREFIX_MFMA) ++np;
        if (np > 2 * (size_t)kCusPerXcd - 8 && qq.size() > np) {
          // Pairs would leave fewer than 4 of the XCD's CUs to the mat-vec
          // units at the start (16 groups of 8x100, 64 tiles an XCD: 0.392
          // ms spread, 0.407 in pairs).  Tiles whose prefix chunk
          // has several row tiles read it from L2 and are bound by their
          // compute: spread evenly over the first 3/4 of the queue, they run
          // beside the HBM-bound mat-vec units instead of in a phase of
          // their own, and short mat-vec units end the launch (7 prefill
          // chunks + 256 decode queries: 0.149 ms, tiles first 0.162).
          // Tiles that are their chunk's only row tile stream it from HBM
          // themselves: when they are the majority, plain longest first
          // (flattened 4x16x16, two thirds of its tiles: 0.239 ms, spread
          // 0.244).
          size_t streaming = 0;
          for (size_t k = 0; k < np; ++k) streaming += set_size[units[qq[k]].set] == 1;
          if (2 * streaming > np) continue;
          const size_t n = qq.size();
          const size_t span = std::max(np, (size_t)(0.75 * (double)n));
          std::vector<int64_t> re;
          re.reserve(n);
          size_t mv = np, tk = 0;
          for (size_t pos = 0; pos < n; ++pos) {
            const bool tile = tk < np && (mv >= n || tk * span <= pos * np);
            re.push_back(tile ? qq[tk++] : qq[mv++]);
          }
          qq.swap(re);
          continue;
        }
        if (np < 2 || qq.size() < kCusPerXcd + np - (np + 1) / 2) continue;
        const size_t h = (np + 1) / 2;
        std::vector<int64_t> re;
        re.reserve(qq.size());
        size_t mv = np;  // next non-MFMA unit
        for (size_t k = 0; k < h; ++k) re.push_back(qq[k]);
        while (re.size() < (size_t)kCusPerXcd) re.push_back(qq[mv++]);
        for (size_t k = h; k < np; ++k) re.push_back(qq[k]);
        while (mv < qq.size()) re.push_back(qq[mv++]);
        qq.swap(re);
      }
    }
    size_t longest = 0;
    for (auto& qq : q) longest = std::max(longest, qq.size());
    for (size_t k = 0; k < longest; ++k)
      for (int x = 0; x < kXcd; ++x)
        if (k < q[x].size()) ordered.push_back(units[q[x][k]]);
  }
  if (ordered.size() > (size_t)INT32_MAX / kUnitItems) {
    delete plan;
    return set_error(PSA_ERR_UNSUPPORTED, "work list too long");
  }
  std::vector<WorkItem> items;
  items.reserve(ordered.size() * kUnitItems);
  for (const Unit& u : ordered)
    for (int w = 0; w < kUnitItems; ++w) items.push_back(u.it[w]);

  // ---- workspace image ----
  ImageLayout L{};
  int64_t off = 0;
  auto sect = [&](int64_t bytes) {
    int64_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.header = sect(8);
  L.items = sect((int64_t)items.size() * (int64_t)sizeof(WorkItem));
  L.pages = sect((n_gpages + n_qpages) * 4);
  L.member_off = sect((G + 1) * 4);
  L.members = sect((int64_t)members.size() * 4);
  L.expected = sect(N * 4);
  L.slot_off = sect(N * 4);
  L.qlim = limited ? sect(N * 4) : -1;
  L.counters = sect((int64_t)N * hkv * 4);
  L.meta_bytes = off;
  const int64_t part_o_bytes = slots * hkv * r * d * 4;
  const int64_t part_ml_bytes = slots * hkv * r * 2 * 4;
  if (part_o_bytes >= (int64_t)UINT32_MAX) {
    delete plan;
    return set_error(PSA_ERR_UNSUPPORTED, "partial results exceed 4 GiB; use larger chunks");
  }
  L.part_o = sect(part_o_bytes);
  L.part_ml = sect(part_ml_bytes);
  L.total_bytes = off;
  plan->layout = L;
  plan->part_o_bytes = (uint32_t)part_o_bytes;
  plan->part_ml_bytes = (uint32_t)part_ml_bytes;

  std::vector<uint8_t>& img = plan->image;
  try {
    img.assign((size_t)L.meta_bytes, 0);
  } catch (...) {
    delete plan;
    return set_error(PSA_ERR_ALLOC, "out of memory for the plan image");
  }
  auto put32 = [&](int64_t at, int64_t idx, int64_t v) {
    int32_t x = (int32_t)v;
    std::memcpy(img.data() + at + idx * 4, &x, 4);
  };
  plan->id = next_plan_id();
  const uint32_t header[2] = {kImageMagic, plan->id};
  std::memcpy(img.data() + L.header, header, sizeof(header));
  if (!items.empty()) std::memcpy(img.data() + L.items, items.data(), items.size() * sizeof(WorkItem));
  for (int64_t t = 0; t < n_gpages; ++t) put32(L.pages, t, b->group_pages[t]);
  for (int64_t t = 0; t < n_qpages; ++t) put32(L.pages, n_gpages + t, b->query_pages[t]);
  for (int g = 0; g < G; ++g) put32(L.member_off, g, mstart[g]);
  put32(L.member_off, G, (int64_t)members.size());
  for (size_t t = 0; t < members.size(); ++t) put32(L.members, t, members[t]);
  for (int i = 0; i < N; ++i) {
    put32(L.expected, i, expected[i]);
    put32(L.slot_off, i, slot_off[i]);
    if (limited) put32(L.qlim, i, visible(i));
  }
  // counters stay zero
  plan->num_units = (int64_t)ordered.size();
  plan->num_group_pages = n_gpages;

  // ---- statistics ----
  psa_plan_info& info = plan->info;
  info.workspace_bytes = (size_t)L.total_bytes;
  info.num_items = plan->num_units;
  info.num_prefix_items = n_prefix_items;
  info.num_matvec_items = n_matvec_items;
  info.num_partial_slots = slots * hkv;
  int64_t logical = 0, processed = 0, prefix_logical = 0;
  for (int g = 0; g < G; ++g)
    if (nmem[g] > 0) processed += b->group_prefix_len[g];
  for (int i = 0; i < N; ++i) {
    const int64_t lp = visible(i);
    logical += lp + b->query_distinct_len[i];
    prefix_logical += lp;
    processed += b->query_distinct_len[i];
  }
  info.logical_tokens = logical;
  info.processed_tokens = processed;
  info.saved_tokens = logical - processed;
  int64_t prefix_once = 0, distinct_tok = 0;
  for (int g = 0; g < G; ++g)
    if (nmem[g] > 0) prefix_once += b->group_prefix_len[g];
  for (int i = 0; i < N; ++i) distinct_tok += b->query_distinct_len[i];
  const double tok_bytes = (double)hkv * d * 2 * e;
  info.prefix_kv_bytes = (double)prefix_once * tok_bytes;
  info.distinct_kv_bytes = (double)distinct_tok * tok_bytes;
  info.algorithmic_bytes = info.prefix_kv_bytes + info.distinct_kv_bytes + (double)N * c.num_q_heads * d * e +
                           (double)N * c.num_q_heads * d * (c.out_dtype == PSA_BF16 ? 2 : 4);
  info.algorithmic_flops = 4.0 * d * c.num_q_heads * (double)logical;
  info.prefix_flops = 4.0 * d * c.num_q_heads * (double)prefix_logical;
  // KV tokens in distinct (page, slot) places: a page named by several groups'
  // prefixes (the shared root of a flattened tree) counts once, with the most
  // slots any of them uses.
  {
    std::vector<std::pair<int32_t, int32_t>> use;  // (page id, slots used)
    use.reserve((size_t)(n_gpages + n_qpages));
    auto mark = [&](const int32_t* pages, int64_t off, int64_t len) {
      for (int64_t t = 0; t < len; t += P) use.emplace_back(pages[off + t / P], (int32_t)std::min<int64_t>(P, len - t));
    };
    for (int g = 0; g < G; ++g) {
      int64_t vis = 0;
      for (int t = mstart[g]; t < mend(g); ++t) vis = std::max(vis, visible(members[t]));
      mark(b->group_pages, b->group_page_off[g], vis);
    }
    for (int i = 0; i < N; ++i) mark(b->query_pages, b->query_page_off[i], b->query_distinct_len[i]);
    std::sort(use.begin(), use.end());
    int64_t unique_tok = 0;
    for (size_t t = 0; t < use.size(); ++t)
      if (t + 1 == use.size() || use[t + 1].first != use[t].first) unique_tok += use[t].second;  // max per page
    info.unique_kv_bytes = (double)unique_tok * tok_bytes;
  }
  info.image_bytes = (size_t)L.meta_bytes;

  plan->members = members;
  plan->items = std::move(items);
  plan->expected = std::move(expected);
  plan->slot_off = std::move(slot_off);
  *out = plan;
  return PSA_OK;
}

}  // namespace psa
