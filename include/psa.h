/*
 * psa.h - prefix-shared decode attention on MI355X (gfx950), C ABI.
 *
 * What the library computes (BatchLLM summary, papercache.org, §2.2 Eq. 1 and
 * §5): every decode query of a prefix-sharing group attends once to the
 * group's shared-prefix KV and once to its own distinct KV; the two partial
 * results are merged by online softmax.  Prefix and distinct work run in ONE
 * horizontally fused kernel launch, in different workgroups with different
 * tilings (§5 "horizontal fusion of prefix-shared attention").  The KV cache is
 * paged: logically contiguous tokens live in scattered fixed-size pages named
 * by a block table (BatchLLM §2.2; continuous-batching post on guijiagi.com,
 * "block management").  Groups are single-level (BatchLLM §5: the input is a
 * list of (prefix, [distinct ...]) tuples); a multi-level prefix tree is first
 * flattened by dynamic programming (BatchLLM §4.2, Fig. 4) with
 * psa_flatten_prefix_tree.
 *
 * Result for query i, query head h (kv head kvh = h / (Hq/Hkv)):
 *   context = prefix tokens of group(i) (none if group(i) == -1) ++ distinct
 *             tokens of i;
 *   s_t = sm_scale * <q[i,h,:], K[t]>;  m = max_t s_t;  l = sum_t exp(s_t - m);
 *   out[i,h,:] = sum_t exp(s_t - m) V[t] / l.
 * out_m / out_l (optional) receive m (natural-log units) and l.
 *
 * Conventions.
 *   - Every function returns psa_status; nothing aborts or throws across the
 *     ABI.  On a non-OK status psa_last_error() returns a thread-local message.
 *   - "Device pointer" = memory allocated on the current HIP device (e.g. a
 *     torch tensor's data_ptr()); "host pointer" = ordinary CPU memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously; PSA_OK means "enqueued".
 *   - The library never allocates device memory.  The caller owns every device
 *     buffer, including the workspace.  The plan owns a pinned host staging
 *     buffer (allocated on first upload).
 *
 * Tensor layouts (contiguous, row-major, base pointers 16-byte aligned):
 *   q                [num_queries, num_q_heads, head_dim]        kv_dtype
 *   k_pool, v_pool   [num_pages, num_kv_heads, page_size, head_dim] kv_dtype
 *                    (token t of a segment sits in page pages[t / page_size],
 *                     slot t % page_size; a (page, kv head) tile is contiguous)
 *   out              [num_queries, num_q_heads, head_dim]        out_dtype
 *   out_m, out_l     [num_queries, num_q_heads]                  float32
 * Slots of a segment's last page past its length are never read: they may
 * hold anything, NaN and Inf included.
 */
#ifndef PSA_H
#define PSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSA_VERSION 1

typedef enum {
  PSA_OK = 0,
  PSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad CSR, Hq % Hkv != 0,
                                   negative length, empty context, ... */
  PSA_ERR_UNSUPPORTED = 2,      /* head_dim not in {64,128}, page_size != 16,
                                   Hq/Hkv not in {1,2,4,8}, unknown dtype */
  PSA_ERR_OUT_OF_RANGE = 3,     /* page id >= num_pages, length > pages * page_size */
  PSA_ERR_WORKSPACE_TOO_SMALL = 4,
  PSA_ERR_HIP = 5,              /* a HIP runtime call failed; message has its text */
  PSA_ERR_ALLOC = 6             /* host allocation failed */
} psa_status;

typedef enum { PSA_BF16 = 0, PSA_F32 = 1 } psa_dtype;

/* Model/cache shape.  sm_scale <= 0 selects 1/sqrt(head_dim) (the scale of
 * the continuous-batching post's "attention computation" section). */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;   /* 64 or 128 */
  int32_t page_size;  /* 16 */
  int32_t num_pages;  /* pages in each of k_pool / v_pool */
  int32_t kv_dtype;   /* psa_dtype of q, k_pool, v_pool */
  int32_t out_dtype;  /* psa_dtype of out (PSA_F32 recommended) */
  float sm_scale;
} psa_config;

/* Single-level prefix-sharing groups (BatchLLM §5: tuple(prefix, [distinct...]))
 * over paged KV.  Host pointers, borrowed for the duration of the call only.
 * CSR page tables: group g's prefix pages are
 * group_pages[group_page_off[g] .. group_page_off[g+1]), holding
 * group_prefix_len[g] tokens; likewise per query for its distinct part.
 * query_group[i] = -1: query i shares no prefix.  A query whose context is
 * empty (no prefix and distinct length 0) is rejected.
 *
 * query_prefix_len (may be NULL): query i sees only the first
 * query_prefix_len[i] tokens of its group's prefix (0 <= value <= the
 * group's prefix_len; ignored for queries without a group).  This is how a
 * chunk of prefill tokens shares one launch with decode queries (BatchLLM
 * §4.3 token batching, Fig. 10c): the chunk is a group whose prefix is the
 * request's context up to the chunk's end, each chunk token a query that
 * sees that context up to and including itself (causal), with no distinct
 * part.  NULL: every query sees its whole group prefix. */
typedef struct {
  int32_t num_groups;
  const int32_t* group_prefix_len;   /* [num_groups] */
  const int64_t* group_page_off;     /* [num_groups + 1], starts at 0, non-decreasing */
  const int32_t* group_pages;        /* [group_page_off[num_groups]] */
  int32_t num_queries;
  const int32_t* query_group;        /* [num_queries], -1 or a group id */
  const int32_t* query_distinct_len; /* [num_queries], may be 0 */
  const int64_t* query_page_off;     /* [num_queries + 1] */
  const int32_t* query_pages;        /* [query_page_off[num_queries]] */
  const int32_t* query_prefix_len;   /* [num_queries] or NULL (see above) */
} psa_batch;

/* Plan flags. */
#define PSA_PLAN_PREFIX_ONLY 0x1u   /* cover only prefix tokens: out = prefix partial */
#define PSA_PLAN_DISTINCT_ONLY 0x2u /* cover only distinct tokens: out = distinct partial */
#define PSA_PLAN_FORCE_MATVEC 0x4u  /* no MFMA prefix tiles: every range per query */
#define PSA_PLAN_DEBUG_POISON 0x8u  /* psa_plan_upload fills partial slots with NaN */
#define PSA_PLAN_NO_XCD_ORDER 0x10u /* plain longest-first order, no XCD grouping */
#define PSA_PLAN_NO_TILE_PAIRS 0x20u /* MFMA prefix tiles lead each XCD queue (no pairs, no spreading) */
#define PSA_PLAN_NO_PAGE_SHARING 0x40u /* no shared-page tiles: groups whose prefixes begin with the
                                          same pages each cover those pages themselves */

/* Plan options; pass NULL for defaults.  Zero fields take defaults. */
typedef struct {
  uint32_t flags;
  int32_t prefix_chunk_tokens;   /* KV-range chunk of prefix work (split-K); default 2048 */
  int32_t distinct_chunk_tokens; /* chunk of distinct work, <= 1024; default 1024 */
  int32_t mfma_min_rows;         /* group rows (members * Hq/Hkv) at or above which the
                                    prefix uses the MFMA tile; default 16 */
  int32_t mfma_tile_rows;        /* max rows per MFMA prefix tile, multiple of 16, <= 128;
                                    default 128 */
} psa_plan_opts;

/* Plan statistics (host side). */
typedef struct {
  size_t workspace_bytes;    /* device workspace psa_plan_upload/psa_decode_attention need */
  int64_t num_items;         /* workgroups of the fused launch */
  int64_t num_prefix_items;  /* MFMA prefix tiles */
  int64_t num_matvec_items;  /* mat-vec tiles (distinct ranges, small-group prefixes) */
  int64_t num_partial_slots; /* (query, kv head) partial results written to the workspace */
  int64_t logical_tokens;    /* sum over queries of attended tokens */
  int64_t processed_tokens;  /* prefix tokens once per group + distinct tokens */
  int64_t saved_tokens;      /* logical - processed (BatchLLM §3.2 Eq. 2 numerator) */
  double algorithmic_bytes;  /* KV read once per group/query + q + out (fp32 or bf16) */
  double algorithmic_flops;  /* 4 * head_dim * Hq per attended token */
  double prefix_flops;       /* part of algorithmic_flops on prefix tokens */
  double prefix_kv_bytes;    /* prefix KV bytes, once per group */
  double distinct_kv_bytes;  /* distinct KV bytes */
  size_t image_bytes;        /* leading part of the workspace that psa_plan_upload fills (the
                                plan image); what psa_decode_attention_noalloc needs */
  double unique_kv_bytes;    /* KV bytes over distinct (page, slot) places: a page named by several
                                groups' prefixes (e.g. the shared root of a flattened tree) once */
} psa_plan_info;

typedef struct psa_plan psa_plan;

/* Validate `batch` against `cfg`, split every KV range into chunks, classify
 * them into MFMA prefix tiles and mat-vec tiles, order the work list (longest
 * first, tiles sharing a prefix chunk on the same XCD) and lay out the
 * workspace.  Groups whose prefixes begin with the same page ids (whatever
 * their numbering; psa_flatten_prefix_tree produces such groups from the
 * nodes above them) share those pages: every run of groups with a common
 * leading part of at least 64 tokens beyond an enclosing run's covers it
 * once, with MFMA tiles over all the run's requests, nested to any depth,
 * unless PSA_PLAN_NO_PAGE_SHARING is set.  Host only; copies everything it
 * needs.  *out receives a new plan on PSA_OK (free with psa_destroy_plan). */
psa_status psa_build_plan(const psa_config* cfg, const psa_batch* batch,
                          const psa_plan_opts* opts, psa_plan** out);

psa_status psa_plan_get_info(const psa_plan* plan, psa_plan_info* info);

/* Copy the plan's work list and page tables into the device workspace
 * `d_workspace` on `stream`, and zero its merge counters.  The workspace must
 * hold info.workspace_bytes for psa_decode_attention, or at least
 * info.image_bytes for psa_decode_attention_noalloc.  Needed once per (plan, workspace) pair; afterwards the workspace
 * serves any number of psa_decode_attention calls of this plan (counters
 * reset themselves), until another plan is uploaded into it.  The image
 * begins with a header naming the plan (a process-unique id).  The plan must
 * stay alive until the copy has completed (synchronise the stream before
 * psa_destroy_plan). */
psa_status psa_plan_upload(psa_plan* plan, void* d_workspace, size_t workspace_bytes,
                           void* stream);

/* One fused launch of the decode step described by `plan` (BatchLLM §5).
 * d_q / d_k_pool / d_v_pool / d_out: device pointers, layouts above.
 * d_out_m, d_out_l: device pointers or NULL.  d_workspace: the workspace
 * uploaded for this plan.  Concurrent calls on one workspace race (the merge
 * counters live there); use one workspace per stream.
 * Errors: PSA_ERR_INVALID_ARGUMENT if `d_workspace` was never uploaded for
 * this plan on the current device, or another plan was uploaded into it
 * since.  The kernel also compares the image header with the plan before it
 * reads anything else from the workspace: if the memory was overwritten
 * outside the library (e.g. freed and reused), every element of out, out_m
 * and out_l is set to NaN instead.  (A workspace whose header survived but
 * whose body was overwritten is not detected: keep it owned while the plan
 * uses it.) */
psa_status psa_decode_attention(const psa_plan* plan, const void* d_q, const void* d_k_pool,
                                const void* d_v_pool, void* d_out, float* d_out_m,
                                float* d_out_l, void* d_workspace, size_t workspace_bytes,
                                void* stream);

/* psa_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc):
 * the same kernels, with their scratch (the merge counters and the fp32
 * partial results) in a static device array of the library, 64 MiB per GPU,
 * held until the process ends.  `d_image` is a buffer into which
 * psa_plan_upload copied this plan (>= info.image_bytes; the rest of the
 * workspace is not needed).  The call clears the counters with a fill kernel
 * and launches the decode on `stream`; it allocates nothing and calls no
 * allocating routine.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (different streams, or host threads) race.
 * Errors: PSA_ERR_WORKSPACE_TOO_SMALL if the plan needs more scratch than the
 * array holds (info.workspace_bytes - info.image_bytes > 64 MiB, e.g. very many
 * partial results; use psa_decode_attention with a workspace then) or
 * image_bytes < info.image_bytes; otherwise as psa_decode_attention. */
psa_status psa_decode_attention_noalloc(const psa_plan* plan, const void* d_q, const void* d_k_pool,
                                        const void* d_v_pool, void* d_out, float* d_out_m,
                                        float* d_out_l, const void* d_image, size_t image_bytes,
                                        void* stream);

/* Eq. 1's online_softmax merge of two partial results, elementwise over `rows`
 * rows of `head_dim` (a power of two in [4, 256]):
 *   m = max(m_a, m_b); w_x = l_x * exp(m_x - m); l = w_a + w_b;
 *   o = (w_a o_a + w_b o_b) / l.
 * Partials carry o normalised by their own l, m in natural-log units; the
 * empty partial (o = 0, m = -inf, l = 0) is the identity.  All device
 * pointers, fp32 (o_a, o_b, o 16-byte aligned); outputs may alias the `a`
 * inputs.  PSA_ERR_UNSUPPORTED for another head_dim. */
psa_status psa_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* m_a,
                     const float* l_a, const float* o_b, const float* m_b, const float* l_b,
                     float* o, float* m, float* l, void* stream);

/* Multi-level input: a compact prefix tree over page-aligned KV segments
 * (BatchLLM §4.2, Fig. 4).  Node d holds node_len[d] tokens in pages
 * node_pages[node_page_off[d] .. node_page_off[d+1]); node_parent[d] = -1 for
 * a child of the (empty) root.  Query i shares the whole path root..query_node[i]
 * (-1 = nothing) and owns query_distinct_len[i] further tokens.  Host pointers. */
typedef struct {
  int32_t num_nodes;
  const int32_t* node_parent;   /* [num_nodes], parent id < own id not required */
  const int32_t* node_len;      /* [num_nodes], multiple of page_size, > 0 */
  const int64_t* node_page_off; /* [num_nodes + 1] */
  const int32_t* node_pages;
  int32_t num_queries;
  const int32_t* query_node;         /* [num_queries] */
  const int32_t* query_distinct_len; /* [num_queries] */
  const int64_t* query_page_off;     /* [num_queries + 1] */
  const int32_t* query_pages;
} psa_tree;

typedef struct psa_batch_owned psa_batch_owned;

/* Flatten `tree` to single-level groups maximising first-level token reuse,
 * sum over groups of prefix_len * (members - 1) (BatchLLM §4.2).  Each group is
 * a tree node's root-to-node path; nodes below it are unfolded into the
 * members' distinct parts.  Groups are numbered by node id, queries keep their
 * order.  *out receives a library-owned batch (free with psa_free_batch). */
psa_status psa_flatten_prefix_tree(const psa_tree* tree, int32_t page_size,
                                   psa_batch_owned** out);

/* View of a flattened batch (pointers stay valid until psa_free_batch) and
 * the saved-token count of its grouping. */
psa_status psa_batch_owned_view(const psa_batch_owned* owned, psa_batch* view,
                                int64_t* saved_tokens);

void psa_free_batch(psa_batch_owned* owned);
void psa_destroy_plan(psa_plan* plan);

/* Prefix identification from token ids (BatchLLM summary §4.2, and its
 * prefix-identification step of §5: nested input ids in, prefix-sharing
 * groups out).  Request i is tokens[token_off[i] .. token_off[i+1]) (host
 * arrays, borrowed for the call; token_off has num_requests + 1 entries,
 * starts at 0, non-decreasing).  The requests' compact prefix tree is built
 * from their lexicographic order and the common prefix lengths of neighbours,
 * and the dynamic program of psa_flatten_prefix_tree picks the groups that
 * maximise sum over groups of prefix_len * (members - 1).  A group's members
 * share their first prefix_len tokens (token-granular: the caller computes
 * that KV once and each member's distinct part starts at token prefix_len in
 * pages of its own).  Groups are numbered in the order of their first member.
 * *out receives a library-owned result (free with psa_free_prefix_groups).
 * Errors: NULL arrays, offsets not starting at 0 or decreasing
 * (PSA_ERR_INVALID_ARGUMENT); a request longer than 2^31 tokens
 * (PSA_ERR_UNSUPPORTED); PSA_ERR_ALLOC. */
typedef struct psa_prefix_groups psa_prefix_groups;
psa_status psa_identify_prefix_groups(int32_t num_requests, const int64_t* token_off,
                                      const int32_t* tokens, psa_prefix_groups** out);

/* View of a result (pointers stay valid until psa_free_prefix_groups; any
 * output pointer may be NULL): group_prefix_len[num_groups],
 * group_first_request[num_groups] (a member whose first prefix_len tokens
 * are the group's prefix), request_group[num_requests] (-1 = no group), and
 * the saved-token count of the grouping. */
psa_status psa_prefix_groups_view(const psa_prefix_groups* groups, int32_t* num_groups,
                                  const int32_t** group_prefix_len,
                                  const int32_t** group_first_request,
                                  const int32_t** request_group, int64_t* saved_tokens);

void psa_free_prefix_groups(psa_prefix_groups* groups);

/* Thread-local text of the last non-OK status ("" if none). */
const char* psa_last_error(void);

int32_t psa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PSA_H */
