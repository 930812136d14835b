// C ABI of the prefix-shared decode attention library (declared in psa.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>
#include <cstring>
#include <new>
#include <string>

#include "plan.h"
#include "psa_internal.h"

namespace psa {

hipError_t launch_decode(const DecodeParams& p, int head_dim, int r, bool bf16, hipStream_t s);
hipError_t launch_read_peak(const void* buf, uint32_t bytes, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_mfma_peak(float* out, int iters, int blocks, hipStream_t s);
hipError_t launch_issue_probe(int pattern, int64_t* cycles, int iters, int blocks, hipStream_t s);
hipError_t launch_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* m_a, const float* l_a,
                        const float* o_b, const float* m_b, const float* l_b, float* o, float* m, float* l,
                        hipStream_t s);
hipError_t launch_fill(uint32_t* dst, int64_t n, uint32_t value, hipStream_t s);

namespace {
thread_local std::string g_err;

psa_status hip_fail(hipError_t e, const char* what) {
  return set_error(PSA_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A device pointer of the current device (or managed memory); host pointers
// and pointers of another device are rejected before any kernel sees them.
psa_status check_device_ptr(const void* ptr, const char* name, int device) {
  if (!ptr) return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
  if (!aligned16(ptr)) return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(name) + " is not 16-byte aligned");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(name) + " is not device memory");
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(name) + " is not device memory");
  if (attr.device != device)
    return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(name) + " lives on another device");
  return PSA_OK;
}
}  // namespace

psa_status set_error(psa_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// Which plan's image each (workspace, device) holds: the last upload into it.
// A decode call must name that plan; an upload of another plan into the same
// workspace, or the destruction of the plan, invalidates the entry.  (The
// kernel checks the image header as well, which also catches a workspace
// overwritten outside the library.)
namespace {
struct Upload {
  uintptr_t ws;
  int dev;
  uint32_t plan_id;
};
std::mutex g_uploads_mu;
std::vector<Upload> g_uploads;

void record_upload(uintptr_t ws, int dev, uint32_t plan_id) {
  std::lock_guard<std::mutex> lk(g_uploads_mu);
  for (Upload& u : g_uploads)
    if (u.ws == ws && u.dev == dev) {
      u.plan_id = plan_id;
      return;
    }
  g_uploads.push_back({ws, dev, plan_id});
}

// 1: holds this plan's image; 0: never uploaded on this device; -1: holds another plan's image.
// dev < 0: on any device (1 if some device's copy holds this plan's image).
int upload_state(uintptr_t ws, int dev, uint32_t plan_id) {
  std::lock_guard<std::mutex> lk(g_uploads_mu);
  int state = 0;
  for (const Upload& u : g_uploads)
    if (u.ws == ws && (dev < 0 || u.dev == dev)) {
      if (u.plan_id == plan_id) return 1;
      state = -1;
    }
  return state;
}

void forget_plan(uint32_t plan_id) {
  std::lock_guard<std::mutex> lk(g_uploads_mu);
  g_uploads.erase(std::remove_if(g_uploads.begin(), g_uploads.end(),
                                 [&](const Upload& u) { return u.plan_id == plan_id; }),
                  g_uploads.end());
}
}  // namespace

}  // namespace psa

using psa::set_error;

constexpr int kPeakBlocks = 2048;  // workgroups of the peak kernels: 8 per CU, 4 waves each

extern "C" {

const char* psa_last_error(void) { return psa::g_err.c_str(); }

int32_t psa_version(void) { return PSA_VERSION; }

psa_status psa_build_plan(const psa_config* cfg, const psa_batch* batch, const psa_plan_opts* opts,
                          psa_plan** out) {
  try {
    return psa::build_plan(cfg, batch, opts, out);
  } catch (const std::bad_alloc&) {
    return set_error(PSA_ERR_ALLOC, "out of host memory");
  } catch (...) {
    return set_error(PSA_ERR_INVALID_ARGUMENT, "unexpected exception while planning");
  }
}

psa_status psa_plan_get_info(const psa_plan* plan, psa_plan_info* info) {
  if (!plan || !info) return set_error(PSA_ERR_INVALID_ARGUMENT, "plan or info is NULL");
  *info = plan->info;
  return PSA_OK;
}

psa_status psa_plan_upload(psa_plan* plan, void* d_workspace, size_t bytes, void* stream) {
  if (!plan) return set_error(PSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (bytes < (size_t)plan->layout.meta_bytes)
    return set_error(PSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs " + std::to_string(plan->layout.meta_bytes) +
                                                      " bytes for the plan image, got " + std::to_string(bytes));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
  psa_status s = psa::check_device_ptr(d_workspace, "workspace", dev);
  if (s != PSA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t meta = (size_t)plan->layout.meta_bytes;
  {
    std::lock_guard<std::mutex> lk(plan->mu);
    if (!plan->pinned && meta > 0) {
      e = hipHostMalloc(&plan->pinned, meta, hipHostMallocDefault);
      if (e != hipSuccess) {
        plan->pinned = nullptr;
        return psa::hip_fail(e, "hipHostMalloc");
      }
      std::memcpy(plan->pinned, plan->image.data(), meta);
    }
  }
  if (meta > 0) {
    e = hipMemcpyAsync(d_workspace, plan->pinned, meta, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return psa::hip_fail(e, "hipMemcpyAsync (plan upload)");
  }
  if (plan->opts.flags & PSA_PLAN_DEBUG_POISON) {
    const int64_t words = (plan->layout.total_bytes - plan->layout.part_o) / 4;
    e = psa::launch_fill(reinterpret_cast<uint32_t*>(static_cast<char*>(d_workspace) + plan->layout.part_o), words,
                         0x7fc00000u /* quiet NaN */, st);
    if (e != hipSuccess) return psa::hip_fail(e, "poison fill launch");
  }
  psa::record_upload(reinterpret_cast<uintptr_t>(d_workspace), dev, plan->id);
  return PSA_OK;
}

}  // extern "C"

namespace psa {
// The fused launch.  scratch == nullptr: counters and partials live in the
// workspace after the image (which then needs layout.total_bytes); otherwise
// they live at `scratch` (layout.total_bytes - layout.counters bytes, the
// caller checked the size), the workspace holds only the image, and the
// counters are cleared by a fill kernel first.
psa_status decode_impl(const psa_plan* plan, const void* d_q, const void* d_k_pool, const void* d_v_pool,
                       void* d_out, float* d_out_m, float* d_out_l, const void* d_workspace, size_t bytes,
                       uint64_t* d_trace, void* stream, char* scratch) {
  if (!plan) return set_error(PSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  const psa::ImageLayout& L = plan->layout;
  const int64_t need = scratch ? L.meta_bytes : L.total_bytes;
  if (bytes < (size_t)need)
    return set_error(PSA_ERR_WORKSPACE_TOO_SMALL,
                     std::string(scratch ? "plan image needs " : "workspace needs ") + std::to_string(need) +
                         " bytes, got " + std::to_string(bytes));
  if (psa::upload_state(reinterpret_cast<uintptr_t>(d_workspace), -1, plan->id) == 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "workspace was not uploaded for this plan (call psa_plan_upload)");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
  const int state = psa::upload_state(reinterpret_cast<uintptr_t>(d_workspace), dev, plan->id);
  if (state == 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT,
                     "workspace was not uploaded for this plan on this device (call psa_plan_upload)");
  if (state < 0)
    return set_error(PSA_ERR_INVALID_ARGUMENT,
                     "workspace holds another plan's upload (call psa_plan_upload for this plan)");
  if (plan->items.empty()) return PSA_OK;
  psa_status s;
  if ((s = psa::check_device_ptr(d_q, "q", dev)) != PSA_OK) return s;
  if ((s = psa::check_device_ptr(d_k_pool, "k_pool", dev)) != PSA_OK) return s;
  if ((s = psa::check_device_ptr(d_v_pool, "v_pool", dev)) != PSA_OK) return s;
  if ((s = psa::check_device_ptr(d_out, "out", dev)) != PSA_OK) return s;
  if (d_out_m && (s = psa::check_device_ptr(d_out_m, "out_m", dev)) != PSA_OK) return s;
  if (d_out_l && (s = psa::check_device_ptr(d_out_l, "out_l", dev)) != PSA_OK) return s;

  char* ws = static_cast<char*>(const_cast<void*>(d_workspace));
  psa::DecodeParams p{};
  p.header = reinterpret_cast<const uint32_t*>(ws + L.header);
  p.plan_id = plan->id;
  p.num_queries = (int32_t)plan->expected.size();
  p.q = d_q;
  p.k = d_k_pool;
  p.v = d_v_pool;
  p.out = d_out;
  p.out_m = d_out_m;
  p.out_l = d_out_l;
  p.items = reinterpret_cast<const psa::WorkItem*>(ws + L.items);
  p.pages = reinterpret_cast<const int32_t*>(ws + L.pages);
  p.member_off = reinterpret_cast<const int32_t*>(ws + L.member_off);
  p.members = reinterpret_cast<const int32_t*>(ws + L.members);
  p.expected = reinterpret_cast<const int32_t*>(ws + L.expected);
  p.slot_off = reinterpret_cast<const int32_t*>(ws + L.slot_off);
  p.qlim = L.qlim >= 0 ? reinterpret_cast<const int32_t*>(ws + L.qlim) : nullptr;
  // counters and partials: after the image in the workspace, or at the start of the scratch array
  // (same relative offsets, all 256-byte aligned)
  char* cbase = scratch ? scratch : ws + L.counters;
  p.counters = reinterpret_cast<int32_t*>(cbase);
  p.part_o = reinterpret_cast<float*>(cbase + (L.part_o - L.counters));
  p.part_ml = reinterpret_cast<float*>(cbase + (L.part_ml - L.counters));
  p.part_o_bytes = plan->part_o_bytes;
  p.part_ml_bytes = plan->part_ml_bytes;
  p.num_units = (int32_t)plan->num_units;
  p.hq = plan->cfg.num_q_heads;
  p.hkv = plan->cfg.num_kv_heads;
  p.scale_log2 = plan->sm_scale * 1.4426950408889634f;
  p.out_bf16 = plan->cfg.out_dtype == PSA_BF16;
  p.trace = d_trace;
  if (scratch) {  // the array keeps the last call's contents: counters must start at zero
    e = psa::launch_fill(reinterpret_cast<uint32_t*>(p.counters), (int64_t)p.num_queries * p.hkv, 0u,
                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return psa::hip_fail(e, "counter clear launch");
  }
  e = psa::launch_decode(p, plan->cfg.head_dim, plan->r, plan->cfg.kv_dtype == PSA_BF16,
                         reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa::hip_fail(e, "decode kernel launch");
  return PSA_OK;
}
}  // namespace psa

extern "C" {

psa_status psa_decode_attention(const psa_plan* plan, const void* d_q, const void* d_k_pool, const void* d_v_pool,
                                void* d_out, float* d_out_m, float* d_out_l, void* d_workspace, size_t bytes,
                                void* stream) {
  return psa::decode_impl(plan, d_q, d_k_pool, d_v_pool, d_out, d_out_m, d_out_l, d_workspace, bytes, nullptr, stream,
                           nullptr);
}

psa_status psa_decode_attention_traced(const psa_plan* plan, const void* d_q, const void* d_k_pool,
                                       const void* d_v_pool, void* d_out, float* d_out_m, float* d_out_l,
                                       void* d_workspace, size_t bytes, void* d_trace, int64_t trace_capacity,
                                       void* stream) {
  if (!plan) return set_error(PSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!d_trace) return set_error(PSA_ERR_INVALID_ARGUMENT, "trace is NULL");
  if (trace_capacity < plan->num_units * 4)
    return set_error(PSA_ERR_WORKSPACE_TOO_SMALL,
                     "trace needs " + std::to_string(plan->num_units * 4) + " uint64 entries");
  if (!plan->items.empty()) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
    psa_status s = psa::check_device_ptr(d_trace, "trace", dev);
    if (s != PSA_OK) return s;
  }
  return psa::decode_impl(plan, d_q, d_k_pool, d_v_pool, d_out, d_out_m, d_out_l, d_workspace, bytes,
                          static_cast<uint64_t*>(d_trace), stream, nullptr);
}

psa_status psa_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* m_a, const float* l_a,
                     const float* o_b, const float* m_b, const float* l_b, float* o, float* m, float* l,
                     void* stream) {
  if (rows < 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (head_dim < 4 || head_dim > 256 || (head_dim & (head_dim - 1)))
    return set_error(PSA_ERR_UNSUPPORTED, "psa_merge: head_dim must be a power of two in [4, 256]");
  if (rows == 0) return PSA_OK;
  const void* ptrs[] = {o_a, m_a, l_a, o_b, m_b, l_b, o, m, l};
  const char* names[] = {"o_a", "m_a", "l_a", "o_b", "m_b", "l_b", "o", "m", "l"};
  for (int t = 0; t < 9; ++t)
    if (!ptrs[t]) return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(names[t]) + " is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
  for (int t = 0; t < 9; ++t) {
    if (t == 0 || t == 3 || t == 6) {
      psa_status s = psa::check_device_ptr(ptrs[t], names[t], dev);
      if (s != PSA_OK) return s;
    } else {
      if (reinterpret_cast<uintptr_t>(ptrs[t]) & 3u)
        return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(names[t]) + " is not 4-byte aligned");
      hipPointerAttribute_t attr;
      if (hipPointerGetAttributes(&attr, ptrs[t]) != hipSuccess ||
          (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) || attr.device != dev) {
        (void)hipGetLastError();
        return set_error(PSA_ERR_INVALID_ARGUMENT, std::string(names[t]) + " is not device memory of this device");
      }
    }
  }
  e = psa::launch_merge(rows, head_dim, o_a, m_a, l_a, o_b, m_b, l_b, o, m, l, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa::hip_fail(e, "merge kernel launch");
  return PSA_OK;
}

psa_status psa_flatten_prefix_tree(const psa_tree* tree, int32_t page_size, psa_batch_owned** out) {
  try {
    return psa::flatten_tree(tree, page_size, out);
  } catch (const std::bad_alloc&) {
    return set_error(PSA_ERR_ALLOC, "out of host memory");
  }
}

psa_status psa_batch_owned_view(const psa_batch_owned* o, psa_batch* v, int64_t* saved_tokens) {
  if (!o || !v) return set_error(PSA_ERR_INVALID_ARGUMENT, "owned batch or view is NULL");
  v->num_groups = (int32_t)o->group_prefix_len.size();
  v->group_prefix_len = o->group_prefix_len.data();
  v->group_page_off = o->group_page_off.data();
  v->group_pages = o->group_pages.data();
  v->num_queries = (int32_t)o->query_group.size();
  v->query_group = o->query_group.data();
  v->query_distinct_len = o->query_distinct_len.data();
  v->query_page_off = o->query_page_off.data();
  v->query_pages = o->query_pages.data();
  v->query_prefix_len = nullptr;
  if (saved_tokens) *saved_tokens = o->saved_tokens;
  return PSA_OK;
}

void psa_free_batch(psa_batch_owned* o) { delete o; }

void psa_destroy_plan(psa_plan* plan) {
  if (!plan) return;
  psa::forget_plan(plan->id);
  if (plan->pinned) (void)hipHostFree(plan->pinned);
  delete plan;
}

// ---- debug helpers (psa_debug.h): expose the host copy of a plan ----
psa_status psa_plan_debug_items(const psa_plan* plan, int32_t* out, int64_t capacity_items) {
  if (!plan || (!out && capacity_items > 0)) return set_error(PSA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (capacity_items < (int64_t)plan->items.size())
    return set_error(PSA_ERR_INVALID_ARGUMENT, "capacity too small");
  std::memcpy(out, plan->items.data(), plan->items.size() * sizeof(psa::WorkItem));
  return PSA_OK;
}

psa_status psa_plan_debug_members(const psa_plan* plan, int32_t* out, int64_t capacity, int64_t* count) {
  if (!plan || !count) return set_error(PSA_ERR_INVALID_ARGUMENT, "NULL plan or count");
  *count = (int64_t)plan->members.size();
  if (capacity < *count) return set_error(PSA_ERR_INVALID_ARGUMENT, "capacity too small");
  if (*count > 0 && !out) return set_error(PSA_ERR_INVALID_ARGUMENT, "NULL output");
  if (*count > 0) std::memcpy(out, plan->members.data(), plan->members.size() * 4);
  return PSA_OK;
}

psa_status psa_plan_debug_queries(const psa_plan* plan, int32_t* expected, int32_t* slot_off, int64_t capacity) {
  if (!plan) return set_error(PSA_ERR_INVALID_ARGUMENT, "NULL plan");
  if (capacity < (int64_t)plan->expected.size()) return set_error(PSA_ERR_INVALID_ARGUMENT, "capacity too small");
  if (!plan->expected.empty() && (!expected || !slot_off)) return set_error(PSA_ERR_INVALID_ARGUMENT, "NULL output");
  std::memcpy(expected, plan->expected.data(), plan->expected.size() * 4);
  std::memcpy(slot_off, plan->slot_off.data(), plan->slot_off.size() * 4);
  return PSA_OK;
}

psa_status psa_debug_read_peak(const void* d_buf, size_t bytes, uint32_t* d_sink, int64_t sink_capacity,
                               void* stream) {
  if (!d_buf || !d_sink) return set_error(PSA_ERR_INVALID_ARGUMENT, "buffer or sink is NULL");
  if (bytes == 0 || bytes % 16 || bytes > (size_t)1 << 31)
    return set_error(PSA_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16, at most 2 GiB");
  if (sink_capacity < (int64_t)kPeakBlocks * 256)
    return set_error(PSA_ERR_WORKSPACE_TOO_SMALL, "sink needs " + std::to_string(kPeakBlocks * 256) + " entries");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
  psa_status st = psa::check_device_ptr(d_buf, "buffer", dev);
  if (st != PSA_OK) return st;
  st = psa::check_device_ptr(d_sink, "sink", dev);
  if (st != PSA_OK) return st;
  e = psa::launch_read_peak(d_buf, (uint32_t)bytes, d_sink, kPeakBlocks, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa::hip_fail(e, "read peak kernel launch");
  return PSA_OK;
}

psa_status psa_debug_mfma_peak(float* d_out, int64_t out_capacity, int32_t iters, void* stream) {
  if (!d_out) return set_error(PSA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (iters <= 0 || iters % 8) return set_error(PSA_ERR_INVALID_ARGUMENT, "iters must be a positive multiple of 8");
  if (out_capacity < (int64_t)kPeakBlocks * 256)
    return set_error(PSA_ERR_WORKSPACE_TOO_SMALL, "out needs " + std::to_string(kPeakBlocks * 256) + " entries");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
  psa_status st = psa::check_device_ptr(d_out, "out", dev);
  if (st != PSA_OK) return st;
  e = psa::launch_mfma_peak(d_out, iters, kPeakBlocks, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa::hip_fail(e, "mfma peak kernel launch");
  return PSA_OK;
}

psa_status psa_debug_issue_probe(int32_t pattern, int64_t* d_cycles, int64_t capacity, int32_t iters,
                                 void* stream) {
  if (!d_cycles) return set_error(PSA_ERR_INVALID_ARGUMENT, "cycles is NULL");
  if (pattern < 0 || pattern > 7) return set_error(PSA_ERR_INVALID_ARGUMENT, "pattern must be 0..7");
  if (iters <= 0) return set_error(PSA_ERR_INVALID_ARGUMENT, "iters must be positive");
  const int blocks = 256;
  if (capacity < (int64_t)blocks * 4)
    return set_error(PSA_ERR_WORKSPACE_TOO_SMALL, "cycles needs " + std::to_string(blocks * 4) + " entries");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::hip_fail(e, "hipGetDevice");
  psa_status st = psa::check_device_ptr(d_cycles, "cycles", dev);
  if (st != PSA_OK) return st;
  e = psa::launch_issue_probe(pattern, d_cycles, iters, blocks, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa::hip_fail(e, "issue probe kernel launch");
  return PSA_OK;
}

}  // extern "C"
