// psa_decode_attention_noalloc: the fused decode launch for callers that
// cannot allocate device memory.  The kernels' scratch (arrival counters and
// fp32 partial results) lives in a static device array of this library
// instead of a caller workspace; the caller passes only the uploaded plan
// image, the inputs and the outputs.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// its device address (one per GPU, each GPU holding its own copy) comes from
// hipGetSymbolAddress, taken once per device on the first call there, with
// that device current, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "plan.h"
#include "psa_internal.h"

namespace psa {
psa_status decode_impl(const psa_plan* plan, const void* d_q, const void* d_k_pool, const void* d_v_pool,
                       void* d_out, float* d_out_m, float* d_out_l, const void* d_workspace, size_t bytes,
                       uint64_t* d_trace, void* stream, char* scratch);
}  // namespace psa

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU, until the process ends
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up yet)

}  // namespace

extern "C" psa_status psa_decode_attention_noalloc(const psa_plan* plan, const void* d_q, const void* d_k_pool,
                                                   const void* d_v_pool, void* d_out, float* d_out_m,
                                                   float* d_out_l, const void* d_image, size_t image_bytes,
                                                   void* stream) {
  if (!plan) return psa::set_error(PSA_ERR_INVALID_ARGUMENT, "plan is NULL");
  const int64_t need = plan->layout.total_bytes - plan->layout.counters;  // counters + partials
  if (need > (int64_t)kScratchBytes)
    return psa::set_error(PSA_ERR_WORKSPACE_TOO_SMALL,
                          "plan needs " + std::to_string(need) + " bytes of scratch; the library's static array holds " +
                              std::to_string(kScratchBytes) + " (use psa_decode_attention with a workspace)");
  if (image_bytes < (size_t)plan->layout.meta_bytes)
    return psa::set_error(PSA_ERR_WORKSPACE_TOO_SMALL, "plan image needs " + std::to_string(plan->layout.meta_bytes) +
                                                           " bytes, got " + std::to_string(image_bytes));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return psa::set_error(PSA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return psa::set_error(PSA_ERR_UNSUPPORTED, "device ordinal " + std::to_string(dev) + " beyond 63");
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return psa::set_error(PSA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      g_scratch[dev] = ptr;
    }
    base = g_scratch[dev];
  }
  return psa::decode_impl(plan, d_q, d_k_pool, d_v_pool, d_out, d_out_m, d_out_l, d_image, image_bytes, nullptr,
                          stream, static_cast<char*>(base));
}
