// Two measurement kernels that give the rooflines a measured ceiling next to
// the published one: a streaming read of device memory and a run of
// dependent bf16 MFMAs.  Diagnostics only; attention does not use them.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace psa {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
typedef float f32x4p __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));

constexpr int kPeakThreads = 256;
constexpr int kReadUnroll = 8;

// Each workgroup reads one contiguous span of the buffer, 256 x 16 bytes per
// load instruction and kReadUnroll instructions in flight per thread, with
// non-temporal buffer loads (measured fastest of strided / contiguous,
// default / non-temporal variants); loads past the end read zeros (the
// descriptor bounds the buffer).  The xor of everything read goes to
// sink[thread], so no load is dead.
__global__ __launch_bounds__(kPeakThreads) void read_peak_kernel(const char* buf, uint32_t bytes, uint32_t* sink) {
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(buf), (short)0, (int)bytes, 0x00020000);
  const uint32_t nchunks = bytes / 16;
  const uint32_t per = (nchunks + gridDim.x - 1) / gridDim.x;  // chunks per workgroup
  const uint32_t base = blockIdx.x * per;
  u32x4p acc = {0u, 0u, 0u, 0u};
  for (uint32_t c = threadIdx.x; c < per; c += kPeakThreads * kReadUnroll) {
    u32x4p v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const uint32_t chunk = base + c + (uint32_t)u * kPeakThreads;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (chunk < base + per ? chunk : nchunks) * 16u, 0,
                                                   2 /* non-temporal */);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  sink[blockIdx.x * kPeakThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Each wave runs one chain of `iters` dependent v_mfma_f32_16x16x32_bf16
// (16384 flop each); several waves per SIMD keep the matrix core busy.
__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8p a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)((lane + i) & 7));
    b[i] = (__bf16)(1e-3f * (float)((lane * 3 + i) & 7));
  }
  f32x4p c = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  out[blockIdx.x * kPeakThreads + threadIdx.x] = c[0] + c[1] + c[2] + c[3];
}

hipError_t launch_read_peak(const void* buf, uint32_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(read_peak_kernel, dim3(blocks), dim3(kPeakThreads), 0, s, static_cast<const char*>(buf), bytes,
                     sink);
  return hipGetLastError();
}

hipError_t launch_mfma_peak(float* out, int iters, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(kPeakThreads), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace psa
