// Standalone merge of two partial attention results (BatchLLM summary,
// papercache.org, §2.2 Eq. 1: O = online_softmax(O_prefix, O_distinct)),
// plus a fill kernel used to poison workspace slots in debug plans.
//
// Memory bound: each row reads 2 * (head_dim + 2) floats and writes
// head_dim + 2.  A row is handled by head_dim/4 consecutive lanes of one
// wave (16-byte accesses), so reading m/l before writing them is ordered by
// the wave's lockstep execution and in-place use (o == o_a) is safe.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace psa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void merge_kernel(int64_t rows, int32_t head_dim, const float* o_a,
                                                    const float* m_a, const float* l_a, const float* o_b,
                                                    const float* m_b, const float* l_b, float* o, float* m,
                                                    float* l) {
  const int tpr = head_dim / 4;  // threads per row, divides 64
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t / tpr;
  const int c = (int)(t % tpr);
  if (row >= rows) return;
  const float ma = m_a[row], mb = m_b[row], la = l_a[row], lb = l_b[row];
  const f32x4 xa = *reinterpret_cast<const f32x4*>(o_a + row * head_dim + c * 4);
  const f32x4 xb = *reinterpret_cast<const f32x4*>(o_b + row * head_dim + c * 4);
  const float M = fmaxf(ma, mb);
  const float wa = la > 0.f ? la * expf(ma - M) : 0.f;
  const float wb = lb > 0.f ? lb * expf(mb - M) : 0.f;
  const float L = wa + wb;
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  if (L > 0.f) {
    const float ia = wa / L, ib = wb / L;
    r = xa * ia + xb * ib;
  }
  *reinterpret_cast<f32x4*>(o + row * head_dim + c * 4) = r;
  if (c == 0) {
    m[row] = L > 0.f ? M : -INFINITY;
    l[row] = L;
  }
}

__global__ __launch_bounds__(256) void fill_kernel(uint32_t* dst, int64_t n, uint32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = value;
}

hipError_t launch_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* m_a, const float* l_a,
                        const float* o_b, const float* m_b, const float* l_b, float* o, float* m, float* l,
                        hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t threads = rows * (head_dim / 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, rows, head_dim, o_a, m_a, l_a, o_b, m_b,
                     l_b, o, m, l);
  return hipGetLastError();
}

hipError_t launch_fill(uint32_t* dst, int64_t n, uint32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

}  // namespace psa
