// Plain streaming read of a device buffer: the attainable-bandwidth reference
// that the HBM-bound decode is compared with.  Each thread keeps four 128-bit
// loads in flight over a grid-stride walk and folds them with XOR.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace attn {

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* __restrict__ p, size_t n, unsigned* sink) {
  unsigned acc = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

hipError_t launch_hbm_read(const void* p, size_t bytes, unsigned* sink, int cus, hipStream_t stream) {
  const size_t n = bytes / 16;
  // four work-groups per CU: enough loads in flight to cover HBM latency
  size_t grid = (size_t)cus * 4;
  const size_t need = (n + 255) / 256;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)p, n, sink);
  return hipGetLastError();
}

}  // namespace attn
