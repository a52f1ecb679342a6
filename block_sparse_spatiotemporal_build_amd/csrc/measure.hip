// Read-only HBM streaming probe: the measured reference for the HBM-bound
// kernels' rooflines (a plain read of a buffer larger than the last-level
// cache, no writes but one word per launch).

#include "launch.h"

namespace bsa {

// Each thread loads four 16-byte words per round (grid-stride) and folds them
// into an XOR, written only if it equals a value the caller never expects, so
// the loads cannot be removed.
__global__ void __launch_bounds__(256) hbm_read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* sink,
                                                       uint32_t never) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = i + (size_t)u * 256 < n16 ? p[i + (size_t)u * 256] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == never) sink[0] = acc;
}

bsa_status launch_hbm_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(4096), dim3(256), 0, stream, (const u32x4*)p, bytes / 16, sink,
                     0x9e3779b9u);
  return launch_ok("hbm_read_probe") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
