// The streaming-read probe of mkd_read_probe: not part of the decode kernels
// (kept out of their translation units, so their code and its digest do
// not change with it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mkd.h"

namespace mkd {

// A plain streaming read of `n16` 16-byte units, four loads in flight per
// thread, non-temporal: the achievable HBM read rate of the device, the
// context for the decode kernels' fraction of the published peak.  The sink
// is written only if the XOR of everything read equals a value it will not
// (so no load can be dropped).
typedef unsigned int probe_u4 __attribute__((ext_vector_type(4)));
extern "C" __global__ void __launch_bounds__(256) mkd_read_probe_kernel(const probe_u4* p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const probe_u4 a = __builtin_nontemporal_load(p + i);
    const probe_u4 b = __builtin_nontemporal_load(p + i + stride);
    const probe_u4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const probe_u4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const probe_u4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

int read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream, const char** why) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    *why = "device query";
    return MKD_E_HIP;
  }
  hipLaunchKernelGGL(mkd_read_probe_kernel, dim3(8 * n_cu), dim3(256), 0, (hipStream_t)stream,
                     (const probe_u4*)buf, bytes / 16, sink);
  if (hipGetLastError() != hipSuccess) {
    *why = "read probe launch failed";
    return MKD_E_HIP;
  }
  return MKD_OK;
}

}  // namespace mkd
