// Launch code of the persistent decode megakernel: the buffer-reset kernel,
// the LDS size of a launch, the co-residency query and the cooperative launch
// itself.  The three persistent kernels live in their own translation units
// (mkd_kernel_dense.hip, mkd_kernel_moe.hip, mkd_kernel_batch.hip).
#include <hip/hip_runtime.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "mkd_internal.h"

namespace mkd {

// The workspace of handles made by mkd_init_static: a device array of this
// library, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a
// stand-in): it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int static_workspace(int device, void** ptr, const char** why) {
  if (device < 0 || device >= kMaxDevices) {
    *why = "device index out of range for the static workspace";
    return MKD_E_INVALID;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess || cur != device) {
      *why = "the handle's device must be current when its static workspace is looked up";
      return MKD_E_HIP;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *why = "hipGetSymbolAddress of the static workspace failed";
      return MKD_E_HIP;
    }
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return MKD_OK;
}

extern "C" __global__ void mkd_reset(uint64_t* ll, size_t n, int32_t* status) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) ll[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x < S_WORDS) {
    const int k = threadIdx.x;
    status[k] = (k == S_WG || k == S_INSTR || k == S_TOKEN) ? -1 : 0;
  }
}

// ---------------------------------------------------------------- host-side launch

size_t lds_bytes(const KParams& p) {
  return ((size_t)p.x_floats + (size_t)p.res_floats + (size_t)p.out_floats + kRed) * sizeof(float) +
         (p.pre_off ? 0 : (size_t)p.pre_units * kWaves * 1024);
}

// the persistent kernel for `batch` sequences of a dense or MoE model (each
// defined in its own translation unit, which hands out its host-side handle)
static const void* kernel_for(int batch, bool moe) {
  return batch > 1 ? kernel_batch() : (moe ? kernel_moe() : kernel_dense());
}

int max_coop_blocks(int device, size_t lds, int batch, bool moe, int* out) {
  if (hipSetDevice(device) != hipSuccess) return MKD_E_HIP;
  const void* k = kernel_for(batch, moe);
  if (lds > 64 * 1024 && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return MKD_E_HIP;
  int per_cu = 0, n_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, lds) != hipSuccess)
    return MKD_E_HIP;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return MKD_E_HIP;
  *out = per_cu * n_cu;
  return MKD_OK;
}

int launch(const KParams& p, size_t ll_words, void* stream, void* ev0, void* ev1, bool cooperative,
           const char** why) {
  hipStream_t s = (hipStream_t)stream;
  const size_t lds = lds_bytes(p);
  int blocks = (int)((ll_words + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(mkd_reset, dim3(blocks), dim3(256), 0, s, p.h, ll_words, p.status);
  if (hipGetLastError() != hipSuccess) { *why = "reset kernel launch failed"; return MKD_E_HIP; }
  const void* k = kernel_for(p.B, p.E > 0);
  if (lds > 64 * 1024 && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    *why = "cannot raise the kernel's LDS limit";
    return MKD_E_HIP;
  }
  KParams pc = p;
  void* args[] = {&pc};
  if (ev0 && hipEventRecord((hipEvent_t)ev0, s) != hipSuccess) { *why = "hipEventRecord"; return MKD_E_HIP; }
  // A plain dispatch of the same grid (cooperative false) is for profilers
  // that cannot finish their output after a cooperative one: the grid was
  // checked to fit co-resident (max_coop_blocks), so on an idle device every
  // workgroup is resident at once either way.
  const hipError_t e =
      cooperative ? hipLaunchCooperativeKernel(k, dim3(p.n_wg), dim3(kThreads), args, (unsigned)lds, s)
                  : hipLaunchKernel(k, dim3(p.n_wg), dim3(kThreads), args, (unsigned)lds, s);
  if (e == hipErrorCooperativeLaunchTooLarge) {
    *why = "grid does not fit co-resident on the device";
    return MKD_E_COOPERATIVE;
  }
  if (e != hipSuccess) {
    *why = hipGetErrorString(e);
    return MKD_E_HIP;
  }
  if (ev1 && hipEventRecord((hipEvent_t)ev1, s) != hipSuccess) { *why = "hipEventRecord"; return MKD_E_HIP; }
  return MKD_OK;
}

}  // namespace mkd
