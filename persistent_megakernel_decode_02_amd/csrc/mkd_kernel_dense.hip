// The persistent decode kernel for one sequence of a dense model.
#include "mkd_device.h"

namespace mkd {

extern "C" __global__ void __launch_bounds__(kThreads, 1) mkd_megakernel(KParams params) {
  (void)params;
  megakernel_body<K_DENSE>();
}

const void* kernel_dense() { return (const void*)mkd_megakernel; }

}  // namespace mkd
