// The persistent decode kernel for one sequence of a top-2 MoE model.
#include "mkd_device.h"

namespace mkd {

extern "C" __global__ void __launch_bounds__(kThreads, 1) mkd_megakernel_moe(KParams params) {
  (void)params;
  megakernel_body<K_MOE>();
}

const void* kernel_moe() { return (const void*)mkd_megakernel_moe; }

}  // namespace mkd
