// The persistent decode kernel for 2-8 sequences of a dense model decoded together.
#include "mkd_device.h"

namespace mkd {

extern "C" __global__ void __launch_bounds__(kThreads, 1) mkd_megakernel_batch(KParams params) {
  (void)params;
  megakernel_body<K_BATCH>();
}

const void* kernel_batch() { return (const void*)mkd_megakernel_batch; }

}  // namespace mkd
