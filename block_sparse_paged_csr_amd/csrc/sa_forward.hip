// Forward dispatch: the wavefront-reduction kernel takes the units tagged
// "wave" by the build, the MFMA kernel the units tagged "mfma". Both read
// their unit counts on the device, so nothing here waits for the build.
#include "sa_internal.h"

namespace sa {

unsigned cu_count() {
  static thread_local int dev_cached = -1;
  static thread_local unsigned cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != dev_cached) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = (unsigned)n;
    dev_cached = dev;
  }
  return cus;
}

hipError_t launch_forward(const sa_index* idx, const FwdArgs& a, hipStream_t s) {
  // Wave path: a persistent grid, never larger than the unit bound.
  const int64_t cap = 1 << 20;
  const unsigned max_grid = (unsigned)(idx->max_units < cap ? idx->max_units : cap);
  hipError_t e = small_kernel_fits(a.head_dim, a.block_size, a.page_size, a.qhead)
                     ? launch_forward_small(idx, a, s, max_grid)
                     : launch_forward_wave(idx, a, s, max_grid);
  if (e != hipSuccess) return e;
  // MFMA path: one persistent workgroup per CU pulling units from a queue.
  if (idx->mfma_min_rows != INT32_MAX) e = launch_forward_mfma(idx, a, s, cu_count());
  return e;
}

}  // namespace sa
