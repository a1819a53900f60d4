// Forward dispatch: the wavefront-reduction kernel takes the units tagged
// "wave" by the build; the MFMA kernel (when built) takes the others. Both
// are persistent grids whose unit counts are read on the device, so nothing
// here waits for the build.
#include "sa_internal.h"

namespace sa {

bool mfma_enabled() { return false; }

hipError_t launch_forward(const sa_index* idx, const FwdArgs& a, hipStream_t s) {
  // One workgroup per unit up to a cap; past the cap workgroups loop. Units
  // beyond the device-side count exit at once.
  const int64_t cap = 16384;
  const unsigned grid = (unsigned)(idx->max_units < cap ? idx->max_units : cap);
  return launch_forward_wave(idx, a, s, grid);
}

}  // namespace sa
