// Forward dispatch: the wavefront-reduction kernel takes the units tagged
// "wave" by the build; the MFMA kernel (when built) takes the others. Both
// are persistent grids whose unit counts are read on the device, so nothing
// here waits for the build.
#include "sa_internal.h"

namespace sa {

bool mfma_enabled() { return false; }

hipError_t launch_forward(const sa_index* idx, const FwdArgs& a, hipStream_t s) {
  // Enough workgroups to fill 256 CUs a few times over; each loops over units.
  const unsigned grid = 1024;
  return launch_forward_wave(idx, a, s, grid);
}

}  // namespace sa
