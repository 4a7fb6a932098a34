// Grouped gate+up with FP8 weights (kernels in grouped_impl.h).
#include "grouped_impl.h"

namespace moe {

hipError_t launch_gate_up_fp8(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s) {
  return a.scale_rows ? grouped_detail::launch<kFmtFP8, true, true>(a, rowcap, tiled, s)
                      : grouped_detail::launch<kFmtFP8, false, true>(a, rowcap, tiled, s);
}

}  // namespace moe
