// Grouped down with FP8 weights (kernels in grouped_impl.h).
#include "grouped_impl.h"

namespace moe {

hipError_t launch_down_fp8(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s) {
  return a.scale_rows ? grouped_detail::launch<kFmtFP8, true, false>(a, rowcap, tiled, s)
                      : grouped_detail::launch<kFmtFP8, false, false>(a, rowcap, tiled, s);
}

}  // namespace moe
