// Grouped down projection with MXFP4 weights (kernels in grouped_impl.h).
#include "grouped_impl.h"

namespace moe {

hipError_t launch_down_fp4(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s) {
  return grouped_detail::launch<kFmtFP4, false, false>(a, rowcap, tiled, s);
}

}  // namespace moe
