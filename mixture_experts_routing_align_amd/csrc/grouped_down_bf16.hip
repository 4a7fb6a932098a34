// Grouped down with BF16 weights (kernels in grouped_impl.h).
#include "grouped_impl.h"

namespace moe {

hipError_t launch_down_bf16(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s) {
  return grouped_detail::launch<kFmtBF16, false, false>(a, rowcap, tiled, s);
}

}  // namespace moe
