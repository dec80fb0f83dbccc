// Instantiation of the skinny GEMM launches for f32 storage and 1 M-tile of 16 rows.
#include "gemm_impl.h"

namespace specdec {
namespace gemm_detail {
template hipError_t dispatch_epi<float, 1, false>(int, int, const GemmArgs&, hipStream_t, const LaunchTiming*);
}  // namespace gemm_detail
}  // namespace specdec
