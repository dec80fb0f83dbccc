// Instantiation of the skinny GEMM launches for bf16 storage and 4 M-tiles of 16 rows.
#include "gemm_impl.h"

namespace specdec {
namespace gemm_detail {
template hipError_t dispatch_epi<bf16_t, 4, false>(int, int, const GemmArgs&, hipStream_t, const LaunchTiming*);
}  // namespace gemm_detail
}  // namespace specdec
