// Instantiation of the skinny GEMM launches for 4-bit block weights (bf16 activations) and 1
// M-tile of 16 rows.
#include "gemm_impl.h"

namespace specdec {
namespace gemm_detail {
template hipError_t dispatch_epi<bf16_t, 1, true>(int, int, const GemmArgs&, hipStream_t, const LaunchTiming*);
}  // namespace gemm_detail
}  // namespace specdec
