// Entry point of the weight-streaming skinny GEMM (the kernel and its design: gemm_impl.h).

#include "gemm_impl.h"

namespace specdec {
namespace gemm_detail {
// each instantiation lives in its own translation unit (gemm_<format>_m<MT>.hip)
extern template hipError_t dispatch_epi<bf16_t, 1, false>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<bf16_t, 2, false>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<bf16_t, 4, false>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<float, 1, false>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<float, 2, false>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<float, 4, false>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<bf16_t, 1, true>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<bf16_t, 2, true>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
extern template hipError_t dispatch_epi<bf16_t, 4, true>(int, int, const GemmArgs&, hipStream_t,
                                                          const LaunchTiming*);
}  // namespace gemm_detail

using gemm_detail::dispatch_mt;

hipError_t launch_gemm(int dtype, int MT, int NU, int epi, const GemmArgs& a, hipStream_t st,
                       const LaunchTiming* tm) {
  if (a.n_units <= 0) return hipSuccess;
  if (a.KW < 1 || (a.NW != 4 && a.NW != 8 && a.NW != 16) || a.NW % a.KW) return hipErrorInvalidValue;
  if (a.M > MT * 16) return hipErrorInvalidValue;
  if (a.wq4) {
    // whole 128-element k-groups per split
    if (dtype != DT_BF16 || a.nkb % 4 || a.kb_per_split % 4) return hipErrorInvalidValue;
    return dispatch_mt<bf16_t, true>(MT, NU, epi, a, st, tm);
  }
  return dtype == DT_BF16 ? dispatch_mt<bf16_t, false>(MT, NU, epi, a, st, tm)
                          : dispatch_mt<float, false>(MT, NU, epi, a, st, tm);
}

}  // namespace specdec
