// The low-bit projection's kernels for 3-bit codes (kernel and launch
// logic in wlowbit_gemm_impl.h).
#include "wlowbit_gemm_impl.h"

namespace ttq {
template hipError_t launch_gemm_q<3>(bool, bool, int, int, const GemmArgs&, hipStream_t);
}  // namespace ttq
