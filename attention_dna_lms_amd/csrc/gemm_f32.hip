// fp32 instantiation of the skinny GEMM (fp32 models: all casts are exact).
#include "gemm_impl.h"

namespace evs {
template hipError_t launch_gemm<float>(int, int, int, int, const GemmArgs&, int, size_t, hipStream_t);
}  // namespace evs
