// bf16 instantiation of the skinny GEMM (all row-tile counts and epilogues).
#include "gemm_impl.h"

namespace evs {
template hipError_t launch_gemm<bf16>(int, int, int, int, const GemmArgs&, int, size_t, hipStream_t);
}  // namespace evs
