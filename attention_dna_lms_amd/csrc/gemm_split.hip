// bf16 split-K instantiation for multi-tile launches (k-range partials, then
// the reduction and epilogue of the one-kernel path).
#include "gemm_impl.h"

namespace evs {
hipError_t launch_gemm_split(int MT, int NT, int epi, const GemmArgs& a, int slices, size_t lds, hipStream_t st) {
  return launch_gemm_split_impl<bf16>(MT, NT, epi, a, slices, lds, st);
}
}  // namespace evs
