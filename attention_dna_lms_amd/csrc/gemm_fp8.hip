// FP8 (E4M3) weight instantiation of the skinny GEMM: bf16 activations, weight
// fragments converted to bf16 in registers, per-row scales on the reduced tile.
#include "gemm_impl.h"

namespace evs {
hipError_t launch_gemm_w8(int MT, int NT, int amode, int epi, const GemmArgs& a, int slices, size_t lds,
                          hipStream_t st) {
  return launch_gemm_w8_impl(MT, NT, amode, epi, a, slices, lds, st);
}
}  // namespace evs
