// Measurement aid: stream one packed weight matrix exactly as gemm_kernel
// streams it (same workgroups, same fragment order and strides, same
// 16-byte non-temporal loads, two chunks of CH steps in flight) and do
// nothing else: no activations, no MFMA, no reduction, no epilogue. Its time
// is the floor of the projection's weight read on this part, against which
// the GEMM's own time is judged.
#include "evs_dev.h"

namespace evs {

template <int NT, int CH>
__global__ void __launch_bounds__(512) stream_kernel(const uint4* __restrict__ W, long long gstride, long long wstride,
                                                     long long tstride, int ksteps, unsigned* sink) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x;
  const int per_wave = (ksteps + 7) / 8;
  const int wk0 = min(wave * per_wave, ksteps), wk1 = min(wk0 + per_wave, ksteps);
  const int nch = (wk1 - wk0 + CH - 1) / CH;
  const u32x4* wp = reinterpret_cast<const u32x4*>(W) + lane + (nch > 0 ? (size_t)g * gstride + (size_t)wave * wstride : 0);
  auto wstep = [&](int k) { return max(min(k, wk1 - 1) - wk0, 0); };
  uint4 w0[CH][NT], w1[CH][NT];
  auto issue = [&](uint4 (&w)[CH][NT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        w[u][nt] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(wp + (size_t)wstep(k0 + u) * tstride + nt * 64));
  };
  unsigned acc = 0;
  auto consume = [&](uint4 (&w)[CH][NT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (k0 + u >= wk1) break;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc ^= w[u][nt].x ^ w[u][nt].y ^ w[u][nt].z ^ w[u][nt].w;
    }
  };
  issue(w0, wk0);
  issue(w1, wk0 + CH);
  int c = 0;
  for (; c + 3 < nch; c += 2) {
    consume(w0, wk0 + c * CH);
    __builtin_amdgcn_sched_barrier(0);
    issue(w0, wk0 + (c + 2) * CH);
    __builtin_amdgcn_sched_barrier(0);
    consume(w1, wk0 + (c + 1) * CH);
    __builtin_amdgcn_sched_barrier(0);
    issue(w1, wk0 + (c + 3) * CH);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (nch - c == 3) {
    consume(w0, wk0 + c * CH);
    issue(w0, wk0 + (c + 2) * CH);
    consume(w1, wk0 + (c + 1) * CH);
    consume(w0, wk0 + (c + 2) * CH);
  } else if (nch - c == 2) {
    consume(w0, wk0 + c * CH);
    consume(w1, wk0 + (c + 1) * CH);
  } else if (nch - c == 1) {
    consume(w0, wk0 + c * CH);
  }
  sink[(size_t)g * 512 + tid] = acc;
}

hipError_t launch_stream(int NT, int CH, const uint4* W, long long gstride, long long wstride, long long tstride,
                         int ksteps, int n_groups, unsigned* sink, hipStream_t st) {
  dim3 grid(n_groups), block(512);
  if (NT == 1 && CH == 2) stream_kernel<1, 2><<<grid, block, 0, st>>>(W, gstride, wstride, tstride, ksteps, sink);
  else if (NT == 2 && CH == 2) stream_kernel<2, 2><<<grid, block, 0, st>>>(W, gstride, wstride, tstride, ksteps, sink);
  else if (NT == 3 && CH == 1) stream_kernel<3, 1><<<grid, block, 0, st>>>(W, gstride, wstride, tstride, ksteps, sink);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace evs
