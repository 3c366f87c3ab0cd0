// Balanced ("stream-K") skinny GEMM for matrices whose column-group count is
// not a multiple of the workgroup count (the gated-MLP gate/up projection:
// 688 groups of 2 x 16 columns at d_ff = 11008).
//
// The packed weights of all groups form one stream of k-steps
// ([group][k-step][NT][64 lanes], consecutive groups adjacent in memory). The
// stream is cut into SK_WG * 8 equal contiguous runs, one per wave, so every
// workgroup reads the same number of bytes and the launch is a single round
// of one workgroup per CU. A wave's run crosses at most one group boundary;
// it accumulates the two sides separately. Inside a workgroup the waves'
// pieces of a group are summed in wave order; a group cut between two
// workgroups is finished by whichever of the two arrives second, which adds
// the lower workgroup's partial to the upper one's (fixed order, independent
// of arrival order and of the number of rows). Partials cross workgroups
// through device-coherent (sc1) stores and loads and an agent-scope counter
// that the finishing workgroup resets.
#pragma once

#include "gemm_impl.h"

namespace evs {

constexpr int SK_WG = SK_WGS;   // workgroups per launch (one per CU on MI355X)
constexpr int SK_MAXG = 4;     // groups one workgroup may touch
constexpr int SK_LDS_MAX = 156 * 1024;   // dynamic LDS limit set for the staged launch (160 KB minus static)

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The end of a balanced launch: the waves' pieces of each touched group are
// summed in wave order; cut groups (shared with a neighbour workgroup) are
// published first and their arrival counters bumped in one go; whole groups
// are finished while those round trips are in flight; then the second arrival
// of each cut group adds the lower workgroup's partial first and finishes it.
// `region` holds 8 * 2 * NT * 256 + NT * 256 floats (+ epilogue scratch).
template <typename T, int NT, int EPI>
__device__ __forceinline__ void sk_finish(const GemmArgs& a, const f32x4 (&accA)[NT], const f32x4 (&accB)[NT],
                                          const int (&tb)[9], int ks, float* region) {
  constexpr int MT = 1, WV = 8, TILE = NT * 256;
  __shared__ int last_s[SK_MAXG];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S0 = tb[0], S1 = tb[WV];
  const int rows = a.M;
  float* slotb = region;                            // [8 waves][2 sides][TILE]
  float* ep = slotb + WV * 2 * TILE;                // [TILE] epilogue tile + scratch
  // this wave's pieces: side 0 = its first group, side 1 = the next one
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    *reinterpret_cast<f32x4*>(slotb + (wave * 2 + 0) * TILE + nt * 256 + lane * 4) = accA[nt];
    *reinterpret_cast<f32x4*>(slotb + (wave * 2 + 1) * TILE + nt * 256 + lane * 4) = accB[nt];
  }
  __syncthreads();

  // Sum the workgroup's pieces of each group it touches (at most SK_MAXG),
  // in wave order. Cut groups (shared with a neighbour) are published first
  // and their arrival counters bumped in one go; whole groups are finished
  // while those round trips are in flight; then the second arrival of each
  // cut group adds the lower workgroup's partial first and finishes it.
  constexpr int PT = (TILE + 511) / 512;           // elements per thread
  const int gA = S0 / ks, ng = (S1 - 1) / ks - gA + 1;
  float v[SK_MAXG][PT];
#pragma unroll
  for (int gi = 0; gi < SK_MAXG; ++gi) {
#pragma unroll
    for (int q = 0; q < PT; ++q) v[gi][q] = 0.f;
    if (gi >= ng) continue;
    const int g = gA + gi;
#pragma unroll
    for (int jw = 0; jw < WV; ++jw) {
      const int t0 = tb[jw], t1 = tb[jw + 1];
      if (t0 >= t1) continue;
      const int gj = t0 / ks;
      int side = -1;
      if (g == gj) side = 0;
      else if (g == gj + 1 && t1 > (gj + 1) * ks) side = 1;
      if (side < 0) continue;
#pragma unroll
      for (int q = 0; q < PT; ++q) {
        const int e = tid + q * 512;
        if (e < TILE) v[gi][q] += slotb[(jw * 2 + side) * TILE + e];
      }
    }
  }
  auto is_whole = [&](int g) { return g * ks >= S0 && (g + 1) * ks <= S1; };
  auto side_of = [&](int g) { return g * ks < S0 ? 1 : 0; };   // 1: this workgroup holds the group's upper part
  bool any_cut = false;
#pragma unroll
  for (int gi = 0; gi < SK_MAXG; ++gi) {
    const int g = gA + gi;
    if (gi >= ng || is_whole(g)) continue;
    any_cut = true;
    float* mine = a.part + ((size_t)g * 2 + side_of(g)) * TILE;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int e = tid + q * 512;
      if (e < TILE) st_coherent(mine + e, v[gi][q]);
    }
  }
  if (any_cut) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid < SK_MAXG) {
      const int g = gA + tid;
      last_s[tid] = (tid < ng && !is_whole(g)) &&
                    __hip_atomic_fetch_add(a.cnt + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
    }
  }
  auto finish = [&](int g, const float (&vv)[PT]) {
    // MFMA D fragment (nt, lane l, i) holds output column 4 * (l / 16) + i of
    // activation row l % 16 -> epilogue tile ep[nt][row][column]
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int e = tid + q * 512;
      if (e < TILE) {
        const int nt = e / 256, l = (e / 4) & 63, i = e & 3;
        ep[(nt * 16 + (l & 15)) * 16 + 4 * (l >> 4) + i] = vv[q];
      }
    }
    __syncthreads();
    EpiPre pf{};
    gemm_epilogue<T, MT, NT, EPI>(a, pf, ep, ep + TILE, g, 0, rows);
    __syncthreads();
  };
#pragma unroll
  for (int gi = 0; gi < SK_MAXG; ++gi)
    if (gi < ng && is_whole(gA + gi)) finish(gA + gi, v[gi]);
  if (!any_cut) return;
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < SK_MAXG; ++gi) {
    const int g = gA + gi;
    if (gi >= ng || is_whole(g) || !last_s[gi]) continue;
    const int side = side_of(g);
    const float* other = a.part + ((size_t)g * 2 + (side ^ 1)) * TILE;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int e = tid + q * 512;
      if (e < TILE) {
        const float o = ld_coherent(other + e);
        v[gi][q] = side == 0 ? v[gi][q] + o : o + v[gi][q];
      }
    }
    if (tid == 0) a.cnt[g] = 0;
    finish(g, v[gi]);
  }
}

template <typename T, int NT, int AMODE, int EPI>
__global__ void __launch_bounds__(512) gemm_sk_kernel(GemmArgs a) {
  constexpr int MT = 1, WV = 8;
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP;
  constexpr int TILE = NT * 256;                   // floats of one group's output tile
  constexpr int AREG = (AMODE == A_NORM && sizeof(T) == 2) ? 2 : 1;
  constexpr int PER = 20 / (NT + AREG * MT);
  constexpr int CH = PER >= 8 ? 8 : PER >= 4 ? 4 : PER >= 2 ? 2 : 1;
  extern __shared__ float lds[];
  float* rinv = lds;                                // [16], then the finish region
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = a.ksteps;
  const long long total = (long long)a.n_groups * ks;
  // run boundaries of this workgroup's waves (the launch has exactly SK_WG
  // workgroups, so the division is by a power of two)
  constexpr long long NSLOT = (long long)SK_WG * WV;
  int tb[WV + 1];
#pragma unroll
  for (int jw = 0; jw <= WV; ++jw) tb[jw] = (int)(total * ((long long)blockIdx.x * WV + jw) / NSLOT);
  const int s0 = (int)(total * ((long long)blockIdx.x * WV + wave) / NSLOT);
  const int s1 = (int)(total * ((long long)blockIdx.x * WV + wave + 1) / NSLOT);
  const int g0 = s0 / ks;
  const int bnd = (g0 + 1) * ks;                    // first step of the next group
  const int rows = a.M;
  const int rl = lane & 15, aoff = (lane >> 4) * E;
  const size_t arow = (size_t)min(rl, rows - 1);
  const bool have = s1 > s0;
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.W) + lane + (have ? (size_t)s0 * NT * 64 : 0);

  uint4 w0[CH][NT], w1[CH][NT];
  AFrag<T, AMODE> x0[CH][MT], x1[CH][MT];
  // the k-column of step s inside its group
  auto kcol = [&](int s) { return s < bnd ? s - (bnd - ks) : s - bnd; };
  // steps past s1 re-read step s1 - 1 and are skipped by compute, so every
  // load is unconditional
  auto clampk = [&](int k) { return have ? min(k, s1 - 1) : 0; };
  auto issue_w = [&](uint4 (&w)[CH][NT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        w[u][nt] = ld_stream(wp + (size_t)(have ? clampk(k0 + u) - s0 : 0) * NT * 64 + nt * 64);
  };
  auto issue_x = [&](AFrag<T, AMODE> (&x)[CH][MT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) x[u][0].load(a, arow, (have ? kcol(clampk(k0 + u)) : 0) * KSTEP + aoff);
  };
  f32x4 accA[NT], accB[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { accA[nt] = f32x4{0.f, 0.f, 0.f, 0.f}; accB[nt] = accA[nt]; }
  float rr = 1.f;
  auto compute = [&](uint4 (&w)[CH][NT], AFrag<T, AMODE> (&x)[CH][MT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (k0 + u >= s1) break;
      const uint4 xv = x[u][0].get(rr);
      if (k0 + u < bnd) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) accA[nt] = mma_frag(w[u][nt], xv, accA[nt], T());
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) accB[nt] = mma_frag(w[u][nt], xv, accB[nt], T());
      }
    }
  };

  // start-up: norm partials, then two chunks, then the prologue waits for
  // its own loads only
  const int nch = (s1 - s0 + CH - 1) / CH;
  float nv[8];
  const int r = tid >> 5, j = tid & 31;
  if constexpr (AMODE == A_NORM) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = j + 32 * q;
      nv[q] = (r < rows && i < a.n_part) ? a.nrm_part[(size_t)i * a.nrm_ld + r] : 0.f;
    }
  }
  issue_x(x0, s0);
  issue_w(w0, s0);
  issue_x(x1, s0 + CH);
  issue_w(w1, s0 + CH);
  if constexpr (AMODE == A_NORM) {
    // rinv[r] from the per-16-column sums of squares (32 lanes per row)
    float sum = ((nv[0] + nv[1]) + (nv[2] + nv[3])) + ((nv[4] + nv[5]) + (nv[6] + nv[7]));
    for (int i0 = 256; i0 < a.n_part; i0 += 256) {   // wide models only
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + j + 32 * q;
        v[q] = (r < rows && i < a.n_part) ? a.nrm_part[(size_t)i * a.nrm_ld + r] : 0.f;
      }
      sum += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 32);
    if (j == 0) rinv[r] = (r < rows) ? 1.0f / sqrtf(sum / a.fd + a.eps) : 0.f;
    __syncthreads();
    rr = rinv[arow];
  }
  {
    int c = 0;
    for (; c + 3 < nch; c += 2) {
      compute(w0, x0, s0 + c * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_x(x0, s0 + (c + 2) * CH);
      issue_w(w0, s0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, x1, s0 + (c + 1) * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_x(x1, s0 + (c + 3) * CH);
      issue_w(w1, s0 + (c + 3) * CH);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nch - c == 3) {
      compute(w0, x0, s0 + c * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_x(x0, s0 + (c + 2) * CH);
      issue_w(w0, s0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, x1, s0 + (c + 1) * CH);
      compute(w0, x0, s0 + (c + 2) * CH);
    } else if (nch - c == 2) {
      compute(w0, x0, s0 + c * CH);
      compute(w1, x1, s0 + (c + 1) * CH);
    } else if (nch - c == 1) {
      compute(w0, x0, s0 + c * CH);
    }
  }

  sk_finish<T, NT, EPI>(a, accA, accB, tb, ks, lds + 16);
}

// Balanced launch for bf16 models with an RMSNorm'ed fp32 input (the gate/up
// projection): a workgroup's k-step runs wrap around groups, so it would read
// every activation column about 2.7 times. Instead the workgroup normalises
// the input rows once into LDS as bf16 (u = bf16(x * rinv), exactly the operand
// the per-step conversion forms) and the waves read their MFMA operands from
// there. The LDS region is reused by the finish after the main loop.
template <int NT, int EPI>
__global__ void __launch_bounds__(512) gemm_sk_staged_kernel(GemmArgs a) {
  using T = bf16;
  constexpr int WV = 8, KSTEP = 32;
  constexpr int CH = 4;
  extern __shared__ float lds[];
  float* rinv = lds;                                // [16]
  bf16* u = reinterpret_cast<bf16*>(lds + 16);      // [rows][K + 8]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = a.ksteps, K = ks * KSTEP, US = K + 8;
  const long long total = (long long)a.n_groups * ks;
  constexpr long long NSLOT = (long long)SK_WG * WV;
  int tb[WV + 1];
#pragma unroll
  for (int jw = 0; jw <= WV; ++jw) tb[jw] = (int)(total * ((long long)blockIdx.x * WV + jw) / NSLOT);
  const int s0 = (int)(total * ((long long)blockIdx.x * WV + wave) / NSLOT);
  const int s1 = (int)(total * ((long long)blockIdx.x * WV + wave + 1) / NSLOT);
  const int g0 = s0 / ks;
  const int bnd = (g0 + 1) * ks;
  const int rows = a.M;
  const int rl = lane & 15, aoff = (lane >> 4) * 8;
  const bf16* urow = u + (size_t)min(rl, rows - 1) * US + aoff;
  const bool have = s1 > s0;
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.W) + lane + (have ? (size_t)s0 * NT * 64 : 0);
  auto kcol = [&](int s) { return s < bnd ? s - (bnd - ks) : s - bnd; };
  auto clampk = [&](int k) { return have ? min(k, s1 - 1) : 0; };
  uint4 w0[CH][NT], w1[CH][NT];
  auto issue_w = [&](uint4 (&w)[CH][NT], int k0) {
#pragma unroll
    for (int q = 0; q < CH; ++q)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        w[q][nt] = ld_stream(wp + (size_t)(have ? clampk(k0 + q) - s0 : 0) * NT * 64 + nt * 64);
  };
  f32x4 accA[NT], accB[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { accA[nt] = f32x4{0.f, 0.f, 0.f, 0.f}; accB[nt] = accA[nt]; }
  auto compute = [&](uint4 (&w)[CH][NT], int k0) {
    uint4 xv[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) xv[q] = *reinterpret_cast<const uint4*>(urow + kcol(clampk(k0 + q)) * KSTEP);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (k0 + q >= s1) break;
      if (k0 + q < bnd) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) accA[nt] = mma_frag(w[q][nt], xv[q], accA[nt], T());
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) accB[nt] = mma_frag(w[q][nt], xv[q], accB[nt], T());
      }
    }
  };

  // start-up: norm partials, the first two weight chunks, the first half of
  // the input rows; then the norm, then the rows are normalised into LDS
  const int nch = (s1 - s0 + CH - 1) / CH;
  const int r = tid >> 5, j = tid & 31;
  float nv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = j + 32 * q;
    nv[q] = (r < rows && i < a.n_part) ? a.nrm_part[(size_t)i * a.nrm_ld + r] : 0.f;
  }
  issue_w(w0, s0);
  issue_w(w1, s0 + CH);
  constexpr int XB = 8;                              // float8 pieces per thread per pass
  const int n8 = rows * (K / 8);                     // 8-column pieces of the input rows
  const float* X = reinterpret_cast<const float*>(a.A);
  float4 xb[XB][2];
  auto load_x = [&](int pass) {
#pragma unroll
    for (int q = 0; q < XB; ++q) {
      const int idx = min((pass * XB + q) * 512 + tid, n8 - 1);
      const int rr = idx / (K / 8), kk = (idx % (K / 8)) * 8;
      const float* xr = X + act_off<8>(rr, kk, a.lda);
      xb[q][0] = *reinterpret_cast<const float4*>(xr);
      xb[q][1] = *reinterpret_cast<const float4*>(xr + 4);
    }
  };
  auto store_u = [&](int pass) {
#pragma unroll
    for (int q = 0; q < XB; ++q) {
      const int idx = (pass * XB + q) * 512 + tid;
      if (idx >= n8) break;
      const int rr = idx / (K / 8), kk = (idx % (K / 8)) * 8;
      const float sc = rinv[rr];
      bf16x8 o;
      o[0] = (bf16)(xb[q][0].x * sc); o[1] = (bf16)(xb[q][0].y * sc); o[2] = (bf16)(xb[q][0].z * sc); o[3] = (bf16)(xb[q][0].w * sc);
      o[4] = (bf16)(xb[q][1].x * sc); o[5] = (bf16)(xb[q][1].y * sc); o[6] = (bf16)(xb[q][1].z * sc); o[7] = (bf16)(xb[q][1].w * sc);
      *reinterpret_cast<bf16x8*>(u + (size_t)rr * US + kk) = o;
    }
  };
  load_x(0);
  {
    float sum = ((nv[0] + nv[1]) + (nv[2] + nv[3])) + ((nv[4] + nv[5]) + (nv[6] + nv[7]));
    for (int i0 = 256; i0 < a.n_part; i0 += 256) {   // wide models only
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + j + 32 * q;
        v[q] = (r < rows && i < a.n_part) ? a.nrm_part[(size_t)i * a.nrm_ld + r] : 0.f;
      }
      sum += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 32);
    if (j == 0) rinv[r] = (r < rows) ? 1.0f / sqrtf(sum / a.fd + a.eps) : 0.f;
  }
  __syncthreads();
  const int npass = (n8 + XB * 512 - 1) / (XB * 512);
  for (int pass = 0; pass < npass; ++pass) {
    if (pass > 0) load_x(pass);
    store_u(pass);
  }
  __syncthreads();

  {
    int c = 0;
    for (; c + 3 < nch; c += 2) {
      compute(w0, s0 + c * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(w0, s0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, s0 + (c + 1) * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(w1, s0 + (c + 3) * CH);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nch - c == 3) {
      compute(w0, s0 + c * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(w0, s0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, s0 + (c + 1) * CH);
      compute(w0, s0 + (c + 2) * CH);
    } else if (nch - c == 2) {
      compute(w0, s0 + c * CH);
      compute(w1, s0 + (c + 1) * CH);
    } else if (nch - c == 1) {
      compute(w0, s0 + c * CH);
    }
  }
  __syncthreads();   // every wave is done with the staged rows: the region is reused
  sk_finish<T, NT, EPI>(a, accA, accB, tb, ks, lds + 16);
}

template <typename T>
hipError_t launch_gemm_sk(int NT, int amode, int epi, const GemmArgs& a, size_t lds, hipStream_t st) {
  if (!(NT == 2 && amode == A_NORM && epi == E_GELU)) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    // the staged input rows need more than the default 64 KB of dynamic LDS
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_sk_staged_kernel<2, E_GELU>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, SK_LDS_MAX);
    if (attr != hipSuccess) return attr;
    gemm_sk_staged_kernel<2, E_GELU><<<SK_WG, 512, lds, st>>>(a);
  } else {
    gemm_sk_kernel<T, 2, A_NORM, E_GELU><<<SK_WG, 512, lds, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace evs
