// Skinny GEMM for the block-verification forward: Y[M, N] = A[M, K] * W[N, K]^T
// with M = batch * (gamma + 1) small (13 rows at gamma = 12). At such M every
// projection is bound by reading W from HBM once, so the kernel is a weight
// streamer: W is pre-packed into 1 KB MFMA fragments in exactly the order a
// wave consumes them (each wave reads one contiguous run of memory), the
// activations ride along from L2, and MFMA does the dot products.
//
// Work split: workgroup = (group of NT 16-column tiles, k-split); its 8 waves
// split the k-range further and are reduced through LDS in a fixed tree, so
// every output's summation order depends only on K and the launch shape, never
// on M or on other rows (block verify == sequential decode bit for bit).
// K-splits across workgroups meet in the last-arriving workgroup, which sums
// the partials in split order.
//
// Prologue (A_NORM): RMSNorm of fp32 residual rows, from per-16-column sums of
// squares the producing epilogue left behind. Epilogues: plain store (LM head),
// residual add + sums of squares (out / down projections), gated GELU (MLP up),
// and the mixer epilogue (in-projection + FIR or IIR operator, or the KV append
// of attention), which keeps each channel tile's q, k, v in one workgroup.
#pragma once

#include "evs_dev.h"

namespace evs {

template <int MT, int NT, int WV = 8> struct GemmCfg {
  static constexpr int WAVES = WV;
  static constexpr int BUFS = (4 * NT * MT <= 48) ? 4 : ((2 * NT * MT <= 48) ? 2 : 1);
  static constexpr int RS = NT * MT * 256;                          // floats per wave partial
};

// Activation fragment of one k-step for one 16-row tile, loaded raw and
// turned into the MFMA operand only when it is consumed (so the conversion
// never stalls the load pipeline). Rows past `rows` re-read the last valid
// row: an MFMA output column depends only on its own activation row and the
// columns of rows past `rows` are never stored, so no masking is needed.
// weights are read exactly once per call: non-temporal loads keep them from
// displacing the activations in the caches
__device__ __forceinline__ uint4 ld_stream(const u32x4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(p));
}

template <typename T, int AMODE> struct AFrag;
template <typename T> struct AFrag<T, A_ACT> {            // storage-type rows
  uint4 v;
  __device__ __forceinline__ void load(const GemmArgs& a, size_t m, int kofs) {
    v = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.A) + m * a.lda + kofs);
  }
  __device__ __forceinline__ uint4 get(float) const { return v; }
};
template <> struct AFrag<bf16, A_NORM> {                  // fp32 rows, RMSNorm -> bf16
  float4 lo, hi;
  __device__ __forceinline__ void load(const GemmArgs& a, size_t m, int kofs) {
    const float* xr = reinterpret_cast<const float*>(a.A) + m * a.lda + kofs;
    lo = *reinterpret_cast<const float4*>(xr);
    hi = *reinterpret_cast<const float4*>(xr + 4);
  }
  __device__ __forceinline__ uint4 get(float r) const {
    bf16x8 o;
    o[0] = (bf16)(lo.x * r); o[1] = (bf16)(lo.y * r); o[2] = (bf16)(lo.z * r); o[3] = (bf16)(lo.w * r);
    o[4] = (bf16)(hi.x * r); o[5] = (bf16)(hi.y * r); o[6] = (bf16)(hi.z * r); o[7] = (bf16)(hi.w * r);
    return __builtin_bit_cast(uint4, o);
  }
};
template <> struct AFrag<float, A_NORM> {                 // fp32 rows, RMSNorm -> fp32
  float4 v;
  __device__ __forceinline__ void load(const GemmArgs& a, size_t m, int kofs) {
    v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.A) + m * a.lda + kofs);
  }
  __device__ __forceinline__ uint4 get(float r) const {
    return __builtin_bit_cast(uint4, make_float4(v.x * r, v.y * r, v.z * r, v.w * r));
  }
};

__device__ __forceinline__ float gelu_f(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// ---------------------------------------------------------------- epilogues
// Epilogue inputs that do not depend on the product (the residual tile, the
// FIR window and taps, the committed IIR modes) are loaded when the kernel
// starts, so their latency hides under the weight stream.
constexpr int FIR_PRE = 4;   // window / tap values prefetched per thread (filters of <= 128 taps)

struct EpiPre {
  float4 xr[4];              // E_RESID: 16 residual values of this thread's row
  float win[FIR_PRE];        // MIX_FIR: window of the slice's first sequence
  float tap[FIR_PRE];        // MIX_FIR: taps of this channel tile
  float s0, lam, res;        // MIX_IIR: committed mode, pole, residue of (c, n)
};

template <typename T, int MT, int NT, int EPI>
__device__ __forceinline__ void epi_prefetch(const GemmArgs& a, EpiPre& pf, int g, int row0, int rows) {
  const int tid = threadIdx.x;
  constexpr int MR = MT * 16;
  if constexpr (EPI == E_RESID) {
    static_assert(NT * MR <= 512, "one residual row segment per thread");
    const int nt = tid / MR, m = tid % MR;
    if (tid < NT * MR && m < rows) {
      const float4* xr = reinterpret_cast<const float4*>(a.x + (size_t)(row0 + m) * a.ldx + (g * NT + nt) * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) pf.xr[q] = xr[q];
    }
  } else if constexpr (EPI == E_MIXER) {
    const MixArgs& x = a.mix;
    const int ch0 = g * 16;
    if (x.kind == MIX_FIR && x.L <= FIR_PRE * 32) {
      const int b = x.seq0 + row0 / x.P;
      const int tb = x.t[b];
      const float* ring = x.ring + (size_t)b * x.ring_bs;
#pragma unroll
      for (int q = 0; q < FIR_PRE; ++q) {
        const int idx = tid + q * 512, jj = idx >> 4, c = idx & 15;
        const int pos = tb - (x.L - 1) + jj;   // ring rows are always in range; pos < 0 reads as 0
        const float v = ring[(size_t)(pos & (x.R - 1)) * x.d + ch0 + c];
        pf.win[q] = (jj < x.L - 1 && pos >= 0) ? v : 0.f;
        const int tc = idx / x.L, tj = idx % x.L;
        pf.tap[q] = idx < 16 * x.L ? x.taps[(size_t)(ch0 + tc) * x.L + tj] : 0.f;
      }
    } else if (x.kind == MIX_IIR && tid < 256) {
      const int c = tid >> 4, n = tid & 15, ch = ch0 + c;
      const bool vn = n < x.N;
      const int b = x.seq0 + row0 / x.P;
      const int buf = x.iir_buf[b], slot = x.iir_slot[b];
      const float* base = x.iirst + (size_t)b * x.iir_bs;
      const size_t so = (size_t)buf * x.iir_buf_s + ((size_t)(slot < 0 ? 0 : slot) * x.d + ch) * x.N + (vn ? n : 0);
      const float sv = base[so];
      pf.s0 = (vn && slot >= 0) ? sv : 0.f;
      pf.lam = vn ? x.lam[(size_t)ch * x.N + n] : 0.f;
      pf.res = vn ? x.res[(size_t)ch * x.N + n] : 0.f;
    }
  }
}

template <typename T, int MT, int NT, int EPI>
__device__ void gemm_epilogue(const GemmArgs& a, const EpiPre& pf, const float* ep, float* scratch, int g,
                              int row0, int rows) {
  const int tid = threadIdx.x, nth = blockDim.x;
  constexpr int MR = MT * 16;
  if constexpr (EPI == E_STORE) {
    T* out = reinterpret_cast<T*>(a.out);
    for (int idx = tid; idx < NT * MR * 16; idx += nth) {
      const int nt = idx / (MR * 16), m = (idx / 16) % MR, n = idx & 15;
      const int col = (g * NT + nt) * 16 + n;
      if (m < rows && col < a.N) out[(size_t)(row0 + m) * a.ldo + col] = from_f<T>(ep[idx]);
    }
  } else if constexpr (EPI == E_RESID) {
    const int nt = tid / MR, m = tid % MR;
    if (tid < NT * MR && m < rows) {
      const int col0 = (g * NT + nt) * 16;
      float* xr = a.x + (size_t)(row0 + m) * a.ldx + col0;
      const float* er = ep + (nt * MR + m) * 16;
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[4 * q + 0] = pf.xr[q].x; v[4 * q + 1] = pf.xr[q].y; v[4 * q + 2] = pf.xr[q].z; v[4 * q + 3] = pf.xr[q].w;
      }
      float ss = 0.f;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        v[n] = v[n] + rnd<T>(er[n]);
        ss = fmaf(v[n], v[n], ss);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        reinterpret_cast<float4*>(xr)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      a.nrm_out[(size_t)(g * NT + nt) * a.nrm_ld + row0 + m] = ss;
    }
  } else if constexpr (EPI == E_GELU) {
    T* out = reinterpret_cast<T*>(a.out);
    for (int idx = tid; idx < MR * 16; idx += nth) {
      const int m = idx / 16, n = idx & 15;
      if (m >= rows) continue;
      const float gv = rnd<T>(ep[idx]);
      const float uv = rnd<T>(ep[MR * 16 + idx]);
      out[(size_t)(row0 + m) * a.ldo + g * 16 + n] = from_f<T>(gelu_f(gv) * uv);
    }
  } else {  // E_MIXER: ep[0] = q, ep[1] = k, ep[2] = v for channels g*16 .. g*16+15
    const MixArgs& x = a.mix;
    const float* eq = ep;
    const float* ek = ep + MR * 16;
    const float* ev = ep + 2 * MR * 16;
    T* out = reinterpret_cast<T*>(a.out);
    const int ch0 = g * 16;
    const int P = x.P;
    const int nseq = rows / P;
    const int sbase = x.seq0 + row0 / P;
    if (x.kind == MIX_ATTN) {
      T* kc = reinterpret_cast<T*>(x.kc);
      T* vt = reinterpret_cast<T*>(x.vt);
      for (int idx = tid; idx < rows * 16; idx += nth) {
        const int m = idx / 16, c = idx & 15;
        const int b = sbase + m / P, p = m % P;
        const int pos = x.t[b] + p;
        const int ch = ch0 + c, h = ch / x.Dh, dh = ch % x.Dh;
        out[(size_t)(row0 + m) * a.ldo + ch] = from_f<T>(eq[idx]);
        if (pos < x.cap) {
          kc[(size_t)b * x.kv_bs + ((size_t)h * x.cap + pos) * x.Dh + dh] = from_f<T>(ek[idx]);
          vt[(size_t)b * x.kv_bs + ((size_t)h * x.Dh + dh) * x.cap + pos] = from_f<T>(ev[idx]);
        } else {
          atomicOr(x.err, 2);
        }
      }
    } else if (x.kind == MIX_FIR) {
      const int L = x.L, W = L - 1 + P;
      const bool pre = L <= FIR_PRE * 32;
      float* tp = scratch;             // [16][L] taps
      float* hw = scratch + 16 * L;    // [W][16]: filter inputs at positions t-L+1 .. t+P-1
      if (pre) {
#pragma unroll
        for (int q = 0; q < FIR_PRE; ++q) {
          const int idx = tid + q * 512;
          if (idx < 16 * L) tp[idx] = pf.tap[q];
        }
      } else {
        for (int idx = tid; idx < 16 * L; idx += nth) tp[idx] = x.taps[(size_t)(ch0 + idx / L) * L + idx % L];
      }
      for (int j = 0; j < nseq; ++j) {
        const int b = sbase + j;
        const int tb = x.t[b];
        float* ring = x.ring + (size_t)b * x.ring_bs;
        if (j == 0 && pre) {
#pragma unroll
          for (int q = 0; q < FIR_PRE; ++q) {
            const int idx = tid + q * 512;
            if (idx < (L - 1) * 16) hw[idx] = pf.win[q];
          }
        } else {
          for (int idx = tid; idx < (L - 1) * 16; idx += nth) {
            const int pos = tb - (L - 1) + (idx >> 4);
            const float v = ring[(size_t)(pos & (x.R - 1)) * x.d + ch0 + (idx & 15)];
            hw[idx] = pos >= 0 ? v : 0.f;
          }
        }
        for (int idx = tid; idx < P * 16; idx += nth) {
          const int p = idx >> 4, c = idx & 15, m = j * P + p;
          const float h = rnd<T>(ek[m * 16 + c]) * rnd<T>(ev[m * 16 + c]);
          hw[(L - 1) * 16 + idx] = h;
          ring[(size_t)((tb + p) & (x.R - 1)) * x.d + ch0 + c] = h;
        }
        __syncthreads();
        for (int idx = tid; idx < P * 16; idx += nth) {
          const int p = idx >> 4, c = idx & 15, m = j * P + p;
          const float* tc = tp + c * L;
          float y = 0.f;
          for (int jj = 0; jj < L; ++jj) y = fmaf(tc[jj], hw[(L - 1 + p - jj) * 16 + c], y);
          out[(size_t)(row0 + m) * a.ldo + ch0 + c] = from_f<T>(rnd<T>(eq[m * 16 + c]) * y);
        }
        __syncthreads();
      }
      (void)W;
    } else {  // MIX_IIR: lanes (c, n), 16 modes of one channel in 16 adjacent lanes
      for (int j = 0; j < nseq; ++j) {
        const int b = sbase + j;
        if (tid < 256) {
          const int c = tid >> 4, n = tid & 15, ch = ch0 + c;
          const bool vn = n < x.N;
          const int buf = x.iir_buf[b], slot = x.iir_slot[b];
          float* base = x.iirst + (size_t)b * x.iir_bs;
          float s, lam, res;
          if (j == 0) {
            s = pf.s0; lam = pf.lam; res = pf.res;
          } else {
            s = (vn && slot >= 0) ? base[(size_t)buf * x.iir_buf_s + ((size_t)slot * x.d + ch) * x.N + n] : 0.f;
            lam = vn ? x.lam[(size_t)ch * x.N + n] : 0.f;
            res = vn ? x.res[(size_t)ch * x.N + n] : 0.f;
          }
          float* dst = base + (size_t)(buf ^ 1) * x.iir_buf_s;
          for (int p = 0; p < P; ++p) {
            const int m = j * P + p;
            const float h = rnd<T>(ek[m * 16 + c]) * rnd<T>(ev[m * 16 + c]);
            s = fmaf(lam, s, h);
            if (vn) dst[((size_t)p * x.d + ch) * x.N + n] = s;
            float r = vn ? res * s : 0.f;
            r += __shfl_xor(r, 8, 16);
            r += __shfl_xor(r, 4, 16);
            r += __shfl_xor(r, 2, 16);
            r += __shfl_xor(r, 1, 16);
            if (n == 0) out[(size_t)(row0 + m) * a.ldo + ch] = from_f<T>(rnd<T>(eq[m * 16 + c]) * r);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- kernel
template <typename T, int MT, int NT, int AMODE, int EPI, int WV = 8, int CHO = 0>
__global__ void __launch_bounds__(WV * 64) gemm_kernel(GemmArgs a) {
  static_assert(EPI != E_MIXER || WV == 8, "the mixer epilogue assumes 512 threads");
  using C = GemmCfg<MT, NT, WV>;
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP, RS = C::RS;
  // k-steps per pipeline chunk: one chunk of NT weight fragments and MT
  // activation fragments (8 registers each for fp32 rows feeding bf16, else 4)
  // per step stays within ~80 registers, two chunks within ~160
  constexpr int AREG = (AMODE == A_NORM && sizeof(T) == 2) ? 2 : 1;
  constexpr int PER = 20 / (NT + AREG * MT);
  constexpr int CH = CHO ? CHO : PER >= 8 ? 8 : PER >= 4 ? 4 : PER >= 2 ? 2 : 1;
  extern __shared__ float lds[];
  __shared__ int flag_s;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values live in scalar registers, so every guard below is a
  // uniform branch and the load/wait schedule stays exact
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x / a.KS, s = blockIdx.x - g * a.KS;
  const int row0 = blockIdx.y * a.rows_per_slice;
  const int rows = min(a.rows_per_slice, a.M - row0);
  float* rinv = lds;                 // [MT*16]
  float* red = lds + MT * 16;        // reduction buffers, then the epilogue tile + scratch

  const int kb = s * a.kps, ke = min(kb + a.kps, a.ksteps);
  const int per_wave = (ke - kb + C::WAVES - 1) / C::WAVES;
  const int wk0 = min(kb + wave * per_wave, ke), wk1 = min(wk0 + per_wave, ke);
  const int nch = (wk1 - wk0) / CH;          // full chunks of CH k-steps
  // this wave's fragment stream: step i of the wave's k-range lives at
  // wp[i * tstride + nt * 64] (the packed layout fixes the strides)
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.W) + (size_t)g * a.gstride + (size_t)wave * a.wstride + lane;
  const int rl = lane & 15, aoff = (lane >> 4) * E;

  // epilogue inputs first (only the workgroup that runs the epilogue needs
  // them, but which one that is is known only at the end)
  EpiPre pf;
  if (a.KS == 1) epi_prefetch<T, MT, NT, EPI>(a, pf, g, row0, rows);
  // each lane feeds activation rows mt*16 + rl (clamped to the last valid row)
  size_t arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = (size_t)(row0 + min(mt * 16 + rl, rows - 1));

  // two chunk buffers
  uint4 w0[CH][NT], w1[CH][NT];
  AFrag<T, AMODE> x0[CH][MT], x1[CH][MT];
  auto issue_w = [&](uint4 (&w)[CH][NT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[u][nt] = ld_stream(wp + (size_t)(k0 - wk0 + u) * a.tstride + nt * 64);
  };
  auto issue_x = [&](AFrag<T, AMODE> (&x)[CH][MT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) x[u][mt].load(a, arow[mt], (k0 + u) * KSTEP + aoff);
  };
  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float rr[MT];   // this lane's RMSNorm scale per row tile (A_NORM)
  auto compute = [&](uint4 (&w)[CH][NT], AFrag<T, AMODE> (&x)[CH][MT]) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 xv = x[u][mt].get(rr[mt]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mma_frag(w[u][nt], xv, acc[nt][mt], T());
      }
  };

  // the first chunk's weights go out before the norm prologue
  if (nch > 0) issue_w(w0, wk0);

  if constexpr (AMODE == A_NORM) {
    // rinv[r] = 1 / sqrt(mean(x_r^2) + eps) from the per-16-column sums of
    // squares: 32 lanes per row each add 8 partials (all loads in flight at
    // once), then a fixed butterfly over the 32 lanes.
    for (int base = 0; base < MT * 16 * 32; base += C::WAVES * 64) {   // whole waves per pass
      const int idx = base + tid;
      const int r = idx >> 5, j = idx & 31;
      if (r < MT * 16) {
        float sum = 0.f;
        for (int i0 = 0; i0 < a.n_part; i0 += 256) {
          float v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int i = i0 + j + 32 * q;
            v[q] = (r < rows && i < a.n_part) ? a.nrm_part[(size_t)i * a.nrm_ld + row0 + r] : 0.f;
          }
          sum += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        }
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 32);
        if (j == 0) rinv[r] = (r < rows) ? 1.0f / sqrtf(sum / a.fd + a.eps) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) rr[mt] = rinv[min(mt * 16 + rl, rows - 1)];
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) rr[mt] = 1.f;
  }
  if (nch > 0) issue_x(x0, wk0);

  // chunk pipeline: the next chunk's loads are issued (and pinned ahead by a
  // scheduling barrier) before this chunk computes; inside the loop the issue
  // is unconditional, so each MFMA waits only for its own fragments.
  if (nch > 0) {
    int c = 0;
    for (; c + 2 < nch; c += 2) {
      issue_w(w1, wk0 + (c + 1) * CH);
      issue_x(x1, wk0 + (c + 1) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w0, x0);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(w0, wk0 + (c + 2) * CH);
      issue_x(x0, wk0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, x1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c + 1 < nch) {
      issue_w(w1, wk0 + (c + 1) * CH);
      issue_x(x1, wk0 + (c + 1) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w0, x0);
      compute(w1, x1);
    } else {
      compute(w0, x0);
    }
  }
  // leftover k-steps (fewer than CH), one at a time
  for (int k = wk0 + nch * CH; k < wk1; ++k) {
    uint4 wr[NT];
    AFrag<T, AMODE> xr[MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wr[nt] = ld_stream(wp + (size_t)(k - wk0) * a.tstride + nt * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xr[mt].load(a, arow[mt], k * KSTEP + aoff);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4 xv = xr[mt].get(rr[mt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mma_frag(wr[nt], xv, acc[nt][mt], T());
    }
  }

  // fixed-tree reduction of the 8 waves' partial tiles through LDS
#pragma unroll
  for (int n = C::WAVES; n > 1;) {
    const int h = (C::BUFS < n / 2) ? C::BUFS : n / 2;
    if (wave >= n - h && wave < n) {
      float* b = red + (wave - (n - h)) * RS;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4*>(b + (nt * MT + mt) * 256 + lane * 4) = acc[nt][mt];
    }
    __syncthreads();
    if (wave >= n - 2 * h && wave < n - h) {
      const float* b = red + (wave - (n - 2 * h)) * RS;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[nt][mt] += *reinterpret_cast<const f32x4*>(b + (nt * MT + mt) * 256 + lane * 4);
    }
    __syncthreads();
    n -= h;
  }

  if (a.KS > 1) {
    const size_t tile = (size_t)blockIdx.y * a.n_groups + g;
    if (wave == 0) {
      float* mp = a.part + (tile * a.KS + s) * RS;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4*>(mp + (nt * MT + mt) * 256 + lane * 4) = acc[nt][mt];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) flag_s = (atomicAdd(a.cnt + tile, 1) == a.KS - 1);
    __syncthreads();
    if (!flag_s) return;
    __threadfence();
    if (wave == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s2 = 0; s2 < a.KS; ++s2) {
        const float* pp = a.part + (tile * a.KS + s2) * RS;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] += *reinterpret_cast<const f32x4*>(pp + (nt * MT + mt) * 256 + lane * 4);
      }
    }
    if (tid == 0) a.cnt[tile] = 0;
  }

  // epilogue tile ep[nt][m][n] (m < MT*16, n < 16)
  float* ep = red;
  if (wave == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4*>(ep + ((nt * MT * 16 + mt * 16 + rl) * 16 + 4 * (lane >> 4))) = acc[nt][mt];
  }
  __syncthreads();
  if (a.KS > 1) epi_prefetch<T, MT, NT, EPI>(a, pf, g, row0, rows);
  gemm_epilogue<T, MT, NT, EPI>(a, pf, ep, ep + NT * MT * 256, g, row0, rows);
}

template <typename T, int MT>
static hipError_t launch_gemm_mt(int NT, int amode, int epi, const GemmArgs& a, int slices,
                                 size_t lds, hipStream_t st) {
  dim3 grid(a.n_groups * a.KS, slices), block(512);
  if (NT == 3 && amode == A_NORM && epi == E_MIXER)
    gemm_kernel<T, MT, 3, A_NORM, E_MIXER><<<grid, block, lds, st>>>(a);
  else if (NT == 1 && amode == A_ACT && epi == E_RESID)
    gemm_kernel<T, MT, 1, A_ACT, E_RESID><<<grid, block, lds, st>>>(a);
  else if (NT == 2 && amode == A_NORM && epi == E_GELU)
    gemm_kernel<T, MT, 2, A_NORM, E_GELU><<<grid, block, lds, st>>>(a);
  else if (NT == 1 && amode == A_NORM && epi == E_STORE)
    gemm_kernel<T, MT, 1, A_NORM, E_STORE><<<grid, block, lds, st>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm(int MT, int NT, int amode, int epi, const GemmArgs& a, int slices,
                       size_t lds, hipStream_t st) {
  switch (MT) {
    case 1: return launch_gemm_mt<T, 1>(NT, amode, epi, a, slices, lds, st);
    case 2: return launch_gemm_mt<T, 2>(NT, amode, epi, a, slices, lds, st);
    case 3: return launch_gemm_mt<T, 3>(NT, amode, epi, a, slices, lds, st);
    case 4: return launch_gemm_mt<T, 4>(NT, amode, epi, a, slices, lds, st);
    case 5: return launch_gemm_mt<T, 5>(NT, amode, epi, a, slices, lds, st);
    case 6: return launch_gemm_mt<T, 6>(NT, amode, epi, a, slices, lds, st);
    case 7: return launch_gemm_mt<T, 7>(NT, amode, epi, a, slices, lds, st);
    case 8: return launch_gemm_mt<T, 8>(NT, amode, epi, a, slices, lds, st);
    case 9: return launch_gemm_mt<T, 9>(NT, amode, epi, a, slices, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace evs
