// Skinny GEMM for the block-verification forward: Y[M, N] = A[M, K] * W[N, K]^T
// with M = batch * (gamma + 1) small (13 rows at gamma = 12). At such M every
// projection is bound by reading W from HBM once, so the kernel is a weight
// streamer: W is pre-packed into 1 KB MFMA fragments ordered by step across
// the whole grid (step i of every wave of every workgroup side by side), so
// the chip reads one contiguous window of W front to back; the activations
// ride along from L2, and MFMA does the dot products.
//
// Work split: workgroup = group of NT 16-column tiles over the whole K; its 8
// waves split the k-range and are reduced through LDS in a fixed tree, so
// every output's summation order depends only on K, never on M or on other
// rows (block verify == sequential decode bit for bit). Splitting K across
// workgroups as well would need a cross-workgroup reduction whose device-scope
// round trip costs more than it saves at these sizes.
//
// Normed projections (A_NORM): the operand is the residual row as the producer
// stored it in the storage type, and the row's RMSNorm scale 1/rms, formed in
// the prologue from the per-16-column sums of squares the producer left
// behind (fixed order), multiplies the reduced fp32 tile: norm(x) W^T =
// rinv * (x W^T) with unit gain. Epilogues: plain store (LM head),
// residual add + sums of squares (out / down projections), gated GELU (MLP up),
// and the mixer epilogue (in-projection + FIR or IIR operator, or the KV append
// of attention), which keeps each channel tile's q, k, v in one workgroup.
#pragma once

#include <algorithm>

#include "evs_dev.h"

namespace evs {

template <int MT, int NT, int WV = 8> struct GemmCfg {
  static constexpr int WAVES = WV;
  static constexpr int BUFS = (4 * NT * MT <= 48) ? 4 : ((2 * NT * MT <= 48) ? 2 : 1);
  static constexpr int RS = NT * MT * 256;                          // floats per wave partial
  static constexpr bool FLAT = WV == 8 && NT * MT <= 4;             // one-barrier reduction
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
    v = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.A) + act_off<St<T>::E>((int)m, kofs, a.lda));
  }
  __device__ __forceinline__ uint4 get(float) const { return v; }
};
// normed projections read the residual rows in the storage type (the norm's
// scale goes onto the reduced tile), so their fragments are storage-type rows too
template <typename T> struct AFrag<T, A_NORM> : AFrag<T, A_ACT> {};

// each 16-lane row rotated by K lanes (DPP row_ror): a lane receives the value
// of the lane K away in its own row
template <int K>
__device__ __forceinline__ float dpp_row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + K, 0xF, 0xF, false));
}

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
  int tb;                    // MIX_FIR, MIX_ATTN: the first sequence's committed length
  int ibuf, islot;           // MIX_IIR: the first sequence's state buffer and slot
};

// Two phases, both issued after the first two chunks of weights and
// activations, so that no wave waits on memory before its weight stream
// starts: epi_prefetch loads what needs no other load (the residual tile,
// taps, poles and residues, the per-sequence integers); epi_prefetch_dep
// loads what is addressed by those integers (the FIR window, the committed
// IIR mode), and its wait for the integers overlaps the chunks' flight.
// (Issued before the weights, the residual tile's row stride sits in an
// argument line of its own, and the wait for that line held the out- and
// down-projections' streams back by one more memory round trip: a round of
// the 7B-shaped stack took 2.605 ms that way against 2.586 ms.)
template <typename T, int MT, int NT, int EPI>
__device__ __forceinline__ void epi_prefetch(const GemmArgs& a, EpiPre& pf, int g, int row0, int rows) {
  const int tid = threadIdx.x;
  constexpr int MR = MT * 16;
  if constexpr (EPI == E_RESID) {
    static_assert(NT * MR <= 512, "one residual row segment per thread");
    const int nt = tid / MR, m = tid % MR;
    if (tid < NT * MR && m < rows) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pf.xr[q] = *reinterpret_cast<const float4*>(a.x + act_off<St<T>::E>(row0 + m, (g * NT + nt) * 16 + 4 * q, a.ldx));
    }
  } else if constexpr (EPI == E_MIXER) {
    const MixArgs& x = a.mix;
    const int ch0 = g * 16;
    const int b = x.seq0 + row0 / x.P;
    if (x.kind == MIX_ATTN) {
      pf.tb = x.t[b];
    } else if (x.kind == MIX_FIR && x.L <= FIR_PRE * 32) {
      pf.tb = x.t[b];
#pragma unroll
      for (int q = 0; q < FIR_PRE; ++q) {
        const int idx = tid + q * 512;
        const int tc = idx / x.L, tj = idx % x.L;
        pf.tap[q] = idx < 16 * x.L ? x.taps[(size_t)(ch0 + tc) * x.L + tj] : 0.f;
      }
    } else if (x.kind == MIX_IIR) {
      // every thread: its channel's pole and residue of mode n; the first 256
      // (the first sequence's threads): that sequence's state buffer and slot
      const int c = (tid >> 4) & 15, n = tid & 15, ch = ch0 + c;
      const bool vn = n < x.N;
      pf.lam = vn ? x.lam[(size_t)ch * x.N + n] : 0.f;
      pf.res = vn ? x.res[(size_t)ch * x.N + n] : 0.f;
      if (tid < 256) {
        pf.ibuf = x.iir_buf[b];
        pf.islot = x.iir_slot[b];
      }
    }
  }
}

template <typename T, int MT, int NT, int EPI>
__device__ __forceinline__ void epi_prefetch_dep(const GemmArgs& a, EpiPre& pf, int g, int row0) {
  if constexpr (EPI == E_MIXER) {
    const int tid = threadIdx.x;
    const MixArgs& x = a.mix;
    const int ch0 = g * 16;
    const int b = x.seq0 + row0 / x.P;
    if (x.kind == MIX_FIR && x.L <= FIR_PRE * 32) {
      const float* ring = x.ring + (size_t)b * x.ring_bs;
#pragma unroll
      for (int q = 0; q < FIR_PRE; ++q) {
        const int idx = tid + q * 512, jj = idx >> 4, c = idx & 15;
        const int pos = pf.tb - (x.L - 1) + jj;   // ring rows are always in range; pos < 0 reads as 0
        const float v = ring[(size_t)(pos & (x.R - 1)) * x.d + ch0 + c];
        pf.win[q] = (jj < x.L - 1 && pos >= 0) ? v : 0.f;
      }
    } else if (x.kind == MIX_IIR) {
      const int c = (tid >> 4) & 15, n = tid & 15, ch = ch0 + c;
      const bool vn = n < x.N;
      pf.s0 = 0.f;
      if (tid < 256) {
        const int slot = pf.islot;
        const float* base = x.iirst + (size_t)b * x.iir_bs;
        const size_t so = (size_t)pf.ibuf * x.iir_buf_s + ((size_t)(slot < 0 ? 0 : slot) * x.d + ch) * x.N + (vn ? n : 0);
        const float sv = base[so];
        pf.s0 = (vn && slot >= 0) ? sv : 0.f;
      }
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
        *reinterpret_cast<float4*>(a.x + act_off<St<T>::E>(row0 + m, col0 + 4 * q, a.ldx)) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      a.nrm_out[(size_t)(row0 + m) * a.nrm_ld + g * NT + nt] = ss;
      if constexpr (sizeof(T) == 2) {
        // the same rows in bf16, two 8-element operand groups
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 b;
#pragma unroll
          for (int n = 0; n < 8; ++n) b[n] = (bf16)v[8 * h + n];
          *reinterpret_cast<uint4*>(a.xb_out + act_off<8>(row0 + m, col0 + 8 * h, a.ldx)) =
              __builtin_bit_cast(uint4, b);
        }
      }
    }
  } else if constexpr (EPI == E_GELU) {
    T* out = reinterpret_cast<T*>(a.out);
    for (int idx = tid; idx < MR * 16; idx += nth) {
      const int m = idx / 16, n = idx & 15;
      if (m >= rows) continue;
      const float gv = rnd<T>(ep[idx]);
      const float uv = rnd<T>(ep[MR * 16 + idx]);
      out[act_off<St<T>::E>(row0 + m, g * 16 + n, a.ldo)] = from_f<T>(gelu_f(gv) * uv);
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
    // (every per-sequence value is loaded before the first store: on this
    // GPU stores and loads share one in-order counter, so a load issued after
    // a store waits for the store too)
    if (x.kind == MIX_ATTN) {
      T* kc = reinterpret_cast<T*>(x.kc);
      T* vt = reinterpret_cast<T*>(x.vt);
      int* tl = reinterpret_cast<int*>(scratch);   // [nseq] committed lengths
      if (nseq > 1) {   // (one sequence: its length came with the prologue)
        for (int j = tid; j < nseq; j += nth) tl[j] = x.t[sbase + j];
        __syncthreads();
      }
      for (int idx = tid; idx < rows * 16; idx += nth) {
        const int m = idx / 16, c = idx & 15;
        const int b = sbase + m / P, p = m % P;
        const int pos = (nseq > 1 ? tl[m / P] : pf.tb) + p;
        const int ch = ch0 + c, h = ch / x.Dh, dh = ch % x.Dh;
        out[act_off<St<T>::E>(row0 + m, ch, a.ldo)] = from_f<T>(eq[idx]);
        if (pos < x.cap) {
          kc[(size_t)b * x.kv_bs + ((size_t)h * x.cap + pos) * x.Dh + dh] = from_f<T>(ek[idx]);
          vt[(size_t)b * x.kv_bs + (size_t)h * x.Dh * x.cap + ((size_t)(pos >> 4) * x.Dh + dh) * 16 + (pos & 15)] =
              from_f<T>(ev[idx]);
        } else {
          atomicOr(x.err, 2);
        }
      }
    } else if (x.kind == MIX_FIR) {
      // Sequences in batches of x.fb: the windows of a batch are loaded
      // together (one memory round trip per batch), its inputs h = k v written
      // to LDS and to each ring, then every (sequence, position, channel)
      // output of the batch is formed in one pass.
      const int L = x.L, LW = L - 1, WR = LW + P;   // window rows; rows per sequence buffer
      const int LP = L | 1;            // odd row stride: the 16 channels' taps sit in 16 distinct banks
      const bool pre = L <= FIR_PRE * 32;
      float* tp = scratch;             // [16][LP] taps
      float* hb = scratch + 16 * LP;   // [fb][WR][16]: a sequence's inputs at positions t-L+1 .. t+P-1
      if (pre) {
#pragma unroll
        for (int q = 0; q < FIR_PRE; ++q) {
          const int idx = tid + q * 512;
          if (idx < 16 * L) tp[(idx / L) * LP + idx % L] = pf.tap[q];
        }
      } else {
        for (int idx = tid; idx < 16 * L; idx += nth) tp[(idx / L) * LP + idx % L] = x.taps[(size_t)(ch0 + idx / L) * L + idx % L];
      }
      const int fb = max(1, min(x.fb, FIR_FB));
      for (int j0 = 0; j0 < nseq; j0 += fb) {
        const int nb = min(fb, nseq - j0);
        // committed lengths and windows of the batch: every load unconditional
        // (indices clamped to the batch), so all are in flight together; a
        // single-sequence launch keeps the window loaded with the prologue
        int tbv[FIR_FB];
        if (pre && nseq == 1) {   // (the length came with the prologue)
#pragma unroll
          for (int u = 0; u < FIR_FB; ++u) tbv[u] = pf.tb;
        } else {
#pragma unroll
          for (int u = 0; u < FIR_FB; ++u) tbv[u] = x.t[sbase + j0 + min(u, nb - 1)];
        }
        if (pre) {
          float wv[FIR_FB][FIR_PRE];
          if (nseq == 1) {
#pragma unroll
            for (int q = 0; q < FIR_PRE; ++q) wv[0][q] = pf.win[q];
          } else {
            // the loads as one group between scheduling barriers, then the
            // masking (pos < 0 reads as 0; ring rows are always in range)
#pragma unroll
            for (int u = 0; u < FIR_FB; ++u) {
              const float* ring = x.ring + (size_t)(sbase + j0 + min(u, nb - 1)) * x.ring_bs;
#pragma unroll
              for (int q = 0; q < FIR_PRE; ++q) {
                const int idx = tid + q * 512;
                wv[u][q] = ring[(size_t)((tbv[u] - LW + (idx >> 4)) & (x.R - 1)) * x.d + ch0 + (idx & 15)];
              }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < FIR_FB; ++u)
#pragma unroll
              for (int q = 0; q < FIR_PRE; ++q) {
                const int idx = tid + q * 512, jw = idx >> 4;
                const int pos = tbv[u] - LW + jw;
                const unsigned keep = (jw < LW && pos >= 0) ? 0xffffffffu : 0u;
                wv[u][q] = __uint_as_float(__float_as_uint(wv[u][q]) & keep);
              }
          }
#pragma unroll
          for (int u = 0; u < FIR_FB; ++u) {
            if (u < nb) {
#pragma unroll
              for (int q = 0; q < FIR_PRE; ++q) {
                const int idx = tid + q * 512;
                if (idx < LW * 16) hb[u * WR * 16 + idx] = wv[u][q];
              }
            }
          }
        } else {
          for (int idx = tid; idx < nb * LW * 16; idx += nth) {
            const int u = idx / (LW * 16), r = idx % (LW * 16);
            const int b = sbase + j0 + u;
            int tb = 0;
#pragma unroll
            for (int v = 0; v < FIR_FB; ++v) tb = v == u ? tbv[v] : tb;
            const int pos = tb - LW + (r >> 4);
            const float v = x.ring[(size_t)b * x.ring_bs + (size_t)(pos & (x.R - 1)) * x.d + ch0 + (r & 15)];
            hb[u * WR * 16 + r] = pos >= 0 ? v : 0.f;
          }
        }
        for (int idx = tid; idx < nb * P * 16; idx += nth) {
          const int u = idx / (P * 16), r = idx % (P * 16), p = r >> 4, c = r & 15;
          const int b = sbase + j0 + u, m = (j0 + u) * P + p;
          const float h = rnd<T>(ek[m * 16 + c]) * rnd<T>(ev[m * 16 + c]);
          int tb = 0;
#pragma unroll
          for (int v = 0; v < FIR_FB; ++v) tb = v == u ? tbv[v] : tb;
          hb[(u * WR + LW) * 16 + r] = h;
          x.ring[(size_t)b * x.ring_bs + (size_t)((tb + p) & (x.R - 1)) * x.d + ch0 + c] = h;
        }
        __syncthreads();
        for (int idx = tid; idx < nb * P * 16; idx += nth) {
          const int u = idx / (P * 16), r = idx % (P * 16), p = r >> 4, c = r & 15;
          const int m = (j0 + u) * P + p;
          const float* tc = tp + c * LP;
          const float* hc = hb + (u * WR + LW + p) * 16 + c;   // input at lag jj: hc[-16 * jj]
          // taps in order 0 .. L-1 (one fma chain); the LDS reads of 16 taps go
          // out together ahead of their fmas
          float y = 0.f;
          int jj = 0;
          for (; jj + 16 <= L; jj += 16) {
            float tv[16], hv[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) { tv[q] = tc[jj + q]; hv[q] = hc[-16 * (jj + q)]; }
#pragma unroll
            for (int q = 0; q < 16; ++q) y = fmaf(tv[q], hv[q], y);
          }
          for (; jj < L; ++jj) y = fmaf(tc[jj], hc[-16 * jj], y);
          out[act_off<St<T>::E>(row0 + m, ch0 + c, a.ldo)] = from_f<T>(rnd<T>(eq[m * 16 + c]) * y);
        }
        __syncthreads();
      }
    } else {  // MIX_IIR
      // Thread (half h, channel c, mode n): the 16 modes of a channel sit in
      // one 16-lane DPP row; the two halves of the workgroup take two
      // sequences at a time. Per position: the recurrence step s = lam s + h
      // (serial in position order, one fma), the mode to the state, r = res s,
      // and the row's 16 r summed by rotate-and-add over 8, 4, 2, 1 lanes:
      // every addition pairs the same two partial sums in either rotation
      // direction, so the row's first lane holds exactly
      // ((r0+r8)+(r4+r12)) + ((r2+r10)+(r6+r14)) +
      // (((r1+r9)+(r5+r13)) + ((r3+r11)+(r7+r15))). No barrier: the inputs
      // are the epilogue tile in LDS, the outputs go to memory.
      const int half = tid >> 8, c = (tid >> 4) & 15, n = tid & 15, ch = ch0 + c;
      const bool vn = n < x.N;
      const int nr = (nseq + 1) / 2;   // rounds of two sequences
      for (int r0 = 0; r0 < nr; r0 += IIR_FB / 2) {
        constexpr int RB = IIR_FB / 2;
        const int nb = min(RB, nr - r0);
        // this half's sequences of the batch (clamped: a missing odd sequence
        // repeats the last and is skipped below)
        int dbv[RB], slv[RB];
        float sv[RB];
        if (nseq == 1) {   // (buffer and slot came with the prologue, to the first 256 threads: the ones that work)
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            dbv[u] = pf.ibuf;
            slv[u] = pf.islot;
          }
        } else {
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const int j = min(2 * (r0 + min(u, nb - 1)) + half, nseq - 1);
            dbv[u] = x.iir_buf[sbase + j];
            slv[u] = x.iir_slot[sbase + j];
          }
        }
        if (nseq == 1) {
#pragma unroll
          for (int u = 0; u < RB; ++u) sv[u] = pf.s0;
        } else {
          // addresses, then the loads as one group (scheduling barriers keep
          // the compiler from issuing them one round trip at a time), then v,
          // or +0 for padding modes and an empty state (a mask, not a select,
          // which would become a branch around each load)
          const float* ap[RB];
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const int j = min(2 * (r0 + min(u, nb - 1)) + half, nseq - 1);
            ap[u] = x.iirst + (size_t)(sbase + j) * x.iir_bs + (size_t)dbv[u] * x.iir_buf_s +
                    ((size_t)(slv[u] < 0 ? 0 : slv[u]) * x.d + ch) * x.N + (vn ? n : 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          float v[RB];
#pragma unroll
          for (int u = 0; u < RB; ++u) v[u] = *ap[u];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const unsigned keep = (vn && slv[u] >= 0) ? 0xffffffffu : 0u;
            sv[u] = __uint_as_float(__float_as_uint(v[u]) & keep);
          }
        }
        if (nseq > 1) {
          // Several sequences: this thread's RB sequences run together, their
          // chains interleaved position by position so that their latencies
          // overlap (each sequence's arithmetic and stores exactly as in the
          // one-sequence loop below). A round past the batch (or past an odd
          // count) computes on the clamped sequence and stores nothing.
          constexpr int ICH = 4;
          const float lam = pf.lam, res = pf.res;
          int jv[RB];
          bool ok[RB];
          float* dst[RB];
          float sr[RB];
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const int j = 2 * (r0 + u) + half;
            ok[u] = u < nb && j < nseq;   // uniform per wave
            jv[u] = min(2 * (r0 + min(u, nb - 1)) + half, nseq - 1);
            dst[u] = x.iirst + (size_t)(sbase + jv[u]) * x.iir_bs + (size_t)(dbv[u] ^ 1) * x.iir_buf_s;
            sr[u] = sv[u];
          }
          for (int p0 = 0; p0 < P; p0 += ICH) {
            const int np = min(ICH, P - p0);
            float hv[RB][ICH], qv[RB][ICH], sq[RB][ICH];
#pragma unroll
            for (int u = 0; u < RB; ++u)
#pragma unroll
              for (int q = 0; q < ICH; ++q) {
                const int m = jv[u] * P + p0 + min(q, np - 1);
                hv[u][q] = rnd<T>(ek[m * 16 + c]) * rnd<T>(ev[m * 16 + c]);
                qv[u][q] = rnd<T>(eq[m * 16 + c]);
              }
#pragma unroll
            for (int q = 0; q < ICH; ++q)
#pragma unroll
              for (int u = 0; u < RB; ++u) {
                sr[u] = q < np ? fmaf(lam, sr[u], hv[u][q]) : sr[u];
                sq[u][q] = sr[u];
              }
            if (vn) {
#pragma unroll
              for (int u = 0; u < RB; ++u)
                if (ok[u]) {
#pragma unroll
                  for (int q = 0; q < ICH; ++q)
                    dst[u][((size_t)(p0 + min(q, np - 1)) * x.d + ch) * x.N + n] = sq[u][q];
                }
            }
#pragma unroll
            for (int u = 0; u < RB; ++u)
#pragma unroll
              for (int q = 0; q < ICH; ++q) {
                float rs = vn ? res * sq[u][q] : 0.f;
                rs += dpp_row_ror<8>(rs);
                rs += dpp_row_ror<4>(rs);
                rs += dpp_row_ror<2>(rs);
                rs += dpp_row_ror<1>(rs);
                sq[u][q] = rs;
              }
            if (n == 0) {
#pragma unroll
              for (int u = 0; u < RB; ++u)
                if (ok[u]) {
#pragma unroll
                  for (int q = 0; q < ICH; ++q)
                    out[act_off<St<T>::E>(row0 + jv[u] * P + p0 + min(q, np - 1), ch, a.ldo)] =
                        from_f<T>(qv[u][q] * sq[u][q]);
                }
            }
          }
        } else
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int j = 2 * (r0 + u) + half;
          if (u < nb && j < nseq) {   // uniform per wave
            float s = sv[u];
            const float lam = pf.lam, res = pf.res;
            float* dst = x.iirst + (size_t)(sbase + j) * x.iir_bs + (size_t)(dbv[u] ^ 1) * x.iir_buf_s;
            for (int p0 = 0; p0 < P; p0 += IIR_CH) {
              const int np = min(IIR_CH, P - p0);
              // a chunk's inputs h = k v and gates q first (LDS), then the
              // recurrence alone (one fma per position), then the state
              // stores, the mode sums and the outputs: no wait and no branch
              // inside the serial part
              float hv[IIR_CH], qv[IIR_CH], sq[IIR_CH];
#pragma unroll
              for (int q = 0; q < IIR_CH; ++q) {
                const int m = j * P + p0 + min(q, np - 1);
                hv[q] = rnd<T>(ek[m * 16 + c]) * rnd<T>(ev[m * 16 + c]);
                qv[q] = rnd<T>(eq[m * 16 + c]);
              }
#pragma unroll
              for (int q = 0; q < IIR_CH; ++q) {
                s = q < np ? fmaf(lam, s, hv[q]) : s;
                sq[q] = s;
              }
              // (slots past the chunk's last position repeat its state and
              // gate: their stores rewrite that position's values, so no
              // branch is needed around them)
              if (vn) {
#pragma unroll
                for (int q = 0; q < IIR_CH; ++q) dst[((size_t)(p0 + min(q, np - 1)) * x.d + ch) * x.N + n] = sq[q];
              }
#pragma unroll
              for (int q = 0; q < IIR_CH; ++q) {
                float rs = vn ? res * sq[q] : 0.f;
                rs += dpp_row_ror<8>(rs);
                rs += dpp_row_ror<4>(rs);
                rs += dpp_row_ror<2>(rs);
                rs += dpp_row_ror<1>(rs);
                sq[q] = rs;
              }
              if (n == 0) {
#pragma unroll
                for (int q = 0; q < IIR_CH; ++q)
                  out[act_off<St<T>::E>(row0 + j * P + p0 + min(q, np - 1), ch, a.ldo)] = from_f<T>(qv[q] * sq[q]);
              }
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- kernel
// FP8 weight fragment (16 bytes per lane: E4M3 values of two consecutive MFMA
// k-steps, 8 each) -> the two bf16 operands. E4M3 values are exact in bf16;
// the row scale is applied to the reduced tile.
template <bool UPPER>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned x) {   // bytes 0,1 (or 2,3) of x
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, UPPER));
}
__device__ __forceinline__ void fp8_to_bf16(uint4 w, uint4& lo, uint4& hi) {
  lo = make_uint4(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x), fp8x2_to_bf16x2<false>(w.y),
                  fp8x2_to_bf16x2<true>(w.y));
  hi = make_uint4(fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z), fp8x2_to_bf16x2<false>(w.w),
                  fp8x2_to_bf16x2<true>(w.w));
}

template <typename T, int MT, int NT, int AMODE, int EPI, int WV = 8, int CHO = 0, int MINB = 1, bool W8 = false,
          bool PART = false>
__global__ void __launch_bounds__(WV * 64, MINB) gemm_kernel(GemmArgs a) {
  static_assert(EPI != E_MIXER || WV == 8, "the mixer epilogue assumes 512 threads");
  static_assert(!W8 || sizeof(T) == 2, "FP8 weights feed the bf16 MFMA");
  using C = GemmCfg<MT, NT, WV>;
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP, RS = C::RS;
  // a weight step: one MFMA k-step, or two for FP8 weights (16 bytes per lane)
  constexpr int KPW = W8 ? 2 : 1;
  // k-steps per pipeline chunk: one chunk of NT weight fragments and MT
  // activation fragments (4 registers each) per step stays within ~64
  // registers, the two chunks in flight within ~128 (normed bf16 rows of a
  // multi-tile launch keep the shallower chunks measured best for them: the
  // registers go to the row tiles)
  constexpr int AREG = (AMODE == A_NORM && MT >= 2 && sizeof(T) == 2) ? 2 : 1;
  constexpr int PER = 16 / (NT + KPW * AREG * MT);
  // Measured at the 7B shapes with the step-major weight layout (round time,
  // 8k context, gamma 12): single-tile bf16 out- and down-projections 2-step
  // chunks (2.623 ms per round against 2.631 / 2.629 with 1 / 3 steps and
  // 2.665 with 4), gate/up 2 (1: +11 us, 3: +61 us); the single-tile
  // in-projection takes 1-step chunks at its launch. Multi-tile and FP8
  // launches keep the depths measured for them before.
  constexpr int CAP = NT == 1 ? ((MT == 1 && !W8) ? 2 : 4) : NT == 2 ? 2 : 8;
  constexpr int CH = CHO ? CHO : PER < 1 ? 1 : PER < CAP ? PER : CAP;
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values live in scalar registers, so every guard below is a
  // uniform branch and the load/wait schedule stays exact
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x;
  const int row0 = blockIdx.y * a.rows_per_slice;
  const int rows = min(a.rows_per_slice, a.M - row0);
  float* rinv = lds;                 // [MT*16] the rows' RMSNorm scales (A_NORM)
  float* red = lds + MT * 16;        // reduction buffers, then the epilogue tile + scratch
  // rinv[r] = 1 / sqrt(mean(x_r^2) + eps) from the row's n_part per-16-column
  // sums of squares (contiguous, nrm_ld per row): per pass of 256, lane j of
  // the row's 32 adds partials 8j .. 8j + 7 in a fixed tree (sum = v when the
  // first pass was loaded early), then a fixed butterfly over the 32
  constexpr int NP = AMODE == A_NORM ? (MT * 16 * 32 + C::WAVES * 64 - 1) / (C::WAVES * 64) : 1;
  auto load8 = [&](float (&v)[8], int r, int i) __attribute__((always_inline)) {
    const float* pr = a.nrm_part + (size_t)(row0 + min(r, rows - 1)) * a.nrm_ld + i;
    if (r < rows && i + 8 <= a.n_part && (a.nrm_ld & 3) == 0) {   // two aligned 16-byte loads
      const float4 lo = *reinterpret_cast<const float4*>(pr), hi = *reinterpret_cast<const float4*>(pr + 4);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (r < rows && i + q < a.n_part) ? pr[q] : 0.f;
    }
  };
  auto row_scales = [&](int pss, float sum, int i_begin) __attribute__((always_inline)) {
    const int idx = pss * C::WAVES * 64 + tid;
    const int r = idx >> 5, j = idx & 31;
    for (int i0 = i_begin; i0 < a.n_part; i0 += 256) {   // wide models only, when loaded early
      float v[8];
      load8(v, r, i0 + 8 * j);
      sum += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 32);
    if (j == 0 && r < MT * 16) rinv[r] = (r < rows) ? 1.0f / sqrtf(sum / a.fd + a.eps) : 0.f;
  };

  const int kb = 0, ke = a.ksteps;
  const int per_wave = (ke - kb + C::WAVES - 1) / C::WAVES;
  const int wk0 = min(kb + wave * per_wave, ke), wk1 = min(wk0 + per_wave, ke);
  const int nch = (wk1 - wk0 + CH - 1) / CH;   // chunks of CH k-steps (the last may be partial)
  // this wave's fragment stream: step i of the wave's k-range lives at
  // wp[i * tstride + nt * 64] (the packed layout fixes the strides). A wave
  // with no k-steps streams nothing useful: its (never consumed) loads read
  // the matrix's first fragment, so every load below is unconditional and
  // each wait covers exactly the loads it needs.
  // (the offset is formed unconditionally and selected, so its strides are
  // read with the other argument fields instead of behind a branch)
  const size_t woff = (size_t)g * a.gstride + (size_t)wave * a.wstride;
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.W) + lane + (nch > 0 ? woff : 0);
  const int rl = lane & 15, aoff = (lane >> 4) * E;

  // epilogue inputs (only the workgroup that runs the epilogue needs them,
  // but which one that is is known only at the end)
  EpiPre pf;
  // each lane feeds activation rows mt*16 + rl (clamped to the last valid row)
  size_t arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = (size_t)(row0 + min(mt * 16 + rl, rows - 1));

  f32x4 acc[NT][MT];
  if constexpr (PART) {
    // the eight k-range partials gemm_part_kernel formed (wave w takes range
    // w's chains, exactly what this kernel's wave w would have computed), or
    // the four pair sums gemm_pair_kernel formed (wave w < 4 takes ranges
    // w + (w + 4), the tree's first level; waves 4..7 hold -0, the exact
    // additive identity, so the tree's remaining levels are unchanged).
    // Issued before the norm's loads, so both are in flight together.
    epi_prefetch<T, MT, NT, EPI>(a, pf, g, row0, rows);
    const int np = a.nparts == 4 ? 4 : 8;
    const f32x4* pp = reinterpret_cast<const f32x4*>(a.part) +
                      ((((size_t)blockIdx.y * np + min(wave, np - 1)) * a.n_groups + g) * MT) * NT * 64 + lane;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = pp[(mt * NT + nt) * 64];
    epi_prefetch_dep<T, MT, NT, EPI>(a, pf, g, row0);
    if constexpr (AMODE == A_NORM) {
#pragma unroll
      for (int pss = 0; pss < NP; ++pss) row_scales(pss, 0.f, 0);
    }
    if (wave >= np) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{-0.f, -0.f, -0.f, -0.f};
    }
  } else {
  // two chunk buffers
  uint4 w0[CH][NT], w1[CH][NT];
  AFrag<T, AMODE> x0[CH][MT][KPW], x1[CH][MT][KPW];
  // steps past wk1 (the tail of the last chunk, or the chunk after it)
  // re-read step wk1 - 1 and are skipped by compute
  auto wstep = [&](int k) { return max(min(k, wk1 - 1) - wk0, 0); };
  auto issue_w = [&](uint4 (&w)[CH][NT], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[u][nt] = ld_stream(wp + (size_t)wstep(k0 + u) * a.tstride + nt * 64);
  };
  auto issue_x = [&](AFrag<T, AMODE> (&x)[CH][MT][KPW], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < KPW; ++h)
          x[u][mt][h].load(a, arow[mt], (max(min(k0 + u, wk1 - 1), 0) * KPW + h) * KSTEP + aoff);
  };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](uint4 (&w)[CH][NT], AFrag<T, AMODE> (&x)[CH][MT][KPW], int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (k0 + u >= wk1) break;
      if constexpr (W8) {
        uint4 wl[NT], wh[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) fp8_to_bf16(w[u][nt], wl[nt], wh[nt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 xa = x[u][mt][0].get(1.f), xb = x[u][mt][KPW - 1].get(1.f);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt][mt] = mma_frag(wl[nt], xa, acc[nt][mt], T());
            acc[nt][mt] = mma_frag(wh[nt], xb, acc[nt][mt], T());
          }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 xv = x[u][mt][0].get(1.f);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mma_frag(w[u][nt], xv, acc[nt][mt], T());
        }
      }
    }
  };

  // Start-up order: the norm's per-16-column sums of squares are loaded
  // first, then the first two chunks of activations and weights, then the
  // epilogue's inputs, and only then does the norm prologue wait (for its
  // own loads alone), so the weight stream starts at once and two chunks are
  // in flight from the start.
  // (many-row launches skip the early load: its registers would spill)
  constexpr bool PRE = AMODE == A_NORM && MT <= 2;
  float nv[PRE ? NP : 1][8];
  const bool nrm_pre = PRE && a.n_part <= 256;
  if constexpr (PRE) {
#pragma unroll
    for (int pss = 0; pss < NP; ++pss) {
      const int idx = pss * C::WAVES * 64 + tid, r = idx >> 5, j = idx & 31;
      load8(nv[pss], nrm_pre ? r : rows, 8 * j);
    }
  }
  issue_x(x0, wk0);
  issue_w(w0, wk0);
  issue_x(x1, wk0 + CH);
  issue_w(w1, wk0 + CH);
  epi_prefetch<T, MT, NT, EPI>(a, pf, g, row0, rows);
  epi_prefetch_dep<T, MT, NT, EPI>(a, pf, g, row0);

  if constexpr (AMODE == A_NORM) {
    // (the scales are read from LDS by the epilogue tile's formation, after
    // the reduction's barriers)
#pragma unroll
    for (int pss = 0; pss < NP; ++pss) {
      float sum = 0.f;
      if constexpr (PRE)
        sum = ((nv[pss][0] + nv[pss][1]) + (nv[pss][2] + nv[pss][3])) +
              ((nv[pss][4] + nv[pss][5]) + (nv[pss][6] + nv[pss][7]));
      row_scales(pss, sum, nrm_pre ? a.n_part : 0);
    }
  }

  // chunk pipeline: chunks c and c + 1 are in flight while chunk c computes;
  // the loop body issues unconditionally (the tail is peeled), so each MFMA
  // waits only for its own fragments.
  {
    int c = 0;
    for (; c + 3 < nch; c += 2) {
      compute(w0, x0, wk0 + c * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_x(x0, wk0 + (c + 2) * CH);
      issue_w(w0, wk0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, x1, wk0 + (c + 1) * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_x(x1, wk0 + (c + 3) * CH);
      issue_w(w1, wk0 + (c + 3) * CH);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nch - c == 3) {
      compute(w0, x0, wk0 + c * CH);
      __builtin_amdgcn_sched_barrier(0);
      issue_x(x0, wk0 + (c + 2) * CH);
      issue_w(w0, wk0 + (c + 2) * CH);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, x1, wk0 + (c + 1) * CH);
      compute(w0, x0, wk0 + (c + 2) * CH);
    } else if (nch - c == 2) {
      compute(w0, x0, wk0 + c * CH);
      compute(w1, x1, wk0 + (c + 1) * CH);
    } else if (nch - c == 1) {
      compute(w0, x0, wk0 + c * CH);
    }
  }

  }   // streaming

  // Reduction of the 8 waves' partial tiles in the fixed tree
  // ((w0 + w4) + (w2 + w6)) + ((w1 + w5) + (w3 + w7)). Small tiles: every wave
  // stores its partial once and each thread sums its elements straight into
  // the epilogue tile (one barrier). Large tiles: the same tree staged through
  // the BUFS buffers that fit.
  float* ep;
  if constexpr (C::FLAT) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4*>(red + wave * RS + (nt * MT + mt) * 256 + lane * 4) = acc[nt][mt];
    __syncthreads();
    ep = red + C::WAVES * RS;
    for (int e = tid; e < RS; e += C::WAVES * 64) {
      const float* pp = red + e;
      const float v = ((pp[0] + pp[4 * RS]) + (pp[2 * RS] + pp[6 * RS])) +
                      ((pp[RS] + pp[5 * RS]) + (pp[3 * RS] + pp[7 * RS]));
      // MFMA D fragment (nt, mt, lane l, i): output column 4 * (l / 16) + i of
      // activation row 16 * mt + l % 16 -> epilogue tile ep[nt][row][column]
      const int ntmt = e >> 8, l = (e >> 2) & 63, i = e & 3;
      const int nt = ntmt / MT, mt = ntmt % MT;
      const float sc = W8 ? a.wscale[(g * NT + nt) * 16 + 4 * (l >> 4) + i] : 1.f;
      const float vs = W8 ? v * sc : v;
      ep[((nt * MT * 16 + mt * 16 + (l & 15)) * 16) + 4 * (l >> 4) + i] =
          AMODE == A_NORM ? vs * rinv[mt * 16 + (l & 15)] : vs;
    }
    __syncthreads();
  } else {
    // The same tree as pairs (dst += src) level by level, BUFS pairs per LDS
    // round trip: w0+=w4, w2+=w6, w1+=w5, w3+=w7 | w0+=w2, w1+=w3 | w0+=w1.
    // The association is the same for any number of buffers, so it does not
    // depend on how many row tiles (and so how much LDS) the launch has.
    static_assert(C::WAVES == 8, "the reduction tree is written for 8 waves");
    constexpr int PDST[7] = {0, 2, 1, 3, 0, 1, 0}, PSRC[7] = {4, 6, 5, 7, 2, 3, 1};
    constexpr int LV[4] = {0, 4, 6, 7};   // first pair of each level
#pragma unroll
    for (int lv = 0; lv < 3; ++lv) {
#pragma unroll
      for (int c0 = LV[lv]; c0 < LV[lv + 1]; c0 += C::BUFS) {
        const int c1 = min(c0 + C::BUFS, LV[lv + 1]);
#pragma unroll
        for (int c = c0; c < c1; ++c) {
          if (wave == PSRC[c]) {
            float* b = red + (c - c0) * RS;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<f32x4*>(b + (nt * MT + mt) * 256 + lane * 4) = acc[nt][mt];
          }
        }
        __syncthreads();
#pragma unroll
        for (int c = c0; c < c1; ++c) {
          if (wave == PDST[c]) {
            const float* b = red + (c - c0) * RS;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[nt][mt] += *reinterpret_cast<const f32x4*>(b + (nt * MT + mt) * 256 + lane * 4);
          }
        }
        __syncthreads();
      }
    }
    // epilogue tile ep[nt][m][n] (m < MT*16, n < 16)
    ep = red;
    if (wave == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 sc = f32x4{1.f, 1.f, 1.f, 1.f};
        if constexpr (W8) sc = *reinterpret_cast<const f32x4*>(a.wscale + (g * NT + nt) * 16 + 4 * (lane >> 4));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 vs = W8 ? acc[nt][mt] * sc : acc[nt][mt];
          *reinterpret_cast<f32x4*>(ep + ((nt * MT * 16 + mt * 16 + rl) * 16 + 4 * (lane >> 4))) =
              AMODE == A_NORM ? vs * rinv[mt * 16 + rl] : vs;
        }
      }
    }
    __syncthreads();
  }
  gemm_epilogue<T, MT, NT, EPI>(a, pf, ep, ep + NT * MT * 256, g, row0, rows);
}

// ------------------------------------------------------------ split K
// Multi-tile launches (bf16 rows) in two kernels.
// gemm_part_kernel: one workgroup per (eight column groups, one of the eight
// k-ranges gemm_kernel gives its waves, row slice); wave w takes group 8c + w
// and forms, for every row tile, exactly the MFMA chain gemm_kernel's wave r
// forms for that group (range r, ascending k, from zero), writing it to the
// partial buffer. The row tiles' activation fragments of each chunk of k-steps
// are staged once in LDS and shared by the eight waves (one stream of
// activations per eight groups instead of one per group), and a wave keeps no
// activation fragments in flight in registers. gemm_kernel<..., PART> then
// loads wave w's partials from range w, reduces them in its fixed tree and
// runs its epilogue, so every output equals the one-kernel result bit for bit.
constexpr int PK = 2;   // k-steps per staged activation chunk

template <typename T, int MT, int NT>
__global__ void __launch_bounds__(512) gemm_part_kernel(GemmArgs a) {
  static_assert(sizeof(T) == 2, "bf16 rows only");
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP;
  constexpr int XF = PK * MT * 64;                   // 16-byte units per staged chunk
  constexpr int XPT = (XF + 511) / 512;              // staging loads per thread
  constexpr int XB = XPT * 512;                      // buffer stride: every thread writes every round
  extern __shared__ float lds[];
  uint4* xs = reinterpret_cast<uint4*>(lds);         // [2][XB]: [PK][MT][64] and padding
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x * 8 + wave;
  const bool gv = g < a.n_groups;
  const int r = blockIdx.y;
  const int row0 = blockIdx.z * a.rows_per_slice;
  const int rows = min(a.rows_per_slice, a.M - row0);
  const int ks = a.ksteps, pw = (ks + 7) / 8;
  const int kb = min(r * pw, ks), ke = min(kb + pw, ks);
  const int nchk = (ke - kb + PK - 1) / PK;
  // range r's steps are gemm_kernel's wave r's: local step k - kb of wave slot r
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.W) + lane + (gv ? (size_t)g * a.gstride + (size_t)r * a.wstride : 0);
  const T* A = reinterpret_cast<const T*>(a.A);

  // staging: unit idx = (u * MT + mt) * 64 + l holds lane l's 16 bytes of row
  // tile mt at k-step u of the chunk (rows past the slice re-read its last row)
  auto x_addr = [&](int idx, int c) __attribute__((always_inline)) -> const uint4* {
    const int l = idx & 63, mt = (idx >> 6) % MT, u = (idx >> 6) / MT;
    const int k = min(kb + c * PK + u, ke - 1);
    const int row = row0 + min(mt * 16 + (l & 15), rows - 1);
    return reinterpret_cast<const uint4*>(A + act_off<E>(row, k * KSTEP + (l >> 4) * E, a.lda));
  };
  auto issue_w = [&](uint4 (&w)[PK][NT], int c) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PK; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int k = min(kb + c * PK + u, ke - 1);
        w[u][nt] = ld_stream(wp + (size_t)max(k - kb, 0) * a.tstride + nt * 64);
      }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 w0[PK][NT], w1[PK][NT];
  if (nchk > 0) {
    // chunk 0's activations straight into LDS buffer 0
#pragma unroll
    for (int q = 0; q < XPT; ++q) xs[tid + q * 512] = *x_addr(min(tid + q * 512, XF - 1), 0);
    issue_w(w0, 0);
    if (nchk > 1) issue_w(w1, 1);
  }
  // chunk c: its activations are in LDS buffer c & 1 and its weights in w0
  // (even c) or w1 (odd c). Chunk c + 1's activations are loaded while chunk c
  // computes and stored to the other buffer afterwards; chunk c + 2's weights
  // replace chunk c's.
  auto step = [&](int c, uint4 (&w)[PK][NT]) __attribute__((always_inline)) {
    __syncthreads();                      // chunk c staged; chunk c - 1's buffer free
    // (after the last chunk this re-stages the last chunk into the free buffer:
    // harmless, and it keeps the staging free of branches)
    // (three named registers rather than an array: at most 3 rounds for 9 row
    // tiles of PK k-steps)
    static_assert(XPT <= 3, "staging rounds");
    const int cn = min(c + 1, nchk - 1);
    uint4 xn0, xn1, xn2;
    xn0 = *x_addr(min(tid, XF - 1), cn);
    if constexpr (XPT > 1) xn1 = *x_addr(min(tid + 512, XF - 1), cn);
    if constexpr (XPT > 2) xn2 = *x_addr(min(tid + 1024, XF - 1), cn);
    const uint4* xb = xs + (c & 1) * XB;
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      if (kb + c * PK + u < ke) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 x = xb[(u * MT + mt) * 64 + lane];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mma_frag(w[u][nt], x, acc[mt][nt], T());
        }
      }
    }
    if (c + 2 < nchk) issue_w(w, c + 2);
    uint4* dst = xs + ((c + 1) & 1) * XB;
    dst[tid] = xn0;
    if constexpr (XPT > 1) dst[tid + 512] = xn1;
    if constexpr (XPT > 2) dst[tid + 1024] = xn2;
  };
  for (int c = 0; c < nchk; c += 2) {
    step(c, w0);
    if (c + 1 < nchk) step(c + 1, w1);
  }
  if (gv) {
    f32x4* pp = reinterpret_cast<f32x4*>(a.part) +
                ((((size_t)blockIdx.z * 8 + r) * a.n_groups + g) * MT) * NT * 64 + lane;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pp[(mt * NT + nt) * 64] = acc[mt][nt];
  }
}

// gemm_pair_kernel: one workgroup per (four column groups, range pair p, row
// slice); wave w takes group 4c + (w & 3) over k-range p + 4 (w >> 2), forming
// the same MFMA chain as gemm_kernel's wave of that range. Both ranges'
// activation chunks are staged in LDS (each shared by four waves); at the end
// the waves of range p + 4 hand their tiles to those of range p through LDS,
// which add them (range p + range p + 4: the first level of gemm_kernel's
// tree) and store one partial per pair: half the partial bytes of
// gemm_part_kernel for twice its activation staging.
template <typename T, int MT, int NT>
__global__ void __launch_bounds__(512) gemm_pair_kernel(GemmArgs a) {
  static_assert(sizeof(T) == 2, "bf16 rows only");
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP;
  constexpr int XF = PK * MT * 64;                   // 16-byte units per staged chunk of one range
  constexpr int XPT = (XF + 511) / 512;              // staging loads per thread and range
  constexpr int XB = XPT * 512;                      // per-range buffer stride
  static_assert(XPT <= 3, "staging rounds");
  extern __shared__ float lds[];
  uint4* xs = reinterpret_cast<uint4*>(lds);         // [2 buffers][2 ranges][XB]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gi = wave & 3, h = wave >> 2;
  const int g = blockIdx.x * 4 + gi;
  const bool gv = g < a.n_groups;
  const int p = blockIdx.y;                          // range pair: ranges p and p + 4
  const int row0 = blockIdx.z * a.rows_per_slice;
  const int rows = min(a.rows_per_slice, a.M - row0);
  const int ks = a.ksteps, pw = (ks + 7) / 8;
  // both ranges of the pair (range p is never shorter than range p + 4)
  const int kb0 = min(p * pw, ks), ke0 = min(kb0 + pw, ks);
  const int kb1 = min((p + 4) * pw, ks), ke1 = min(kb1 + pw, ks);
  const int kb = h ? kb1 : kb0, ke = h ? ke1 : ke0;  // this wave's range
  const int nchk = (ke0 - kb0 + PK - 1) / PK;
  // (an empty range p + 4 re-reads its wave slot's first fragment: the packed
  // buffer holds every slot at full length)
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.W) + lane +
                    (gv ? (size_t)g * a.gstride + (size_t)(h ? p + 4 : p) * a.wstride : 0);
  const T* A = reinterpret_cast<const T*>(a.A);

  // staging unit idx (< 2 * XF): range idx / XF, then (u * MT + mt) * 64 + l
  // within it, as in gemm_part_kernel (k-steps past a range's end re-read its
  // last step; an empty range reads the matrix's last step)
  auto x_addr = [&](int idx, int c) __attribute__((always_inline)) -> const uint4* {
    const int hh = idx >= XF ? 1 : 0, j = idx - hh * XF;
    const int l = j & 63, mt = (j >> 6) % MT, u = (j >> 6) / MT;
    const int b0 = hh ? kb1 : kb0, e0 = hh ? ke1 : ke0;
    const int k = max(min(b0 + c * PK + u, e0 - 1), 0);
    const int row = row0 + min(mt * 16 + (l & 15), rows - 1);
    return reinterpret_cast<const uint4*>(A + act_off<E>(row, k * KSTEP + (l >> 4) * E, a.lda));
  };
  auto x_unit = [&](int q) __attribute__((always_inline)) { return min(q, 2 * XF - 1); };
  auto x_slot = [&](int q) __attribute__((always_inline)) {   // LDS slot of staging unit q
    return q >= XF ? XB + (q - XF) : q;
  };
  auto issue_w = [&](uint4 (&w)[PK][NT], int c) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PK; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int k = min(kb + c * PK + u, ke - 1);
        w[u][nt] = ld_stream(wp + (size_t)max(k - kb, 0) * a.tstride + nt * 64);
      }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 w0[PK][NT], w1[PK][NT];
  // each thread stages units tid + 512 q, q < 2 XPT (both ranges)
  if (nchk > 0) {
#pragma unroll
    for (int q = 0; q < 2 * XPT; ++q) {
      const int uq = tid + q * 512;
      if (uq < 2 * XF) xs[x_slot(uq)] = *x_addr(x_unit(uq), 0);
    }
    issue_w(w0, 0);
    if (nchk > 1) issue_w(w1, 1);
  }
  auto step = [&](int c, uint4 (&w)[PK][NT]) __attribute__((always_inline)) {
    __syncthreads();                      // chunk c staged; chunk c - 1's buffers free
    const int cn = min(c + 1, nchk - 1);
    uint4 xn0, xn1, xn2, xn3, xn4, xn5;
    xn0 = *x_addr(x_unit(tid), cn);
    xn1 = *x_addr(x_unit(tid + 512), cn);
    if constexpr (XPT > 1) { xn2 = *x_addr(x_unit(tid + 1024), cn); xn3 = *x_addr(x_unit(tid + 1536), cn); }
    if constexpr (XPT > 2) { xn4 = *x_addr(x_unit(tid + 2048), cn); xn5 = *x_addr(x_unit(tid + 2560), cn); }
    const uint4* xb = xs + (c & 1) * 2 * XB + h * XB;
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      if (kb + c * PK + u < ke) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 x = xb[(u * MT + mt) * 64 + lane];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mma_frag(w[u][nt], x, acc[mt][nt], T());
        }
      }
    }
    if (c + 2 < nchk) issue_w(w, c + 2);
    uint4* dst = xs + ((c + 1) & 1) * 2 * XB;
    auto put = [&](int uq, const uint4& v) __attribute__((always_inline)) {
      if (uq < 2 * XF) dst[x_slot(uq)] = v;
    };
    put(tid, xn0);
    put(tid + 512, xn1);
    if constexpr (XPT > 1) { put(tid + 1024, xn2); put(tid + 1536, xn3); }
    if constexpr (XPT > 2) { put(tid + 2048, xn4); put(tid + 2560, xn5); }
  };
  for (int c = 0; c < nchk; c += 2) {
    step(c, w0);
    if (c + 1 < nchk) step(c + 1, w1);
  }
  // range p + 4's tiles to range p's waves through LDS (the staging buffers
  // are free once every wave has passed the barrier)
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds) + (size_t)gi * MT * NT * 64 + lane;   // [4][MT][NT][64]
  if (h == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[(mt * NT + nt) * 64] = acc[mt][nt];
  }
  __syncthreads();
  if (h == 0 && gv) {
    f32x4* pp = reinterpret_cast<f32x4*>(a.part) +
                ((((size_t)blockIdx.z * 4 + p) * a.n_groups + g) * MT) * NT * 64 + lane;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pp[(mt * NT + nt) * 64] = acc[mt][nt] + red[(mt * NT + nt) * 64];
  }
}

template <typename T, int MT>
static hipError_t launch_gemm_split_mt(int NT, int epi, const GemmArgs& a, int slices, size_t lds, hipStream_t st) {
  if constexpr (sizeof(T) != 2 || MT < 2) {
    return hipErrorInvalidValue;
  } else {
    const size_t xb = (size_t)((PK * MT * 64 + 511) / 512) * 512 * 16;   // bytes per staged chunk of one range
    dim3 grid(a.n_groups, slices), block(512);
    if (a.nparts == 4) {
      // two buffers of two ranges, or the pair hand-off ([4][MT][NT][64] f32x4)
      const size_t plds = std::max((size_t)4 * xb, (size_t)4 * MT * NT * 64 * 16);
      dim3 pgrid((a.n_groups + 3) / 4, 4, slices);
      if (NT == 3) gemm_pair_kernel<T, MT, 3><<<pgrid, block, plds, st>>>(a);
      else if (NT == 2) gemm_pair_kernel<T, MT, 2><<<pgrid, block, plds, st>>>(a);
      else if (NT == 1) gemm_pair_kernel<T, MT, 1><<<pgrid, block, plds, st>>>(a);
      else return hipErrorInvalidValue;
    } else {
      dim3 pgrid((a.n_groups + 7) / 8, 8, slices);
      if (NT == 3) gemm_part_kernel<T, MT, 3><<<pgrid, block, 2 * xb, st>>>(a);
      else if (NT == 2) gemm_part_kernel<T, MT, 2><<<pgrid, block, 2 * xb, st>>>(a);
      else if (NT == 1) gemm_part_kernel<T, MT, 1><<<pgrid, block, 2 * xb, st>>>(a);
      else return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // (the normed projections take their rows' RMSNorm scales in the reduction kernel)
    if (NT == 3 && epi == E_MIXER) gemm_kernel<T, MT, 3, A_NORM, E_MIXER, 8, 0, 1, false, true><<<grid, block, lds, st>>>(a);
    else if (NT == 2 && epi == E_GELU) gemm_kernel<T, MT, 2, A_NORM, E_GELU, 8, 0, 1, false, true><<<grid, block, lds, st>>>(a);
    else if (NT == 1 && epi == E_RESID) gemm_kernel<T, MT, 1, A_ACT, E_RESID, 8, 0, 1, false, true><<<grid, block, lds, st>>>(a);
    else if (NT == 1 && epi == E_STORE) gemm_kernel<T, MT, 1, A_NORM, E_STORE, 8, 0, 1, false, true><<<grid, block, lds, st>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
}

template <typename T>
hipError_t launch_gemm_split_impl(int MT, int NT, int epi, const GemmArgs& a, int slices, size_t lds, hipStream_t st) {
  switch (MT) {
    case 2: return launch_gemm_split_mt<T, 2>(NT, epi, a, slices, lds, st);
    case 3: return launch_gemm_split_mt<T, 3>(NT, epi, a, slices, lds, st);
    case 4: return launch_gemm_split_mt<T, 4>(NT, epi, a, slices, lds, st);
    case 5: return launch_gemm_split_mt<T, 5>(NT, epi, a, slices, lds, st);
    case 6: return launch_gemm_split_mt<T, 6>(NT, epi, a, slices, lds, st);
    case 7: return launch_gemm_split_mt<T, 7>(NT, epi, a, slices, lds, st);
    case 8: return launch_gemm_split_mt<T, 8>(NT, epi, a, slices, lds, st);
    case 9: return launch_gemm_split_mt<T, 9>(NT, epi, a, slices, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MT>
static hipError_t launch_gemm_mt(int NT, int amode, int epi, const GemmArgs& a, int slices,
                                 size_t lds, hipStream_t st) {
  dim3 grid(a.n_groups, slices), block(512);
  if (NT == 3 && amode == A_NORM && epi == E_MIXER) {
    // single tile: 1-step chunks, two steps in flight (2.623 against 2.631
    // ms per round with 2-step chunks, 2.645 with 3 or 4)
    if constexpr (MT == 1) gemm_kernel<T, 1, 3, A_NORM, E_MIXER, 8, 1><<<grid, block, lds, st>>>(a);
    else gemm_kernel<T, MT, 3, A_NORM, E_MIXER><<<grid, block, lds, st>>>(a);
  } else if (NT == 1 && amode == A_ACT && epi == E_RESID)
    gemm_kernel<T, MT, 1, A_ACT, E_RESID><<<grid, block, lds, st>>>(a);
  else if (NT == 2 && amode == A_NORM && epi == E_GELU) {
    // bf16 rows of 2-4 tiles: 1-step chunks; 5-6 tiles: 2-step chunks
    // (ragged batch of 8 sequences at gamma 2 / 4 / 8 / 10: 4.270 / 4.851 /
    // 6.220 / 6.858 ms per round against 4.372 / 5.034 / 6.238 / 6.915 ms
    // with the register-bound depth; gamma 6, 4 tiles, the same either way)
    constexpr int GU_CH = (MT >= 2 && sizeof(T) == 2) ? (MT <= 4 ? 1 : 2) : 0;
    gemm_kernel<T, MT, 2, A_NORM, E_GELU, 8, GU_CH><<<grid, block, lds, st>>>(a);
  } else if (NT == 1 && amode == A_NORM && epi == E_STORE)
    gemm_kernel<T, MT, 1, A_NORM, E_STORE><<<grid, block, lds, st>>>(a);
  else if (NT == 1 && amode == A_ACT && epi == E_STORE)     // rows normalised by their producer
    gemm_kernel<T, MT, 1, A_ACT, E_STORE><<<grid, block, lds, st>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_gemm_w8_mt(int NT, int amode, int epi, const GemmArgs& a, int slices, size_t lds,
                                    hipStream_t st) {
  dim3 grid(a.n_groups, slices), block(512);
  // one row tile: 1-step chunks (two weight steps of 16 bytes per lane in
  // flight) for the in-, out- and down-projections, measured with the
  // step-major layout: 1.946 / 1.968 / 1.953 ms per round against 1.973 with
  // 3 / 4 / 4 steps; the gate/up pairs keep their 1-step chunks at 4 workgroups
  // per CU
  constexpr int CH1 = MT == 1 ? 1 : 0;
  if (NT == 3 && amode == A_NORM && epi == E_MIXER)
    gemm_kernel<bf16, MT, 3, A_NORM, E_MIXER, 8, CH1, 1, true><<<grid, block, lds, st>>>(a);
  else if (NT == 1 && amode == A_ACT && epi == E_RESID)
    gemm_kernel<bf16, MT, 1, A_ACT, E_RESID, 8, CH1, 1, true><<<grid, block, lds, st>>>(a);
  else if (NT == 2 && amode == A_NORM && epi == E_GELU) {
    // one row tile: one-step chunks within 128 VGPRs, so two workgroups share a CU
    if constexpr (MT == 1) gemm_kernel<bf16, MT, 2, A_NORM, E_GELU, 8, 1, 4, true><<<grid, block, lds, st>>>(a);
    else gemm_kernel<bf16, MT, 2, A_NORM, E_GELU, 8, 0, 1, true><<<grid, block, lds, st>>>(a);
  } else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

inline hipError_t launch_gemm_w8_impl(int MT, int NT, int amode, int epi, const GemmArgs& a, int slices,
                                      size_t lds, hipStream_t st) {
  if (!a.wscale) return hipErrorInvalidValue;
  switch (MT) {
    case 1: return launch_gemm_w8_mt<1>(NT, amode, epi, a, slices, lds, st);
    case 2: return launch_gemm_w8_mt<2>(NT, amode, epi, a, slices, lds, st);
    case 3: return launch_gemm_w8_mt<3>(NT, amode, epi, a, slices, lds, st);
    case 4: return launch_gemm_w8_mt<4>(NT, amode, epi, a, slices, lds, st);
    case 5: return launch_gemm_w8_mt<5>(NT, amode, epi, a, slices, lds, st);
    case 6: return launch_gemm_w8_mt<6>(NT, amode, epi, a, slices, lds, st);
    case 7: return launch_gemm_w8_mt<7>(NT, amode, epi, a, slices, lds, st);
    case 8: return launch_gemm_w8_mt<8>(NT, amode, epi, a, slices, lds, st);
    case 9: return launch_gemm_w8_mt<9>(NT, amode, epi, a, slices, lds, st);
    default: return hipErrorInvalidValue;
  }
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
