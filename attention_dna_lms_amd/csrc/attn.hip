// Block-causal attention over the append-only KV cache for the gamma+1
// candidate queries of a block (Evo2 discussion #232, "The systems problem":
// attention state is an append-only KV cache; the block's own K/V rows were
// appended by the in-projection epilogue before this kernel runs).
//
// Query p of a sequence sits at position t+p and sees keys 0 .. t+p. The work
// is split over keys: chunk c holds keys [256c, 256c+256) and workgroup j of a
// (sequence, query tile, head) visits chunks j, j+S, j+2S, ...; inside a chunk
// wave w takes key tiles 4w .. 4w+3. Each wave keeps an online softmax in fp32,
// waves merge in order inside the workgroup, and a second small kernel merges
// the S workgroup partials in order. Every split boundary sits at an
// absolute key position and masked keys contribute exact zeros, so a query's
// result does not depend on how many other queries share the block.
//
// K rows are [key][Dh]; V rows are stored transposed ([Dh][key]) so both
// MFMA operands load as contiguous vectors: S^T = K q^T puts the 4 keys a lane
// needs for the P V product in its own registers.
#include "evs_dev.h"

namespace evs {

// four consecutive keys of one transposed value row
template <typename T> struct VQuad;
template <> struct VQuad<bf16> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float get(int i) const {
    const unsigned w = i < 2 ? v.x : v.y;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct VQuad<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float get(int i) const { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
};

template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP, NKS = DH / KSTEP, NDT = DH / 16;
  constexpr int ROW = DH + 2;
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float wo[4][16][DH];

  const int j = blockIdx.x, h = blockIdx.y;
  const int bl = blockIdx.z / a.QTN, qt = blockIdx.z % a.QTN;
  const int b = a.seq0 + bl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qc = lane & 15, g = lane >> 4;
  const int t = a.t[b], P = a.P;
  const int kv_len = min(t + P, a.cap);
  const int pe = min(qt * 16 + qc, P - 1);   // padding queries repeat the last real one
  const int qpos = t + pe;

  const T* qrow = reinterpret_cast<const T*>(a.q) + (size_t)(bl * P + pe) * a.d + h * DH;
  uint4 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(qrow + ks * KSTEP + g * E);

  const T* K = reinterpret_cast<const T*>(a.kc) + (size_t)b * a.kv_bs + (size_t)h * a.cap * DH;
  const T* Vt = reinterpret_cast<const T*>(a.vt) + (size_t)b * a.kv_bs + (size_t)h * DH * a.cap;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = j; c * ATTN_CHUNK < kv_len; c += a.S) {
    const int kw = c * ATTN_CHUNK + wave * 64;   // this wave's 4 key tiles
    if (kw >= kv_len) continue;
    // the loads of two tiles go out together; keys past kv_len are read (they
    // lie inside the cache, which is a whole number of chunks) and masked
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kh = kw + half * 32;
      if (kh >= kv_len) break;
      uint4 kf[2][NKS];
      VQuad<T> vf[2][NDT];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int key0 = kh + tt * 16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          kf[tt][ks] = *reinterpret_cast<const uint4*>(K + (size_t)(key0 + qc) * DH + ks * KSTEP + g * E);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vf[tt][dt].load(Vt + (size_t)(dt * 16 + qc) * a.cap + key0 + 4 * g);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int key0 = kh + tt * 16;
        if (key0 >= kv_len) break;
        // S^T tile: rows = keys key0 .. key0+15, columns = the 16 queries
        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sc = mma_frag(kf[tt][ks], qf[ks], sc, T());
        // lane holds scores of keys key0 + 4g + i for query qc
        float sv[4];
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 4 * g + i;
          sv[i] = (key <= qpos) ? sc[i] * a.scale : -INFINITY;
          mt = fmaxf(mt, sv[i]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : expf(m_run - m_new);
        float pv[4];
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = (sv[i] == -INFINITY) ? 0.f : expf(sv[i] - m_new);
          ls += pv[i];
        }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        l_run = l_run * alpha + ls;
        m_run = m_new;
        // O^T += V^T P^T: A rows = head dims, B columns = queries, slots = keys
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          float va[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) va[i] = (key0 + 4 * g + i < kv_len) ? vf[tt][dt].get(i) : 0.f;
          o[dt] = o[dt] * alpha;
          o[dt] = mma_k4(va, pv, o[dt], T());
        }
      }
    }
  }

  // merge the 4 waves (fixed order) into this workgroup's partial
  if (g == 0) { wm[wave][qc] = m_run; wl[wave][qc] = l_run; }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wo[wave][qc][dt * 16 + 4 * g + i] = o[dt][i];
  __syncthreads();
  const size_t head = (size_t)blockIdx.z * a.H + h;
  float* part = a.part + head * a.S * 16 * ROW;
  for (int idx = tid; idx < 16 * ROW; idx += 256) {
    const int q = idx / ROW, e = idx % ROW;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][q]);
    float v = 0.f;
    if (e == DH) {
      v = M;
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = (wm[w][q] == -INFINITY) ? 0.f : expf(wm[w][q] - M);
        v += (e < DH ? wo[w][q][e] : wl[w][q]) * f;
      }
    }
    part[((size_t)j * 16 + q) * ROW + e] = v;
  }
}

// Merge the S workgroup partials of one (sequence, query tile, head) in split
// order and write the normalised output rows. A separate launch, so the
// partials are visible by kernel ordering alone.
template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  constexpr int ROW = DH + 2;
  __shared__ float fac[64][16];
  __shared__ float fl[16];
  const int h = blockIdx.x;
  const int bl = blockIdx.y / a.QTN, qt = blockIdx.y % a.QTN;
  const int tid = threadIdx.x, P = a.P;
  const size_t head = (size_t)blockIdx.y * a.H + h;
  const float* part = a.part + head * a.S * 16 * ROW;
  if (tid < 16) {
    const int q = tid;
    float M = -INFINITY;
    for (int s = 0; s < a.S; ++s) M = fmaxf(M, part[((size_t)s * 16 + q) * ROW + DH]);
    float L = 0.f;
    for (int s = 0; s < a.S; ++s) {
      const float ms = part[((size_t)s * 16 + q) * ROW + DH];
      const float f = (ms == -INFINITY) ? 0.f : expf(ms - M);
      fac[s][q] = f;
      L += part[((size_t)s * 16 + q) * ROW + DH + 1] * f;
    }
    fl[q] = L;
  }
  __syncthreads();
  T* out = reinterpret_cast<T*>(a.out);
  for (int idx = tid; idx < 16 * DH; idx += 256) {
    const int q = idx / DH, e = idx % DH;
    if (qt * 16 + q >= P) continue;
    float v = 0.f;
    for (int s = 0; s < a.S; ++s) v += part[((size_t)s * 16 + q) * ROW + e] * fac[s][q];
    out[(size_t)(bl * P + qt * 16 + q) * a.d + h * DH + e] = from_f<T>(v / fl[q]);
  }
}

template <typename T>
hipError_t launch_attn(const AttnArgs& a, int n_seq, hipStream_t st) {
  if (a.S > 64 || a.S < 1) return hipErrorInvalidValue;
  dim3 grid(a.S, a.H, n_seq * a.QTN), block(256), cgrid(a.H, n_seq * a.QTN);
  switch (a.Dh) {
    case 32: attn_kernel<T, 32><<<grid, block, 0, st>>>(a); attn_combine_kernel<T, 32><<<cgrid, block, 0, st>>>(a); break;
    case 64: attn_kernel<T, 64><<<grid, block, 0, st>>>(a); attn_combine_kernel<T, 64><<<cgrid, block, 0, st>>>(a); break;
    case 128: attn_kernel<T, 128><<<grid, block, 0, st>>>(a); attn_combine_kernel<T, 128><<<cgrid, block, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_attn<bf16>(const AttnArgs&, int, hipStream_t);
template hipError_t launch_attn<float>(const AttnArgs&, int, hipStream_t);

}  // namespace evs
