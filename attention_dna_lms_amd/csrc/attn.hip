// Block-causal attention over the append-only KV cache for the gamma+1
// candidate queries of a block (Evo2 discussion #232, "The systems problem":
// attention state is an append-only KV cache; the block's own K/V rows were
// appended by the in-projection epilogue before this kernel runs).
//
// Query p of a sequence sits at position t+p and sees keys 0 .. t+p. The keys
// are split into S contiguous ranges of LS keys (LS and S depend only on the
// cache capacity, never on the block); workgroup j of a (sequence, query tile,
// head) takes range j. Inside it wave w takes the 16-key tiles w, w+4, w+8, ...
// with the next tile's loads in flight while the current one computes; each
// wave keeps an online softmax in fp32 and the
// waves merge in order; a second small kernel merges the S workgroup
// partials of each (sequence, query tile, head) in range order. Masked keys
// contribute exact zeros, so a query's result does not depend on how many
// other queries share the block.
//
// K rows are [key][Dh]; V is stored in blocks of 16 keys, each block
// dimension-major ([Dh][16 keys], 4 KB contiguous for bf16 at Dh = 128), so
// both MFMA operands load as contiguous runs: S^T = K q^T puts the 4 keys a
// lane needs for the P V product in its own registers, and a tile's values
// are one block.
#include "evs_dev.h"

namespace evs {

// four consecutive keys of one head dimension inside a value block
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
  const int k0 = j * a.LS, k1 = min(k0 + a.LS, kv_len);   // this workgroup's keys

  const T* qm = reinterpret_cast<const T*>(a.q);
  uint4 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *reinterpret_cast<const uint4*>(qm + act_off<E>(bl * P + pe, h * DH + ks * KSTEP + g * E, a.d));

  const T* K = reinterpret_cast<const T*>(a.kc) + (size_t)b * a.kv_bs + (size_t)h * a.cap * DH;
  const T* Vt = reinterpret_cast<const T*>(a.vt) + (size_t)b * a.kv_bs + (size_t)h * DH * a.cap;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's tiles: key0 = k0 + 16 * (wave + 4 * i), i = 0 .. ntile-1,
  // two tiles in flight (double buffer). Tiles past the last re-read the last
  // tile (always inside the cache) and are skipped.
  const int nt_all = (k1 > k0) ? (k1 - k0 + 15) / 16 : 0;
  const int ntile = nt_all > wave ? (nt_all - wave + 3) / 4 : 0;
  auto tile_key = [&](int i) { return k0 + 16 * (wave + 4 * min(i, max(ntile - 1, 0))); };
  struct Buf { uint4 kf[NKS]; VQuad<T> vf[NDT]; };
  auto issue = [&](Buf& bf, int i) {
    const int key0 = ntile > 0 ? tile_key(i) : 0;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      bf.kf[ks] = *reinterpret_cast<const uint4*>(K + (size_t)(key0 + qc) * DH + ks * KSTEP + g * E);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) bf.vf[dt].load(Vt + (size_t)key0 * DH + (dt * 16 + qc) * 16 + 4 * g);
  };
  auto compute = [&](const Buf& bf, int i) {
    const int key0 = tile_key(i);
    // S^T tile: rows = keys key0 .. key0+15, columns = the 16 queries
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sc = mma_frag(bf.kf[ks], qf[ks], sc, T());
    // lane holds scores of keys key0 + 4g + q for query qc
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int key = key0 + 4 * g + q;
      sv[q] = (key <= qpos && key < k1) ? sc[q] * a.scale : -INFINITY;
      mt = fmaxf(mt, sv[q]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = (m_new == -INFINITY) ? 1.f : expf(m_run - m_new);
    float pv[4];
    float ls = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pv[q] = (sv[q] == -INFINITY) ? 0.f : expf(sv[q] - m_new);
      ls += pv[q];
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
      for (int q = 0; q < 4; ++q) va[q] = (key0 + 4 * g + q < k1) ? bf.vf[dt].get(q) : 0.f;
      o[dt] = o[dt] * alpha;
      o[dt] = mma_k4(va, pv, o[dt], T());
    }
  };
  Buf b0, b1;
  issue(b0, 0);
  issue(b1, 1);
  {
    int i = 0;
    for (; i + 3 < ntile; i += 2) {
      compute(b0, i);
      __builtin_amdgcn_sched_barrier(0);
      issue(b0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b1, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(b1, i + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ntile - i == 3) {
      compute(b0, i);
      __builtin_amdgcn_sched_barrier(0);
      issue(b0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b1, i + 1);
      compute(b0, i + 2);
    } else if (ntile - i == 2) {
      compute(b0, i);
      compute(b1, i + 1);
    } else if (ntile - i == 1) {
      compute(b0, i);
    }
  }

  // merge the 4 waves (fixed order) into this workgroup's partial
  if (g == 0) { wm[wave][qc] = m_run; wl[wave][qc] = l_run; }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) wo[wave][qc][dt * 16 + 4 * g + q] = o[dt][q];
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

// bf16 models: the same schedule with 32-key tiles, so every K and V load is a
// full 16-byte-per-lane (1 KB) vector and both products use the 16x16x32 MFMA.
// The two S^T products of a tile take their key rows in the order
// 8 * (r / 4) + 4 * half + r % 4 (r = MFMA row), which leaves lane (query q,
// group g) holding the probabilities of keys 8g .. 8g+7: exactly its P^T
// operand of O^T += V^T P^T, whose V^T operand (head dimension e, keys 8g ..
// 8g+7) is 16 contiguous bytes of a 16-key value block.
// QG query tiles share one pass over the keys (a block of 17-32 positions
// reads the cache once); every query's arithmetic is the same whatever tiles
// share the pass. Tiles past the block's last (an odd tile count) repeat the
// last query and are not stored.
template <int DH, int QG>
__global__ void __launch_bounds__(256, 2) attn32_kernel(AttnArgs a) {
  using T = bf16;
  constexpr int E = 8, KSTEP = 32, NKS = DH / KSTEP, NDT = DH / 16;
  constexpr int ROW = DH + 2;
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float wo[4][16][DH];

  const int j = blockIdx.x, h = blockIdx.y;
  const int NG = (a.QTN + QG - 1) / QG;          // tile groups per sequence
  const int bl = blockIdx.z / NG, qt0 = (blockIdx.z % NG) * QG;
  const int b = a.seq0 + bl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qc = lane & 15, g = lane >> 4;
  const int t = a.t[b], P = a.P;
  const int kv_len = min(t + P, a.cap);
  const int k0 = j * a.LS, k1 = min(k0 + a.LS, kv_len);   // this workgroup's keys

  const T* qm = reinterpret_cast<const T*>(a.q);
  uint4 qf[QG][NKS];
  int qpos[QG];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const int pe = min((qt0 + u) * 16 + qc, P - 1);   // padding queries repeat the last real one
    qpos[u] = t + pe;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[u][ks] = *reinterpret_cast<const uint4*>(qm + act_off<E>(bl * P + pe, h * DH + ks * KSTEP + g * E, a.d));
  }

  const T* K = reinterpret_cast<const T*>(a.kc) + (size_t)b * a.kv_bs + (size_t)h * a.cap * DH;
  const T* Vb = reinterpret_cast<const T*>(a.vt) + (size_t)b * a.kv_bs + (size_t)h * DH * a.cap;

  float m_run[QG], l_run[QG];
  f32x4 o[QG][NDT];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // this wave's tiles: key0 = k0 + 32 * (wave + 4 * i). One tile buffer,
  // refilled as soon as it is consumed: the next tile's K loads go out right
  // after this tile's S^T products, its V loads right after the P V products.
  // Tiles past the last re-read the last one (inside the cache: the capacity
  // is a multiple of 32) and are never used.
  const int nt_all = (k1 > k0) ? (k1 - k0 + 31) / 32 : 0;
  const int ntile = nt_all > wave ? (nt_all - wave + 3) / 4 : 0;
  auto tile_key = [&](int i) { return k0 + 32 * (wave + 4 * min(i, max(ntile - 1, 0))); };
  const int krow = 8 * (qc >> 2) + (qc & 3);   // key of MFMA row qc in the first half
  uint4 kf[2][NKS], vf[NDT];
  auto issue_k = [&](int i) {
    const int key0 = ntile > 0 ? tile_key(i) : 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[hf][ks] = *reinterpret_cast<const uint4*>(K + (size_t)(key0 + krow + 4 * hf) * DH + ks * KSTEP + g * E);
  };
  auto issue_v = [&](int i) {
    const int key0 = ntile > 0 ? tile_key(i) : 0;
    const T* vb = Vb + (size_t)(key0 / 16 + (g >> 1)) * (DH * 16) + 8 * (g & 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vf[dt] = *reinterpret_cast<const uint4*>(vb + (dt * 16 + qc) * 16);
  };
  issue_k(0);
  issue_v(0);
  for (int i = 0; i < ntile; ++i) {
    const int key0 = tile_key(i);
    f32x4 sc[QG][2];
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      sc[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sc[u][0] = mma_frag(kf[0][ks], qf[u][ks], sc[u][0], T());
        sc[u][1] = mma_frag(kf[1][ks], qf[u][ks], sc[u][1], T());
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_k(i + 1);
    __builtin_amdgcn_sched_barrier(0);
    // lane holds the scores of keys key0 + 8g + 4 * half + r (r < 4) for query qc
    const int kb = key0 + 8 * g;
    uint4 pu[QG];
    float alpha[QG];
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      float sv[8];
      float mt = -INFINITY;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int key = kb + q;
        sv[q] = (key <= qpos[u] && key < k1) ? sc[u][q >> 2][q & 3] * a.scale : -INFINITY;
        mt = fmaxf(mt, sv[q]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run[u], mt);
      alpha[u] = (m_new == -INFINITY) ? 1.f : expf(m_run[u] - m_new);
      float ls = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float pv = (sv[q] == -INFINITY) ? 0.f : expf(sv[q] - m_new);
        ls += pv;
        pb[q] = (bf16)pv;
      }
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      l_run[u] = l_run[u] * alpha[u] + ls;
      m_run[u] = m_new;
      pu[u] = __builtin_bit_cast(uint4, pb);
    }
    // values of keys past this workgroup's range are zeroed (the cache rows
    // there may hold anything, and 0 * NaN is NaN)
    if (kb + 8 > k1) {
      const int nv = max(0, min(8, k1 - kb));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        unsigned w[4] = {vf[dt].x, vf[dt].y, vf[dt].z, vf[dt].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (2 * q >= nv) w[q] = 0u;
          else if (2 * q + 1 >= nv) w[q] &= 0xffffu;
        }
        vf[dt] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    // O^T += V^T P^T: A rows = head dims, B columns = queries, k = the tile's keys
#pragma unroll
    for (int u = 0; u < QG; ++u)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        o[u][dt] = o[u][dt] * alpha[u];
        o[u][dt] = mma_frag(vf[dt], pu[u], o[u][dt], T());
      }
    __builtin_amdgcn_sched_barrier(0);
    issue_v(i + 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // merge the 4 waves (fixed order) into this workgroup's partial, one query
  // tile at a time
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const int qt = qt0 + u;
    if (qt >= a.QTN) break;   // uniform: an odd tile count's padding tile
    if (u > 0) __syncthreads();   // the previous tile's merge has read the buffers
    if (g == 0) { wm[wave][qc] = m_run[u]; wl[wave][qc] = l_run[u]; }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) wo[wave][qc][dt * 16 + 4 * g + q] = o[u][dt][q];
    __syncthreads();
    const size_t head = ((size_t)bl * a.QTN + qt) * a.H + h;
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
}

// Merge the S split partials of each (sequence, query tile, head) in range
// order: one thread per (query, head dimension), all of a thread's partial
// loads in flight together. A separate launch, so the partials are visible by
// kernel ordering alone.
template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnArgs a) {
  constexpr int ROW = DH + 2, SB = 16;
  const int e = blockIdx.x * 16 + (threadIdx.x & 15), q = threadIdx.x >> 4;
  const int h = blockIdx.y;
  const int bl = blockIdx.z / a.QTN, qt = blockIdx.z % a.QTN;
  if (qt * 16 + q >= a.P) return;
  const size_t head = (size_t)blockIdx.z * a.H + h;
  const float* part = a.part + head * a.S * 16 * ROW + (size_t)q * ROW;   // split s at part[s * 16 * ROW]
  float M = -INFINITY;
  for (int s0 = 0; s0 < a.S; s0 += SB) {
    float mv[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) mv[u] = part[(size_t)min(s0 + u, a.S - 1) * 16 * ROW + DH];
#pragma unroll
    for (int u = 0; u < SB; ++u) M = fmaxf(M, mv[u]);
  }
  float L = 0.f, v = 0.f;
  for (int s0 = 0; s0 < a.S; s0 += SB) {
    float mv[SB], lv[SB], pv[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float* ps = part + (size_t)min(s0 + u, a.S - 1) * 16 * ROW;
      mv[u] = ps[DH];
      lv[u] = ps[DH + 1];
      pv[u] = ps[e];
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      if (s0 + u < a.S) {
        const float f = (mv[u] == -INFINITY) ? 0.f : expf(mv[u] - M);
        L += lv[u] * f;
        v += pv[u] * f;
      }
    }
  }
  T* out = reinterpret_cast<T*>(a.out);
  out[act_off<St<T>::E>(bl * a.P + qt * 16 + q, h * DH + e, a.d)] = from_f<T>(v / L);
}

template <typename T>
hipError_t launch_attn(const AttnArgs& a, int n_seq, hipStream_t st) {
  // whole 16-key tiles per range (32-key tiles for bf16: the capacity is a
  // multiple of 256, so a range's last tile stays inside the cache)
  if (a.S > 64 || a.S < 1 || a.LS < 16 || a.LS % 16 || a.cap % 256) return hipErrorInvalidValue;
  dim3 grid(a.S, a.H, n_seq * a.QTN), block(256), mgrid(a.Dh / 16, a.H, n_seq * a.QTN);
  // bf16: query tiles in pairs (grid z = sequence x tile pair)
  dim3 grid2(a.S, a.H, n_seq * ((a.QTN + 1) / 2));
  constexpr bool B16 = sizeof(T) == 2;
  const bool pair = a.QTN >= 2;
  switch (a.Dh) {
    case 32:
      if constexpr (B16) {
        if (pair) attn32_kernel<32, 2><<<grid2, block, 0, st>>>(a); else attn32_kernel<32, 1><<<grid, block, 0, st>>>(a);
      } else {
        attn_kernel<T, 32><<<grid, block, 0, st>>>(a);
      }
      attn_merge_kernel<T, 32><<<mgrid, block, 0, st>>>(a);
      break;
    case 64:
      if constexpr (B16) {
        if (pair) attn32_kernel<64, 2><<<grid2, block, 0, st>>>(a); else attn32_kernel<64, 1><<<grid, block, 0, st>>>(a);
      } else {
        attn_kernel<T, 64><<<grid, block, 0, st>>>(a);
      }
      attn_merge_kernel<T, 64><<<mgrid, block, 0, st>>>(a);
      break;
    case 128:
      if constexpr (B16) {
        if (pair) attn32_kernel<128, 2><<<grid2, block, 0, st>>>(a); else attn32_kernel<128, 1><<<grid, block, 0, st>>>(a);
      } else {
        attn_kernel<T, 128><<<grid, block, 0, st>>>(a);
      }
      attn_merge_kernel<T, 128><<<mgrid, block, 0, st>>>(a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_attn<bf16>(const AttnArgs&, int, hipStream_t);
template hipError_t launch_attn<float>(const AttnArgs&, int, hipStream_t);

}  // namespace evs
