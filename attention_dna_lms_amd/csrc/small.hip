// Small kernels of the path: embedding gather, state commit (the rollback),
// weight packing, fills, and the fused verifier.
#include <math.h>

#include "evs_dev.h"

namespace evs {

// One residual row segment of 16 columns (row m, columns 16 tile ..): the fp32
// values into the forward's activation layout, their sum of squares (in column
// order) into the norm partials ([row][tile], nrm_ld partials per row), and for bf16 models the values in bf16, the
// operand of the normed projections.
template <typename T>
__device__ __forceinline__ void store_row16(const float (&v)[16], float* x, bf16* xb, float* nrm, int nrm_ld, int m,
                                            int tile, int K) {
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float* xr = x + act_off<St<T>::E>(m, tile * 16 + 4 * q, K);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      xr[n] = v[4 * q + n];
      ss = fmaf(v[4 * q + n], v[4 * q + n], ss);
    }
  }
  nrm[(size_t)m * nrm_ld + tile] = ss;   // row-major: a row's partials are contiguous
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 b;
#pragma unroll
      for (int n = 0; n < 8; ++n) b[n] = (bf16)v[8 * h + n];
      *reinterpret_cast<uint4*>(xb + act_off<8>(m, tile * 16 + 8 * h, K)) = __builtin_bit_cast(uint4, b);
    }
  }
}

// ---------------------------------------------------------------- embedding
// x[m, :] = E[tok[m], :] in fp32 (and bf16 for bf16 models), plus the
// per-16-column sums of squares the first RMSNorm reads. One thread per (row,
// 16-column tile). Also flags a block that would run past the context capacity.
template <typename T>
__global__ void embed_kernel(const int* __restrict__ tokens, const T* __restrict__ E, float* x, bf16* xb,
                             float* nrm, int nrm_ld, int M, int d, int V, int P, int seq0, const int* t,
                             int max_ctx, int* err) {
  const int ntile = d / 16;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * ntile) return;
  const int m = idx / ntile, tile = idx % ntile;
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {
    if (tile == 0) atomicOr(err, 1);
    tok = 0;
  }
  if (tile == 0 && m % P == 0 && t[seq0 + m / P] + P > max_ctx) atomicOr(err, 2);
  const T* e = E + (size_t)tok * d + tile * 16;
  float v[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) v[n] = to_f(e[n]);
  store_row16<T>(v, x, xb, nrm, nrm_ld, m, tile, d);
}

template <typename T>
hipError_t launch_embed(const int* tokens, const T* E, float* x, bf16* xb, float* nrm, int nrm_ld, int M, int d,
                        int V, int P, int seq0, const int* t, int max_ctx, int* err, hipStream_t st) {
  const int n = M * (d / 16);
  embed_kernel<T><<<(n + 255) / 256, 256, 0, st>>>(tokens, E, x, xb, nrm, nrm_ld, M, d, V, P, seq0, t, max_ctx,
                                                   err);
  return hipGetLastError();
}
template hipError_t launch_embed<bf16>(const int*, const bf16*, float*, bf16*, float*, int, int, int, int, int, int,
                                       const int*, int, int*, hipStream_t);
template hipError_t launch_embed<float>(const int*, const float*, float*, bf16*, float*, int, int, int, int, int,
                                        int, const int*, int, int*, hipStream_t);

// ---------------------------------------------------------------- commit
// Slice each sequence's state to its accepted boundary: the committed length
// advances by n_keep and, if anything was kept, the IIR state pointer moves to
// the buffer the block wrote and the slot of the last kept position. No state
// bytes move (Evo2 discussion #232, "What we implemented": the state is sliced
// directly to the accepted boundary).
__global__ void commit_kernel(int* t, int* ib, int* is, const int* n_keep, int n_all, int B, int P, int* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = n_keep ? n_keep[b] : n_all;
  if (n < 0 || n > P) {
    atomicOr(err, 4);
    n = n < 0 ? 0 : P;
  }
  t[b] += n;
  if (n > 0) {
    ib[b] ^= 1;
    is[b] = n - 1;
  }
}

hipError_t launch_commit(int* t, int* ib, int* is, const int* n_keep, int n_all, int B, int P, int* err,
                         hipStream_t st) {
  commit_kernel<<<(B + 255) / 256, 256, 0, st>>>(t, ib, is, n_keep, n_all, B, P, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fills / copies
__global__ void fill_i32_kernel(int* p, int v, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}
hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_i32_kernel<<<(int)blocks, 256, 0, st>>>(p, v, n);
  return hipGetLastError();
}

__global__ void copy_bytes_kernel(const unsigned char* src, unsigned char* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
hipError_t launch_copy_row(const void* src, void* dst, size_t bytes, hipStream_t st) {
  if (!bytes) return hipSuccess;
  size_t blocks = (bytes + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  copy_bytes_kernel<<<(int)blocks, 256, 0, st>>>((const unsigned char*)src, (unsigned char*)dst, bytes);
  return hipGetLastError();
}

// ---------------------------------------------------------------- packing
// Canonical row-major W [rows, K] -> MFMA fragments of 64 lanes x 16 bytes,
// stored [wave step i][group g][wave w][tile nt]: the GEMM's wave w of
// workgroup g owns steps k = w * pw + i (i < pw = ceil(steps / 8)), so at any
// moment the whole chip reads one contiguous window. Lane l of (g, k, nt)
// holds W[row][k*KSTEP + (l/16)*E .. + E-1] with row = the (l % 16)-th row of
// that tile: consecutive tiles (map_kind 0) or tile g of section nt of size
// map_stride (map_kind 1: q|k|v or gate|up kept side by side). Rows past
// rows_valid, and steps past the last (the padding of the last ranges), are
// zero.
template <typename T>
__global__ void pack_kernel(const T* __restrict__ W, uint4* __restrict__ out, int rows_valid, int K, int n_groups,
                            int NT, int map_kind, int map_stride) {
  constexpr int E = St<T>::E, KSTEP = St<T>::KSTEP;
  const int ksteps = K / KSTEP, pw = (ksteps + PACK_WAVES - 1) / PACK_WAVES;
  const long long total = (long long)pw * n_groups * PACK_WAVES * NT * 64;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    int g, k, nt, lane;
    packed_slot(idx, n_groups, NT, pw, g, k, nt, lane);
    const int r = lane % 16;
    const long long row = map_kind == 0 ? (long long)(g * NT + nt) * 16 + r : (long long)nt * map_stride + g * 16 + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < rows_valid && k < ksteps)
      v = *reinterpret_cast<const uint4*>(W + row * (long long)K + (long long)k * KSTEP + (lane / 16) * E);
    out[idx] = v;
  }
}

template <typename T>
hipError_t launch_pack(const T* W, uint4* out, int rows_valid, int K, int n_groups, int NT, int map_kind,
                       int map_stride, hipStream_t st) {
  pack_kernel<T><<<4096, 256, 0, st>>>(W, out, rows_valid, K, n_groups, NT, map_kind, map_stride);
  return hipGetLastError();
}
template hipError_t launch_pack<bf16>(const bf16*, uint4*, int, int, int, int, int, int, hipStream_t);
template hipError_t launch_pack<float>(const float*, uint4*, int, int, int, int, int, int, hipStream_t);

// ---------------------------------------------------------------- FP8 weights
// Row scales and E4M3 codes of the FP8 weight variant: row n keeps
// e4m3(W[n, k] / s[n]) with s[n] the smallest power of two such that
// max_k |W[n, k]| <= 448 * s[n] (then W / s is exact and the only rounding is
// E4M3's, to nearest with ties to even; OCP FP8 E4M3: 4 exponent bits with
// bias 7, 3 mantissa bits, largest 448, subnormals k * 2^-9).

// canonical row of packed row r of tile nt of group g (as in pack_kernel)
__device__ __forceinline__ long long packed_row(int g, int nt, int r, int NT, int map_kind, int map_stride) {
  return map_kind == 0 ? (long long)(g * NT + nt) * 16 + r : (long long)nt * map_stride + g * 16 + r;
}

// one wave per packed row: max |w| over K, then the power-of-two scale
// (from the binary exponent: max = f * 2^e, 448 = 0.875 * 2^9)
__global__ void fp8_scale_kernel(const bf16* __restrict__ W, float* __restrict__ scales, int rows_valid, int K,
                                 int n_rows, int NT, int map_kind, int map_stride) {
  const int pr = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (pr >= n_rows) return;
  const int g = pr / (NT * 16), nt = (pr / 16) % NT, r = pr % 16;
  const long long row = packed_row(g, nt, r, NT, map_kind, map_stride);
  float m = 0.f;
  if (row < rows_valid)
    for (int k = lane; k < K; k += 64) m = fmaxf(m, fabsf((float)W[row * (long long)K + k]));
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) {
    float s = 1.f;
    if (m > 0.f) {
      int e;
      const float f = frexpf(m, &e);
      s = ldexpf(1.f, f <= 0.875f ? e - 9 : e - 8);
    }
    scales[pr] = s;
  }
}

// E4M3 code of v (an exact multiple of the row scale's inverse grid): round
// |v| to a multiple of 2^max(p - 3, -9), p the exponent of its leading bit
__device__ __forceinline__ unsigned e4m3_code(float v) {
  const unsigned sign = signbit(v) ? 0x80u : 0u;
  const float a = fabsf(v);
  if (!(a > 0.f)) return sign;
  int e;
  frexpf(a, &e);                                  // a = f * 2^e, leading bit 2^(e - 1)
  const int qe = max(e - 4, -9);
  float q = rintf(ldexpf(a, -qe));                // a / 2^qe, to nearest even
  if (qe == -9 && q < 8.f) return sign | (unsigned)q;   // subnormal: exponent field 0
  int p = qe + 3;                                 // value = (q / 8) * 2^p, 8 <= q <= 16
  if (q >= 16.f) { q = 8.f; p += 1; }
  if (p > 8 || (p == 8 && q > 14.f)) return sign | 0x7Eu;   // 448 (not reached after scaling)
  return sign | (unsigned)(((p + 7) << 3) | ((int)q - 8));
}

// Weight steps of 64 k (two MFMA k-steps), in pack_kernel's slot order: lane
// l of (group g, step s, tile nt) holds the codes of W[row][64 s + 8 (l / 16)
// + j] (bytes j = 0..7) and W[row][64 s + 32 + 8 (l / 16) + j] (bytes 8 + j),
// row = packed row (g, nt, l % 16). Rows past rows_valid, and padding steps,
// are zero.
__global__ void pack_fp8_kernel(const bf16* __restrict__ W, const float* __restrict__ scales, uint4* __restrict__ out,
                                int rows_valid, int K, int n_groups, int NT, int map_kind, int map_stride) {
  const int steps = K / 64, pw = (steps + PACK_WAVES - 1) / PACK_WAVES;
  const long long total = (long long)pw * n_groups * PACK_WAVES * NT * 64;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    int g, st, nt, lane;
    packed_slot(idx, n_groups, NT, pw, g, st, nt, lane);
    const int r = lane % 16, kb = lane / 16;
    const long long row = packed_row(g, nt, r, NT, map_kind, map_stride);
    unsigned w[4] = {0u, 0u, 0u, 0u};
    if (row < rows_valid && st < steps) {
      const float inv = 1.f / scales[(g * NT + nt) * 16 + r];   // a power of two: exact
      const bf16* src = W + row * (long long)K + (long long)st * 64 + kb * 8;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float v = (float)src[(j < 8 ? 0 : 32) + (j & 7)] * inv;
        w[j >> 2] |= e4m3_code(v) << (8 * (j & 3));
      }
    }
    out[idx] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_fp8_scales(const bf16* W, float* scales, int rows_valid, int K, int n_groups, int NT,
                             int map_kind, int map_stride, hipStream_t st) {
  const int n_rows = n_groups * NT * 16;
  fp8_scale_kernel<<<(n_rows + 3) / 4, 256, 0, st>>>(W, scales, rows_valid, K, n_rows, NT, map_kind, map_stride);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const bf16* W, const float* scales, uint4* out, int rows_valid, int K, int n_groups,
                           int NT, int map_kind, int map_stride, hipStream_t st) {
  pack_fp8_kernel<<<4096, 256, 0, st>>>(W, scales, out, rows_valid, K, n_groups, NT, map_kind, map_stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------- verifier
// One workgroup per sequence, one wave per position (up to 16 positions per
// round). Target distributions (softmax over the top-k of logits / T) are built
// in parallel. Every fp32 sum a decision depends on is formed in token order,
// ((w0 + w1) + w2) + ..., so it equals a sequential evaluation exactly
// (EvSpark preprint, abstract (iii): exact rejection-sampling verification).
// Such a chain runs on one lane: the P softmax normalisers on P lanes of one
// wave side by side, the draw's running sums on one lane, written over the row
// and then searched by a wave.
//
// LDS holds the P target rows and the residual row, Vs floats apart: Vs is V
// rounded up to a multiple of 4, plus 4 when that is a multiple of 8, so the
// 16-byte reads of one column by lanes on consecutive rows fall in distinct
// banks. Entries V .. Vs-1 hold zeros, which leave a running sum unchanged.

constexpr int VERIFY_MAX_WAVES = 16;

__host__ __device__ inline int verify_row_stride(int V) {
  const int vr = (V + 3) & ~3;
  return ((vr >> 2) & 1) ? vr : vr + 4;
}

// total order used by top-k: larger value first, lower id on ties
__device__ __forceinline__ bool ord_gt(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Wave-wide reductions with every lane of the wave active: DPP steps inside
// each row of 16 lanes (lane ^ 1, lane ^ 2, then the mirrors within 8 and
// within 16 lanes, after which every lane of a row holds the row's result),
// then the four rows' results read as scalars and combined in every lane.
// The operations are exact and order-independent (a maximum in a total
// order), so the result is the same as any other reduction order.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL> __device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// The same total order as one 64-bit key per entry, so a selection step is
// one unsigned compare and a select (no short-circuit control flow): the high
// word is the value's bits made monotone (with -0 read as +0, which the
// float compare treats as equal), the low word 0xFFFFFFFF - id (a lower id is
// the larger key on ties). Key 0 is below every real entry.
typedef unsigned long long okey_t;
__device__ __forceinline__ okey_t ord_key(float v, int y) {
  const unsigned u = __float_as_uint(v + 0.f);
  const unsigned hi = u ^ ((unsigned)((int)u >> 31) | 0x80000000u);
  return ((okey_t)hi << 32) | (okey_t)(0xFFFFFFFFu - (unsigned)y);
}
__device__ __forceinline__ float key_value(okey_t k) {
  const unsigned hi = (unsigned)(k >> 32);
  return __uint_as_float(hi ^ (~(unsigned)((int)hi >> 31) | 0x80000000u));
}
__device__ __forceinline__ int key_index(okey_t k) { return (int)(0xFFFFFFFFu - (unsigned)k); }
__device__ __forceinline__ okey_t key_max(okey_t a, okey_t b) { return a > b ? a : b; }
template <int CTRL> __device__ __forceinline__ okey_t dpp_key(okey_t k) {
  const unsigned lo = (unsigned)dpp_i<CTRL>((int)(unsigned)k);
  const unsigned hi = (unsigned)dpp_i<CTRL>((int)(unsigned)(k >> 32));
  return ((okey_t)hi << 32) | lo;
}
__device__ __forceinline__ okey_t lane_key(okey_t k, int l) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)k, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(k >> 32), l);
  return ((okey_t)hi << 32) | lo;
}
// largest key of the wave, in every lane (the same row steps as wave_argmax)
__device__ __forceinline__ okey_t wave_keymax(okey_t k) {
  k = key_max(k, dpp_key<DPP_XOR1>(k));
  k = key_max(k, dpp_key<DPP_XOR2>(k));
  k = key_max(k, dpp_key<DPP_HALF_MIRROR>(k));
  k = key_max(k, dpp_key<DPP_MIRROR>(k));
  return key_max(key_max(lane_key(k, 0), lane_key(k, 16)), key_max(lane_key(k, 32), lane_key(k, 48)));
}

template <int CTRL> __device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  const float v2 = dpp_f<CTRL>(v);
  const int i2 = dpp_i<CTRL>(i);
  if (ord_gt(v2, i2, v, i)) { v = v2; i = i2; }
}

// (value, index) maximum in the total order of ord_gt, in every lane
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp<DPP_XOR1>(v, i);
  argmax_dpp<DPP_XOR2>(v, i);
  argmax_dpp<DPP_HALF_MIRROR>(v, i);
  argmax_dpp<DPP_MIRROR>(v, i);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float v2 = lane_f(v, 16 * r);
    const int i2 = __builtin_amdgcn_readlane(i, 16 * r);
    if (ord_gt(v2, i2, bv, bi)) { bv = v2; bi = i2; }
  }
  v = bv;
  i = bi;
}

// maximum of non-NaN values, in every lane
__device__ __forceinline__ float wave_fmax(float m) {
  m = fmaxf(m, dpp_f<DPP_XOR1>(m));
  m = fmaxf(m, dpp_f<DPP_XOR2>(m));
  m = fmaxf(m, dpp_f<DPP_HALF_MIRROR>(m));
  m = fmaxf(m, dpp_f<DPP_MIRROR>(m));
  return fmaxf(fmaxf(lane_f(m, 0), lane_f(m, 16)), fmaxf(lane_f(m, 32), lane_f(m, 48)));
}

// integer maximum / minimum, in every lane
__device__ __forceinline__ int wave_imax(int x) {
  x = max(x, dpp_i<DPP_XOR1>(x));
  x = max(x, dpp_i<DPP_XOR2>(x));
  x = max(x, dpp_i<DPP_HALF_MIRROR>(x));
  x = max(x, dpp_i<DPP_MIRROR>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int wave_imin(int x) {
  x = min(x, dpp_i<DPP_XOR1>(x));
  x = min(x, dpp_i<DPP_XOR2>(x));
  x = min(x, dpp_i<DPP_HALF_MIRROR>(x));
  x = min(x, dpp_i<DPP_MIRROR>(x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// LDS visibility between the lanes of one wave: a wave's LDS operations are
// performed in order, so only the compiler has to keep them in program order
// (no wait for outstanding global stores, unlike a workgroup barrier)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave over one row of V values (NaN logits already read as -inf): returns
// the argmax (lowest id among maxima); with soft, the row is replaced by the
// softmax numerators of the top_k largest of z / T (ties in the cut to the
// lower id; top_k of 0 or >= V keeps all): exp(z/T - max) for kept finite
// entries, 0 elsewhere.
__device__ int wave_target_row(float* pr, int V, float temperature, int top_k, bool soft) {
  const int lane = threadIdx.x & 63;
  // selections over ord_key keys; a NaN entry (key 0) is never selected, and
  // every lane starts from (-inf, id 0), so a row with no entry above -inf
  // gives id 0
  okey_t bk = ord_key(-INFINITY, 0);
  for (int y = lane; y < V; y += 64) {
    const float z = pr[y];
    bk = key_max(bk, isnan(z) ? 0 : ord_key(z, y));
  }
  const int bi = key_index(wave_keymax(bk));
  if (!soft) return bi;
  // z / T, then the top-k threshold (the k-th element in the total order)
  for (int y = lane; y < V; y += 64) pr[y] = pr[y] / temperature;
  const bool all = top_k <= 0 || top_k >= V;
  float tv = -INFINITY;
  int ti = V;
  if (!all) {
    // pass r: the largest key below the previous pass's; a lane with none
    // left offers (-inf, id V)
    okey_t pk = ~0ull;
    const okey_t none = ord_key(-INFINITY, V);
    for (int r = 0; r < top_k; ++r) {
      okey_t c = none;
      for (int y = lane; y < V; y += 64) {
        const float z = pr[y];
        const okey_t k = isnan(z) ? 0 : ord_key(z, y);
        c = ((k < pk) & (k > c)) ? k : c;
      }
      pk = wave_keymax(c);
    }
    tv = key_value(pk);
    ti = key_index(pk);
  }
  float m = -INFINITY;
  for (int y = lane; y < V; y += 64) {
    const float z = pr[y];
    if ((all || !ord_gt(tv, ti, z, y)) && isfinite(z)) m = fmaxf(m, z);
  }
  m = wave_fmax(m);
  for (int y = lane; y < V; y += 64) {
    const float z = pr[y];
    const bool keep = (all || !ord_gt(tv, ti, z, y)) && isfinite(z);
    pr[y] = keep ? (float)exp((double)(z - m)) : 0.f;
  }
  return bi;
}

// the sequence's [P][V] target values into rows Vs apart, 16 loads in flight
// per thread (NaN logits read as -inf, NaN probabilities as 0); the row and
// column of a thread's element advance by whole steps of blockDim elements
template <typename S>
__device__ __forceinline__ void stage_rows(const S* src, int P, int V, int Vs, bool logits, float* dst) {
  const int nt = blockDim.x, tid = threadIdx.x, n = P * V;
  const int qn = nt / V, rn = nt - qn * V;
  int r = tid / V, y = tid - r * V;
  for (int i0 = 0; i0 < n; i0 += nt * 16) {
    float zv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) zv[q] = to_f(src[min(i0 + q * nt + tid, n - 1)]);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (i0 + q * nt + tid < n) dst[r * Vs + y] = isnan(zv[q]) ? (logits ? -INFINITY : 0.f) : zv[q];
      y += rn;
      r += qn;
      if (y >= V) { y -= V; ++r; }
    }
  }
}

// Sum of row[0 .. n) in token order on the calling lane (n a multiple of 4,
// row 16-byte aligned): batches of eight 16-byte reads, then the dependent adds
__device__ __forceinline__ float row_sum(const float* row, int n) {
  const float4* r4 = reinterpret_cast<const float4*>(row);
  const int n4 = n >> 2;
  float s = 0.f;
  int j = 0;
#pragma unroll 2
  for (; j + 8 <= n4; j += 8) {
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = r4[j + k];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s = s + v[k].x;
      s = s + v[k].y;
      s = s + v[k].z;
      s = s + v[k].w;
    }
  }
  for (; j < n4; ++j) {
    const float4 v = r4[j];
    s = s + v.x;
    s = s + v.y;
    s = s + v.z;
    s = s + v.w;
  }
  return s;
}

// Running sums of row[0 .. n) in token order written over the row by the
// calling lane; returns the total (n a multiple of 4, row 16-byte aligned)
__device__ __forceinline__ float prefix_in_place(float* row, int n) {
  float4* r4 = reinterpret_cast<float4*>(row);
  const int n4 = n >> 2;
  float c = 0.f;
  int j = 0;
  for (; j + 8 <= n4; j += 8) {
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = r4[j + k];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      c = c + v[k].x;
      v[k].x = c;
      c = c + v[k].y;
      v[k].y = c;
      c = c + v[k].z;
      v[k].z = c;
      c = c + v[k].w;
      v[k].w = c;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) r4[j + k] = v[k];
  }
  for (; j < n4; ++j) {
    float4 v = r4[j];
    c = c + v.x;
    v.x = c;
    c = c + v.y;
    v.y = c;
    c = c + v.z;
    v.z = c;
    c = c + v.w;
    v.w = c;
    r4[j] = v;
  }
  return c;
}

struct DrawShared {
  float sum;
  int last, first;
};

// Inverse-CDF draw over row[0 .. V), called by the whole block: the first y
// whose running sum row[0] + ... + row[y] exceeds t, where t = u * (the row's
// sum) if scale_u, else u; if none does, the last y with row[y] > 0, else the
// fallback. The row is overwritten by its running sums; sum gets the total.
__device__ int draw_row(float* row, int V, int Vr, float u, bool scale_u, int fallback, float& sum,
                        DrawShared& sh) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    int last = -1;
    for (int y = tid; y < V; y += 64)
      if (row[y] > 0.f) last = y;
    last = wave_imax(last);
    if (tid == 0) {
      sh.last = last;
      sh.sum = prefix_in_place(row, Vr);
    }
  }
  __syncthreads();
  const float S = sh.sum;
  const float t = scale_u ? u * S : u;
  if (tid < 64) {
    int first = V;
    for (int y = tid; y < V; y += 64)
      if (row[y] > t) { first = y; break; }
    first = wave_imin(first);
    if (tid == 0) sh.first = first;
  }
  __syncthreads();
  const int first = sh.first, last = sh.last;
  sum = S;
  __syncthreads();
  return first < V ? first : (last >= 0 ? last : fallback);
}

__global__ void __launch_bounds__(64 * VERIFY_MAX_WAVES) verify_kernel(VerifyArgs a) {
  extern __shared__ float4 sm4[];
  __shared__ int amax_s[64], draft_s[64];
  __shared__ float qx_s[64], u_s[64], ssum_s[64];
  __shared__ int rej_s, nacc_s, next_s;
  __shared__ DrawShared draw_s;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nt = blockDim.x, nw = nt >> 6;
  const int gamma = a.gamma, P = gamma + 1, V = a.V;
  const int Vr = (V + 3) & ~3, Vs = verify_row_stride(V);
  const bool logits = a.kind != 3;
  float* prob = reinterpret_cast<float*>(sm4);   // [P][Vs]
  float* w = prob + (size_t)P * Vs;              // [Vs]

  // phase 0: target rows, their zero tails, the residual row's zero tail
  if (a.kind == 1)
    stage_rows(reinterpret_cast<const bf16*>(a.target) + (size_t)b * P * V, P, V, Vs, logits, prob);
  else
    stage_rows(reinterpret_cast<const float*>(a.target) + (size_t)b * P * V, P, V, Vs, logits, prob);
  for (int t = tid; t < (P + 1) * 4; t += nt) {
    const int y = V + (t & 3);
    if (y < Vs) prob[(size_t)(t >> 2) * Vs + y] = 0.f;
  }
  // the draft tokens, and in sampling mode q(x) at each drafted position and
  // the uniforms, one thread per position, so the accept scan reads only LDS
  if (tid < P) {
    if (tid < gamma) {
      int x = a.draft[(size_t)b * gamma + tid];
      if (x < 0 || x >= V) {
        if (a.err) atomicOr(a.err, 8);
        x = x < 0 ? 0 : V - 1;
      }
      draft_s[tid] = x;
      if (!a.greedy) {
        const float qx = a.q[((size_t)b * gamma + tid) * V + x];
        qx_s[tid] = isnan(qx) ? 0.f : qx;
      }
    }
    if (!a.greedy) u_s[tid] = a.u[(size_t)b * P + tid];
  }
  __syncthreads();

  // phase 1: one wave per position: the argmax, and in sampling mode over
  // logits the kept entries' exp(z/T - max) (zeros elsewhere)
  const bool soft = !a.greedy && logits;
  for (int i = wave; i < P; i += nw) {
    const int bi = wave_target_row(prob + (size_t)i * Vs, V, a.temperature, a.top_k, soft);
    if (lane == 0) amax_s[i] = bi;
  }
  __syncthreads();
  if (soft) {
    // the normalisers, lane i summing row i in token order; then p = e / S
    if (wave == 0 && lane < P) ssum_s[lane] = row_sum(prob + (size_t)lane * Vs, Vr);
    __syncthreads();
    for (int i = wave; i < P; i += nw) {
      float* pr = prob + (size_t)i * Vs;
      const float S = ssum_s[i];
      for (int y = lane; y < V; y += 64) pr[y] = (S > 0.f) ? pr[y] / S : 0.f;
    }
    __syncthreads();
  }

  // phase 2: the accept scan, one lane, stopping at the first rejection
  if (tid == 0) {
    int n_acc = gamma, nxt = -1, rej = -1;
    for (int i = 0; i < gamma; ++i) {
      const int x = draft_s[i];
      if (a.greedy) {
        if (x != amax_s[i]) { n_acc = i; nxt = amax_s[i]; break; }
      } else {
        const float px = prob[(size_t)i * Vs + x];
        const float qx = qx_s[i];
        const bool ok = qx > 0.f ? (u_s[i] < px / qx) : (px > 0.f);
        if (!ok) { n_acc = i; rej = i; break; }
      }
    }
    if (a.greedy && nxt < 0) nxt = amax_s[gamma];
    rej_s = rej;
    nacc_s = n_acc;
    next_s = nxt;
  }
  __syncthreads();
  if (a.greedy) {
    if (tid == 0) {
      a.n_acc[b] = nacc_s;
      a.next[b] = next_s;
      if (a.n_keep) a.n_keep[b] = nacc_s + 1;
    }
    return;
  }

  // phase 3: the draw, from the residual max(0, p - q) at a rejection (from p
  // when the residual sums to zero), else from the last position's p
  const int rej = rej_s;
  const float uf = u_s[gamma];
  float S;
  int nxt;
  if (rej >= 0) {
    const float* pr = prob + (size_t)rej * Vs;
    const float* qr = a.q + ((size_t)b * gamma + rej) * V;
    for (int y = tid; y < V; y += nt) {
      float qv = qr[y];
      if (isnan(qv)) qv = 0.f;
      w[y] = fmaxf(0.f, pr[y] - qv);
    }
    __syncthreads();
    nxt = draw_row(w, V, Vr, uf, true, amax_s[rej], S, draw_s);
    if (!(S > 0.f)) nxt = draw_row(prob + (size_t)rej * Vs, V, Vr, uf, false, amax_s[rej], S, draw_s);
  } else {
    nxt = draw_row(prob + (size_t)gamma * Vs, V, Vr, uf, false, amax_s[gamma], S, draw_s);
  }
  if (tid == 0) {
    a.n_acc[b] = nacc_s;
    a.next[b] = nxt;
    if (a.n_keep) a.n_keep[b] = nacc_s + 1;
  }
}

hipError_t launch_verify(const VerifyArgs& a, int B, hipStream_t st) {
  const int P = a.gamma + 1;
  const int waves = P < VERIFY_MAX_WAVES ? P : VERIFY_MAX_WAVES;
  const size_t lds = (size_t)(P + 1) * verify_row_stride(a.V) * sizeof(float);
  verify_kernel<<<B, 64 * waves, lds, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- drafter
// The drafter path around the shared block forward (EvSpark preprint, abstract
// (ii): gamma-parallel trunk, target hidden-state prefix, full-matrix Markov
// head; model card, "Drafter checkpoints": one width-1024 layer injected from
// target layer 27, any gamma' <= gamma an exact causal prefix).

// Hidden-state export: fp32 residual rows from the forward's operand-order
// layout to row-major [M, d], four columns per thread (the layout keeps runs of
// E >= 4 columns of a row contiguous).
// (rows m0 .. m0 + M - 1 of x to rows 0 .. M - 1 of dst)
template <int E>
__global__ void export_rows_kernel(const float* __restrict__ x, float* __restrict__ dst, int m0, int M, int d) {
  const int n4 = d >> 2;
  const long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (idx >= (long long)M * n4) return;
  const int m = (int)(idx / n4), c = (int)(idx % n4) * 4;
  *reinterpret_cast<float4*>(dst + (size_t)m * d + c) =
      *reinterpret_cast<const float4*>(x + act_off<E>(m0 + m, c, d));
}

template <typename T>
hipError_t launch_export_rows(const float* x, float* dst, int m0, int M, int d, hipStream_t st) {
  const long long n = (long long)M * (d / 4);
  export_rows_kernel<St<T>::E><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, dst, m0, M, d);
  return hipGetLastError();
}
template hipError_t launch_export_rows<bf16>(const float*, float*, int, int, int, hipStream_t);
template hipError_t launch_export_rows<float>(const float*, float*, int, int, int, hipStream_t);

// The residual row of block row pick[b] of each sequence (P rows per
// sequence) into row b of dst; sequences with pick[b] < 0 are skipped.
template <int E>
__global__ void export_pick_kernel(const float* __restrict__ x, float* __restrict__ dst, const int* __restrict__ pick,
                                   int P, int d) {
  const int b = blockIdx.y, r = pick[b];
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (r < 0 || c >= d) return;
  *reinterpret_cast<float4*>(dst + (size_t)b * d + c) = *reinterpret_cast<const float4*>(x + act_off<E>(b * P + r, c, d));
}

template <typename T>
hipError_t launch_export_pick(const float* x, float* dst, const int* pick, int B, int P, int d, hipStream_t st) {
  dim3 grid((d / 4 + 255) / 256, B);
  export_pick_kernel<St<T>::E><<<grid, 256, 0, st>>>(x, dst, pick, P, d);
  return hipGetLastError();
}
template hipError_t launch_export_pick<bf16>(const float*, float*, const int*, int, int, int, hipStream_t);
template hipError_t launch_export_pick<float>(const float*, float*, const int*, int, int, int, hipStream_t);

// The injected rows, normalised: sequence b's hidden row h = hidden[b,
// index[b], :] as u = h / sqrt(mean(h^2) + eps) in the storage type (the
// operand of the injection product), in the operand-order layout. One
// workgroup per row sees the whole row, so the scale is applied before the
// rounding and u does not depend on the row's overall scale. The sum of
// squares runs per 16-column tile (column order), then over the tiles in
// order. Indices out of range are clamped and flagged.
template <typename T>
__global__ void __launch_bounds__(256) inject_prep_kernel(const float* __restrict__ hidden, int rows,
                                                          const int* __restrict__ index, int K, float eps, T* u,
                                                          int* err) {
  __shared__ float tile_ss[1024];
  __shared__ float rinv_s;
  const int b = blockIdx.x, ntile = K / 16;
  int r = index ? index[b] : 0;
  if (r < 0 || r >= rows) {
    if (threadIdx.x == 0) atomicOr(err, 16);
    r = r < 0 ? 0 : rows - 1;
  }
  const float* src = hidden + ((size_t)b * rows + r) * K;
  for (int tile = threadIdx.x; tile < ntile; tile += blockDim.x) {
    float ss = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) ss = fmaf(src[tile * 16 + n], src[tile * 16 + n], ss);
    tile_ss[tile] = ss;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int tile = 0; tile < ntile; ++tile) ss += tile_ss[tile];
    rinv_s = 1.0f / sqrtf(ss / (float)K + eps);
  }
  __syncthreads();
  const float rv = rinv_s;
  for (int tile = threadIdx.x; tile < ntile; tile += blockDim.x) {
#pragma unroll
    for (int n = 0; n < 16; ++n) u[act_off<St<T>::E>(b, tile * 16 + n, K)] = from_f<T>(src[tile * 16 + n] * rv);
  }
}

template <typename T>
hipError_t launch_inject_prep(const float* hidden, int rows, const int* index, int B, int K, float eps, T* u,
                              int* err, hipStream_t st) {
  if (K % 16 || K / 16 > 1024) return hipErrorInvalidValue;
  inject_prep_kernel<T><<<B, 256, 0, st>>>(hidden, rows, index, K, eps, u, err);
  return hipGetLastError();
}
template hipError_t launch_inject_prep<bf16>(const float*, int, const int*, int, int, float, bf16*, int*, hipStream_t);
template hipError_t launch_inject_prep<float>(const float*, int, const int*, int, int, float, float*, int*,
                                              hipStream_t);

// The slot rows: x[b * gamma + i] = (embed[last_b] + pos[i]) + z[b] in fp32,
// in the forward's layout, with their per-16-column sums of squares.
template <typename T>
__global__ void slots_kernel(const T* __restrict__ E, const T* __restrict__ pos, const T* __restrict__ z,
                             const int* __restrict__ last, int B, int gamma, int d, int V, float* x, bf16* xb,
                             float* nrm, int nrm_ld, int* err) {
  const int ntile = d / 16;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * gamma * ntile) return;
  const int m = idx / ntile, tile = idx % ntile, b = m / gamma, i = m % gamma;
  int tok = last[b];
  if (tok < 0 || tok >= V) {
    if (tile == 0 && i == 0) atomicOr(err, 1);
    tok = 0;
  }
  const T* e = E + (size_t)tok * d + tile * 16;
  const T* p = pos + (size_t)i * d + tile * 16;
  const T* zz = z + (size_t)b * d + tile * 16;
  float v[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) v[c] = (to_f(e[c]) + to_f(p[c])) + to_f(zz[c]);
  store_row16<T>(v, x, xb, nrm, nrm_ld, m, tile, d);
}

template <typename T>
hipError_t launch_slots(const T* E, const T* pos, const T* z, const int* last, int B, int gamma, int d, int V,
                        float* x, bf16* xb, float* nrm, int nrm_ld, int* err, hipStream_t st) {
  const int n = B * gamma * (d / 16);
  slots_kernel<T><<<(n + 255) / 256, 256, 0, st>>>(E, pos, z, last, B, gamma, d, V, x, xb, nrm, nrm_ld, err);
  return hipGetLastError();
}
template hipError_t launch_slots<bf16>(const bf16*, const bf16*, const bf16*, const int*, int, int, int, int, float*,
                                       bf16*, float*, int, int*, hipStream_t);
template hipError_t launch_slots<float>(const float*, const float*, const float*, const int*, int, int, int, int,
                                        float*, bf16*, float*, int, int*, hipStream_t);

// Markov head and draws: one wave per sequence, the slots one after another
// (each adds the Markov row of the previous draft). Per slot: l' = fp32(l) +
// markov[prev] (NaN read as -inf) and its argmax; then q = the softmax of the
// top_k largest of z = l' / T and the draw (the argmax in greedy mode, else the
// inverse CDF of q at the slot's uniform), with the verifier's arithmetic.
// With 0 < top_k <= DRAFT_TOPK_MAX (< V) the kept entries are found by top_k
// wave passes and everything after runs on them alone, in token order: the
// other entries of q are zero, and adding a zero leaves every sequential sum
// and running sum unchanged, so the normaliser, q and the draw equal the
// full-row evaluation exactly. Otherwise the full row goes through
// wave_target_row, one lane's normaliser and draw_row.
constexpr int DRAFT_TOPK_MAX = 16;

template <typename T>
__global__ void __launch_bounds__(64) draft_kernel(DraftArgs a) {
  extern __shared__ float4 dsm4[];
  float* row = reinterpret_cast<float*>(dsm4);   // [Vr]
  __shared__ DrawShared draw_s;
  __shared__ float ssum_s;
  const int b = blockIdx.x, lane = threadIdx.x, V = a.V, Vr = (V + 3) & ~3;
  const bool sparse = a.top_k > 0 && a.top_k <= DRAFT_TOPK_MAX && a.top_k < V;
  const T* lg = reinterpret_cast<const T*>(a.logits);
  int prev = a.last[b];
  if (prev < 0 || prev >= V) {
    if (lane == 0) atomicOr(a.err, 1);
    prev = 0;
  }
  for (int i = 0; i < a.gamma; ++i) {
    const size_t ro = ((size_t)b * a.gamma + i) * V;
    const float* mk = a.markov + (size_t)prev * V;
    for (int y = lane; y < V; y += 64) {
      const float v = to_f(lg[ro + y]) + mk[y];
      row[y] = isnan(v) ? -INFINITY : v;
    }
    for (int y = V + lane; y < Vr; y += 64) row[y] = 0.f;   // the previous draw left running sums there
    wave_sync();
    const float u = a.greedy ? 0.f : a.u[(size_t)b * a.gamma + i];
    int d;
    if (sparse) {
      float bv = -INFINITY;
      int amax = 0;
      for (int y = lane; y < V; y += 64) {
        const float z = row[y];
        if (ord_gt(z, y, bv, amax)) { bv = z; amax = y; }
      }
      wave_argmax(bv, amax);
      for (int y = lane; y < V; y += 64) row[y] = row[y] / a.temperature;
      wave_sync();
      // the kept entries in value order (all lanes hold the same values)
      float kv[DRAFT_TOPK_MAX];
      int ki[DRAFT_TOPK_MAX];
      float pvv = INFINITY;
      int pii = -1;
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r) {
        kv[r] = -INFINITY;
        ki[r] = V;
        if (r < a.top_k) {
          float cv = -INFINITY;
          int ci = V;
          for (int y = lane; y < V; y += 64) {
            const float z = row[y];
            if (ord_gt(pvv, pii, z, y) && ord_gt(z, y, cv, ci)) { cv = z; ci = y; }
          }
          wave_argmax(cv, ci);
          kv[r] = cv;
          ki[r] = ci;
          pvv = cv;
          pii = ci;
        }
      }
      // softmax numerators of the finite kept entries, then token order
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r)
        if (r < a.top_k && isfinite(kv[r])) m = fmaxf(m, kv[r]);
      float e[DRAFT_TOPK_MAX];
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r)
        e[r] = (r < a.top_k && isfinite(kv[r])) ? (float)exp((double)(kv[r] - m)) : 0.f;
#pragma unroll
      for (int r = 1; r < DRAFT_TOPK_MAX; ++r)
#pragma unroll
        for (int t = DRAFT_TOPK_MAX - 1; t >= r; --t)
          if (ki[t] < ki[t - 1]) {
            const int xi = ki[t]; ki[t] = ki[t - 1]; ki[t - 1] = xi;
            const float xe = e[t]; e[t] = e[t - 1]; e[t - 1] = xe;
          }
      float S = 0.f;
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r) S = S + e[r];
      float p[DRAFT_TOPK_MAX];
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r) p[r] = (S > 0.f) ? e[r] / S : 0.f;
      if (a.q) {
        for (int y = lane; y < V; y += 64) {
          float v = 0.f;
#pragma unroll
          for (int r = 0; r < DRAFT_TOPK_MAX; ++r) v = (ki[r] == y) ? p[r] : v;
          a.q[ro + y] = v;
        }
      }
      d = amax;
      if (!a.greedy) {
        // first kept entry (token order) whose running sum exceeds u; with a
        // negative u that is token 0 (the running sum starts at 0)
        int hit = -1, last = -1;
        float c = 0.f;
#pragma unroll
        for (int r = 0; r < DRAFT_TOPK_MAX; ++r) {
          if (ki[r] < V) {
            c = c + p[r];
            if (p[r] > 0.f) last = ki[r];
            if (hit < 0 && c > u) hit = ki[r];
          }
        }
        d = u < 0.f ? 0 : (hit >= 0 ? hit : (last >= 0 ? last : amax));
      }
    } else {
      const int amax = wave_target_row(row, V, a.temperature, a.top_k, true);
      wave_sync();
      if (lane == 0) ssum_s = row_sum(row, Vr);
      wave_sync();
      const float S = ssum_s;
      for (int y = lane; y < V; y += 64) {
        const float pv = (S > 0.f) ? row[y] / S : 0.f;
        row[y] = pv;
        if (a.q) a.q[ro + y] = pv;
      }
      wave_sync();
      d = amax;
      if (!a.greedy) {
        float tot;
        d = draw_row(row, V, Vr, u, false, amax, tot, draw_s);
      }
    }
    if (lane == 0) a.drafts[(size_t)b * a.gamma + i] = d;
    prev = d;
    wave_sync();
  }
}

// The same computation for V <= 64 * NPL with each lane's NPL entries (tokens
// lane + 64 k) held in registers: both rows are loaded NPL-wide at once, and
// the argmax, the top-k passes, the exps and q need no LDS round trips. The
// sequential sums of the full-row path still go through LDS (one lane walks
// the row in token order); the kept-set path needs none.
template <typename T, int NPL>
__global__ void __launch_bounds__(64) draft_reg_kernel(DraftArgs a) {
  extern __shared__ float4 dsm4[];
  float* row = reinterpret_cast<float*>(dsm4);   // [Vr] (full-row path)
  __shared__ DrawShared draw_s;
  __shared__ float ssum_s;
  const int b = blockIdx.x, lane = threadIdx.x, V = a.V, Vr = (V + 3) & ~3;
  const bool sparse = a.top_k > 0 && a.top_k <= DRAFT_TOPK_MAX && a.top_k < V;
  const bool all = a.top_k <= 0 || a.top_k >= V;
  const T* lg = reinterpret_cast<const T*>(a.logits);
  int prev = a.last[b];
  if (prev < 0 || prev >= V) {
    if (lane == 0) atomicOr(a.err, 1);
    prev = 0;
  }
  for (int i = 0; i < a.gamma; ++i) {
    const size_t ro = ((size_t)b * a.gamma + i) * V;
    const float* mk = a.markov + (size_t)prev * V;
    float lv[NPL], mv[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int y = min(lane + 64 * k, V - 1);
      lv[k] = to_f(lg[ro + y]);
      mv[k] = mk[y];
    }
    // l' (NaN read as -inf) and its argmax; entries past V never win
    float l[NPL];
    okey_t ak = 0;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int y = lane + 64 * k;
      const float v = lv[k] + mv[k];
      l[k] = isnan(v) ? -INFINITY : v;
      ak = key_max(ak, y < V ? ord_key(l[k], y) : 0);
    }
    const int amax = key_index(wave_keymax(ak));
    float z[NPL];
    okey_t zk[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int y = lane + 64 * k;
      z[k] = l[k] / a.temperature;
      // (a NaN z, which a finite temperature cannot produce, would never be
      // kept, as in the verifier's top-k passes)
      zk[k] = (y < V && !isnan(z[k])) ? ord_key(z[k], y) : 0;
    }
    // the top-k cut: top_k passes in the total order (kept entries in value order)
    float kv[DRAFT_TOPK_MAX];
    int ki[DRAFT_TOPK_MAX];
    float tv = -INFINITY;
    int ti = V;
    {
      // pass r: the largest key below the previous pass's (all keys first)
      okey_t pk = ~0ull;
      const int passes = all ? 0 : a.top_k;
      for (int r = 0; r < passes; ++r) {
        okey_t c = 0;
#pragma unroll
        for (int k = 0; k < NPL; ++k) c = ((zk[k] < pk) & (zk[k] > c)) ? zk[k] : c;
        // the same in every lane (scalar registers), so the work on the kept
        // entries below branches uniformly
        pk = wave_keymax(c);
        if (sparse) {
          const float pvv = key_value(pk);
          const int pii = key_index(pk);
#pragma unroll
          for (int rr = 0; rr < DRAFT_TOPK_MAX; ++rr)
            if (rr == r) { kv[rr] = pvv; ki[rr] = pii; }
        }
      }
      tv = passes > 0 ? key_value(pk) : INFINITY;
      ti = passes > 0 ? key_index(pk) : -1;
    }
    const float u = a.greedy ? 0.f : a.u[(size_t)b * a.gamma + i];
    int d = amax;
    if (sparse) {
      // the first top_k entries only (uniform guards: the rest is skipped)
      const int K = a.top_k;
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r)
        if (r < K && isfinite(kv[r])) m = fmaxf(m, kv[r]);
      // in groups of four independent exps (one uniform guard per group)
      float e[DRAFT_TOPK_MAX];
#pragma unroll
      for (int g = 0; g < DRAFT_TOPK_MAX; g += 4) {
#pragma unroll
        for (int r = g; r < g + 4; ++r) e[r] = 0.f;
        if (g < K) {
#pragma unroll
          for (int r = g; r < g + 4; ++r) {
            const bool ok = r < K && isfinite(kv[r]);
            const float x = (float)exp((double)(ok ? kv[r] - m : 0.f));
            e[r] = ok ? x : 0.f;
          }
        }
      }
      // token order (insertion by index among the first K)
#pragma unroll
      for (int r = 1; r < DRAFT_TOPK_MAX; ++r) {
        if (r < K) {
#pragma unroll
          for (int t = r; t > 0; --t)
            if (ki[t] < ki[t - 1]) {
              const int xi = ki[t]; ki[t] = ki[t - 1]; ki[t - 1] = xi;
              const float xe = e[t]; e[t] = e[t - 1]; e[t - 1] = xe;
            }
        }
      }
      float S = 0.f;
#pragma unroll
      for (int r = 0; r < DRAFT_TOPK_MAX; ++r)
        if (r < K) S = S + e[r];
      float p[DRAFT_TOPK_MAX];
      const float Sd = S > 0.f ? S : 1.f;
#pragma unroll
      for (int g = 0; g < DRAFT_TOPK_MAX; g += 4) {
#pragma unroll
        for (int r = g; r < g + 4; ++r) p[r] = 0.f;
        if (g < K) {
#pragma unroll
          for (int r = g; r < g + 4; ++r) {
            const float x = e[r] / Sd;
            p[r] = (r < K && S > 0.f) ? x : 0.f;
          }
        }
      }
      if (a.q) {
        float v[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) v[k] = 0.f;
#pragma unroll
        for (int r = 0; r < DRAFT_TOPK_MAX; ++r) {
          if (r < K) {
            // kept entry r lives in lane ki % 64, register ki / 64
#pragma unroll
            for (int k = 0; k < NPL; ++k)
              if (ki[r] == lane + 64 * k) v[k] = p[r];
          }
        }
#pragma unroll
        for (int k = 0; k < NPL; ++k)
          if (lane + 64 * k < V) a.q[ro + lane + 64 * k] = v[k];
      }
      if (!a.greedy) {
        int hit = -1, last = -1;
        float c = 0.f;
#pragma unroll
        for (int r = 0; r < DRAFT_TOPK_MAX; ++r) {
          if (r < K) {
            c = c + p[r];
            if (p[r] > 0.f) last = ki[r];
            if (hit < 0 && c > u) hit = ki[r];
          }
        }
        d = u < 0.f ? 0 : (hit >= 0 ? hit : (last >= 0 ? last : amax));
      }
    } else {
      // kept entries' exp(z - max) in registers, then the row through LDS for
      // the sequential normaliser and the draw
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < NPL; ++k) {
        const int y = lane + 64 * k;
        if (y < V && (all || !ord_gt(tv, ti, z[k], y)) && isfinite(z[k])) m = fmaxf(m, z[k]);
      }
      m = wave_fmax(m);
#pragma unroll
      for (int k = 0; k < NPL; ++k) {
        const int y = lane + 64 * k;
        const bool keep = y < V && (all || !ord_gt(tv, ti, z[k], y)) && isfinite(z[k]);
        if (y < Vr) row[y] = keep ? (float)exp((double)(z[k] - m)) : 0.f;
      }
      wave_sync();
      if (lane == 0) ssum_s = row_sum(row, Vr);
      wave_sync();
      const float S = ssum_s;
#pragma unroll
      for (int k = 0; k < NPL; ++k) {
        const int y = lane + 64 * k;
        if (y < V) {
          const float pv = (S > 0.f) ? row[y] / S : 0.f;
          row[y] = pv;
          if (a.q) a.q[ro + y] = pv;
        }
      }
      wave_sync();
      if (!a.greedy) {
        float tot;
        d = draw_row(row, V, Vr, u, false, amax, tot, draw_s);
      }
    }
    if (lane == 0) a.drafts[(size_t)b * a.gamma + i] = d;
    prev = d;
    wave_sync();
  }
}

template <typename T>
hipError_t launch_draft(const DraftArgs& a, int B, hipStream_t st) {
  const size_t lds = (size_t)((a.V + 3) & ~3) * sizeof(float);
  if (a.V <= 512)
    draft_reg_kernel<T, 8><<<B, 64, lds, st>>>(a);
  else
    draft_kernel<T><<<B, 64, lds, st>>>(a);
  return hipGetLastError();
}
template hipError_t launch_draft<bf16>(const DraftArgs&, int, hipStream_t);
template hipError_t launch_draft<float>(const DraftArgs&, int, hipStream_t);

}  // namespace evs
