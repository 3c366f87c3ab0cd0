// Device-side types, MFMA fragments and kernel argument blocks shared by the
// HIP kernels of the block-verification path (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte fragment per lane feeds one 16x16 MFMA step: E elements of the
// storage type, KSTEP = 4 * E reduction slots per step for the whole wave.
template <typename T> struct St;
template <> struct St<bf16> { static constexpr int E = 8, KSTEP = 32; };
template <> struct St<float> { static constexpr int E = 4, KSTEP = 16; };

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
// value as held in storage type T (round-to-nearest-even for bf16)
template <typename T> __device__ __forceinline__ float rnd(float x) { return to_f(from_f<T>(x)); }

// Layout of the activations inside the forward (the residual stream x, the
// mixer outputs, the MLP hidden rows, the attention queries): rows in tiles of
// 16, each tile split into k-steps of 4E columns, each step one contiguous
// block [row][4E]. The operand fragment of row tile t and k-step s is that
// block (lane l reads row l % 16, columns (l / 16) * E .. + E - 1), and the
// rows of a partial tile fill its front: a launch whose last tile holds 13
// rows (gamma = 12) points the lanes of rows 13..15 at row 12 and touches 7
// of the block's 8 128-byte lines (rows of a tile past the valid count are
// never written and only feed discarded output columns). E is the storage
// type's per-lane element count (8 for bf16 models, 4 for fp32), also for
// the fp32 residual stream. K is the matrix's column count (a multiple of 4E).
template <int E>
__host__ __device__ __forceinline__ size_t act_off(int m, int c, int K) {
  constexpr int KS = 4 * E;
  return ((size_t)(m >> 4) * (K / KS) + c / KS) * (16 * KS) + (size_t)(m & 15) * KS + (c % KS);
}

// Packed weights: 1 KB fragments (64 lanes x 16 bytes) in the order
// [wave step i][group g][wave w][tile nt], wave w of a workgroup owning the
// weight steps w * pw + i, i < pw. At any moment the waves of every
// workgroup are at about the same step, so the whole chip reads one
// contiguous window of the matrix, front to back (on MI355X 2-8% faster by
// projection than one contiguous run per wave). packed_slot: slot idx (in
// 16-byte units) -> its group, weight step, tile and lane; packed_strides:
// the strides (16-byte units) between groups, waves and steps.
constexpr int PACK_WAVES = 8;
struct MatStrides { long long g, w, t; };
__host__ __device__ __forceinline__ MatStrides packed_strides(int n_groups, int NT) {
  const long long f = (long long)NT * 64;   // one step of one wave: NT fragments
  return MatStrides{PACK_WAVES * f, f, (long long)n_groups * PACK_WAVES * f};
}
__host__ __device__ __forceinline__ void packed_slot(long long idx, int n_groups, int NT, int pw, int& g, int& k,
                                                     int& nt, int& lane) {
  lane = (int)(idx % 64);
  long long r = idx / 64;
  nt = (int)(r % NT);
  r /= NT;
  const int w = (int)(r % PACK_WAVES);
  r /= PACK_WAVES;
  g = (int)(r % n_groups);
  k = w * pw + (int)(r / n_groups);
}

// D += A * B for one 16x16 tile. Fragments: lane l holds row (l % 16) of A and
// column (l % 16) of B over the same reduction slots; D: lane l holds rows
// 4*(l/16) + i (i = 0..3) of column l % 16.
__device__ __forceinline__ f32x4 mma_frag(uint4 a, uint4 b, f32x4 c, bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_frag(uint4 a, uint4 b, f32x4 c, float) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}
// Four reduction slots per lane group (lane l holds slots 4*(l/16) .. +3).
__device__ __forceinline__ f32x4 mma_k4(const float a[4], const float b[4], f32x4 c, bf16) {
  bf16x4 av, bv;
#pragma unroll
  for (int j = 0; j < 4; ++j) { av[j] = (bf16)a[j]; bv[j] = (bf16)b[j]; }
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av),
                                                   __builtin_bit_cast(s16x4, bv), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k4(const float a[4], const float b[4], f32x4 c, float) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// ------------------------------------------------------------------ GEMM args
enum AMode { A_ACT = 0, A_NORM = 1 };   // storage-type rows / the same rows with each row's RMSNorm scale on the product
enum Epi { E_STORE = 0, E_RESID = 1, E_GELU = 2, E_MIXER = 3 };
enum MixKind { MIX_FIR = 1, MIX_IIR = 2, MIX_ATTN = 3 };

struct MixArgs {
  int kind;
  int d;                 // channels
  int P;                 // positions per sequence in this call
  int seq0;              // state index of the sequence owning row 0
  const int* t;          // [B] committed lengths
  const int* iir_buf;    // [B]
  const int* iir_slot;   // [B]
  int* err;              // sticky error word
  // FIR
  float* ring; int R; long long ring_bs; const float* taps; int L;
  int fb;                // sequences whose windows the epilogue stages together (1 .. FIR_FB)
  // IIR
  float* iirst; long long iir_bs; long long iir_buf_s; int N; const float* lam; const float* res;
  // ATTN
  void* kc; void* vt; long long kv_bs; int cap; int Dh;
};

struct GemmArgs {
  const uint4* W;        // packed MFMA fragments (16 bytes per lane)
  long long gstride;     // fragment-row stride (in 16-byte units) between groups,
  long long wstride;     //   between the waves of a group,
  long long tstride;     //   and between consecutive k-steps of one wave
  int ksteps;            // K / KSTEP
  int n_groups;
  const void* A;         // T [M, lda] (A_NORM: the residual rows in the storage type)
  int lda;
  int M;                 // rows in this call
  int rows_per_slice;    // rows per blockIdx.y (a multiple of the positions per sequence)
  const float* nrm_part; int n_part; int nrm_ld; float fd; float eps;      // A_NORM: [row][nrm_ld] sums of squares, fd = d
  const float* wscale;   // FP8 weights: one scale per packed row ([group][tile][16]); else null
  // epilogue
  int N;                 // valid output columns (E_STORE)
  void* out; int ldo;    // E_STORE / E_GELU / E_MIXER output (storage type)
  float* x; int ldx;     // E_RESID residual stream
  float* nrm_out;        // E_RESID per-16-column sums of squares [row][nrm_ld]
  bf16* xb_out;          // E_RESID, bf16 models: the residual rows in bf16 (the normed projections' operand)
  MixArgs mix;
  float* part;           // split-K launches: the k-range partials [slice][nparts][group][MT][NT][64 lanes][4]
  int nparts;            // 8 (one per k-range) or 4 (range pairs r + (r + 4)); 0 reads as 8
};

struct AttnArgs {
  const void* q;         // [M, d] storage type
  void* out;             // [M, d]
  const void* kc;        // [B, H, cap, Dh]
  const void* vt;        // [B, H, cap/16, Dh, 16]: 16-key blocks, dimension-major inside
  long long kv_bs;       // per-sequence stride (elements) of kc / vt
  int cap, H, Dh, d, P, QTN, S, seq0;
  int LS;                // keys per split range (a multiple of 16); S * LS >= cap
  const int* t;
  float scale;
  float* part;           // [B_call, QTN, H, S, 16, Dh + 2] split partials
};

constexpr int ATTN_CHUNK = 256;   // the KV capacity is a multiple of this many keys
constexpr int IIR_CH = 16;        // positions per chunk of the IIR mixer epilogue
constexpr int IIR_FB = 8;         // sequences whose committed IIR modes are loaded together
constexpr int FIR_FB = 8;         // most sequences whose FIR windows are staged together

struct VerifyArgs {
  int gamma, V, kind, top_k, greedy;
  float temperature;
  const void* target; const float* q; const int* draft; const float* u;
  int* n_acc; int* next; int* n_keep; int* err;
};

// ------------------------------------------------------------------ launchers
// FP8 (E4M3) weights, bf16 activations: fragments of 16 bytes per lane hold
// two MFMA k-steps; GemmArgs::ksteps counts those 64-wide steps
hipError_t launch_gemm_w8(int MT, int NT, int amode, int epi, const GemmArgs& a, int slices, size_t lds_bytes,
                          hipStream_t st);
hipError_t launch_fp8_scales(const bf16* W, float* scales, int rows_valid, int K, int n_groups, int NT,
                             int map_kind, int map_stride, hipStream_t st);
hipError_t launch_pack_fp8(const bf16* W, const float* scales, uint4* out, int rows_valid, int K, int n_groups,
                           int NT, int map_kind, int map_stride, hipStream_t st);
template <typename T>
hipError_t launch_gemm(int MT, int NT, int amode, int epi, const GemmArgs& a, int slices,
                       size_t lds_bytes, hipStream_t st);
template <typename T>
hipError_t launch_attn(const AttnArgs& a, int n_seq, hipStream_t st);
// producers of residual rows write fp32 x, its per-16-column sums of squares
// and, for bf16 models (xb non-null), the rows in bf16 for the normed projections
template <typename T>
hipError_t launch_embed(const int* tokens, const T* E, float* x, bf16* xb, float* nrm, int nrm_ld, int M, int d,
                        int V, int P, int seq0, const int* t, int max_ctx, int* err, hipStream_t st);
hipError_t launch_commit(int* t, int* iir_buf, int* iir_slot, const int* n_keep, int n_keep_all,
                         int B, int P, int* err, hipStream_t st);
hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t st);
template <typename T>
hipError_t launch_pack(const T* W, uint4* out, int rows_valid, int K, int n_groups, int NT,
                       int map_kind, int map_stride, hipStream_t st);
hipError_t launch_copy_row(const void* src, void* dst, size_t bytes, hipStream_t st);
hipError_t launch_verify(const VerifyArgs& a, int B, hipStream_t st);
// multi-tile bf16 launches: k-range partials, then the reduction and
// epilogue (results equal launch_gemm's)
hipError_t launch_gemm_split(int MT, int NT, int epi, const GemmArgs& a, int slices, size_t lds, hipStream_t st);

struct DraftArgs {
  const void* logits;    // [B, gamma, V] storage type: the drafter head's logits
  const float* markov;   // [V, V]
  const int* last;       // [B]
  const float* u;        // [B, gamma] (unused when greedy)
  int gamma, V, top_k, greedy;
  float temperature;
  int* drafts;           // [B, gamma]
  float* q;              // [B, gamma, V] or null
  int* err;
};
template <typename T> hipError_t launch_export_rows(const float* x, float* dst, int m0, int M, int d, hipStream_t st);
template <typename T>
hipError_t launch_export_pick(const float* x, float* dst, const int* pick, int B, int P, int d, hipStream_t st);
// measurement aid (measure.hip): the weight stream of one packed matrix alone
hipError_t launch_stream(int NT, int CH, const uint4* W, long long gstride, long long wstride, long long tstride,
                         int ksteps, int n_groups, unsigned* sink, hipStream_t st);
// generation loop (gen.hip)
hipError_t launch_gen_start(const int* next, int B, int n_tokens, int* ids, int* last, int* idx, int* emitted,
                            int* stats, hipStream_t st);
hipError_t launch_gen_cand(const int* last, const int* emitted, int B, int gamma, const int* table, int table_len,
                           const int* replace, int* drafts, int* cand, float* q, int V, hipStream_t st);
hipError_t launch_gen_emit(const int* drafts, int gamma, const int* n_acc, const int* next, int B, int n_tokens,
                           int* ids, int* emitted, int* n_keep, int* last, int* idx, int* stats, hipStream_t st);
// batched prefill: one round's candidate blocks, n_keep and last-row picks; the picked rows
hipError_t launch_prefill_round(const int* tokens, const int* offs, int B, int P, int R, int j, int* cand,
                                int* n_keep, int* pick, hipStream_t st);
hipError_t launch_pick_rows(const void* src, void* dst, const int* pick, int B, int P, size_t row_bytes,
                            hipStream_t st);
template <typename T>
hipError_t launch_inject_prep(const float* hidden, int rows, const int* index, int B, int K, float eps, T* u,
                              int* err, hipStream_t st);
template <typename T>
hipError_t launch_slots(const T* E, const T* pos, const T* z, const int* last, int B, int gamma, int d, int V,
                        float* x, bf16* xb, float* nrm, int nrm_ld, int* err, hipStream_t st);
template <typename T> hipError_t launch_draft(const DraftArgs& a, int B, hipStream_t st);

}  // namespace evs
