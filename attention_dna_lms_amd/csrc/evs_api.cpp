// Host side of the C ABI (include/evs.h): model and state layout, argument and
// state-machine checks, and the launch sequence of the block-verification
// forward, the verifier and the rollback. All device work is enqueued on the
// caller's stream; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/evs.h"
#include "evs_dev.h"

using namespace evs;

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_ROWS_PER_WG = 144;   // 9 MFMA row tiles
constexpr int SPLIT_MT = 7;            // row tiles from which bf16 launches split K across workgroups
constexpr int SPLIT_PAIR_MT = 9;       // row tiles from which split launches store range-pair partials (4, not 8)
constexpr int GEMM_WAVES = PACK_WAVES; // waves per GEMM workgroup (gemm_kernel default)
constexpr int ATTN_CUS = 256;          // compute units the attention split count is sized for
constexpr size_t LDS_MAX = 163840;     // LDS one workgroup may use on gfx950 (160 KB)

size_t align_up(size_t x, size_t a = ALIGN) { return (x + a - 1) / a * a; }
int next_pow2(int x) { int p = 1; while (p < x) p <<= 1; return p; }

struct Mat {            // one packed matrix
  size_t off = 0;       // byte offset in the packed buffer
  int rows_valid = 0, K = 0, n_groups = 0, NT = 1, map_kind = 0, map_stride = 0;
  bool w8 = false;      // FP8 E4M3 fragments (one byte per weight) + row scales at sc_off
  size_t sc_off = 0;
  size_t bytes(int es) const { return (size_t)n_groups * NT * 16 * K * (w8 ? 1 : es); }
  size_t scale_bytes() const { return w8 ? (size_t)n_groups * NT * 16 * 4 : 0; }
  // weight steps: one 1 KB fragment (64 lanes x 16 bytes) per tile and step;
  // kstep = the MFMA k-step of the storage type (FP8 fragments hold two)
  int steps(int kstep) const { return K / (w8 ? 2 * kstep : kstep); }
  int per_wave(int kstep) const { return (steps(kstep) + GEMM_WAVES - 1) / GEMM_WAVES; }
  // the packed buffer holds every wave's range at full length (the last
  // ranges of a K that is not a multiple of 8 steps are zero-padded)
  size_t packed_bytes(int kstep) const { return (size_t)n_groups * NT * GEMM_WAVES * per_wave(kstep) * 1024; }
};

// The kernels' strides of a packed matrix (the layout packed_slot describes)
MatStrides mat_strides(const Mat& mm) { return packed_strides(mm.n_groups, mm.NT); }

// storage type of activations, states and the non-FP8 tensors
int storage_dtype(const evs_model_desc* d) { return d->dtype == EVS_F32 ? EVS_F32 : EVS_BF16; }

struct BlockPlan {
  evs_block_desc d{};
  Mat w_in, w_out, w_gu, w_down;
  size_t taps = 0, lam = 0, res = 0;   // f32 parameter offsets
};

}  // namespace

struct evs_model {
  evs_model_desc desc{};
  std::vector<evs_block_desc> blocks;
  std::vector<BlockPlan> plan;
  char* base = nullptr;
  size_t embed = 0, total = 0;
  Mat lm;
  Mat inj;                          // drafter: the hidden-state injection [d, inject_dim]
  size_t pos = 0, markov = 0;       // drafter: position embeddings, Markov matrix (f32)
  int es = 2, kstep = 32;
  int max_dff = 0, max_heads = 0, max_dh = 0;
};

struct evs_state {
  const evs_model* m = nullptr;
  int B = 0, max_ctx = 0, max_block = 0, cap = 0, S = 1, LS = 1, qtn_max = 1, M_max = 0;
  char* sb = nullptr;   // state buffer
  char* wb = nullptr;   // workspace
  size_t off_t = 0, off_ib = 0, off_is = 0, off_err = 0;
  std::vector<size_t> ring, iir, kc, vt;   // per block
  std::vector<int> R;
  size_t state_total = 0;
  // workspace
  size_t w_x = 0, w_nrm = 0, w_o = 0, w_q = 0, w_h = 0, w_logit = 0, w_apart = 0, ws_total = 0;
  size_t apart_floats = 0;
  size_t w_inj_x = 0, w_z = 0;                  // drafter: the normalised injected rows, the prefix z
  size_t w_xb = 0;                              // bf16 models: the residual rows in bf16 (normed operands)
  size_t w_part = 0, part_bytes = 0;            // bf16 models: split-K partials of multi-tile launches
  size_t w_pre = 0;                             // batched prefill: candidate blocks, n_keep, picks, offsets (int32)
  int export_block = -1;                        // hidden-state export after this block (evs_block_verify)
  float* export_dst = nullptr;
  bool pending = false;
  int pending_P = 0;
  // per-kernel timing (measurement aid): one event pair around each run of
  // consecutive launches of one kernel class
  struct Rec { hipEvent_t a, b; int kc; double bytes; long long n; };
  bool timing = false;
  long long timing_ctx = 0;   // caller-supplied context length used for attention byte counts
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t span_a = nullptr;   // open run: start event, class, launches, bytes, stream
  int span_kc = 0;
  long long span_n = 0;
  double span_bytes = 0;
  hipStream_t span_st = nullptr;
  ~evs_state() {
    for (auto& r : recs) { pool.push_back(r.a); pool.push_back(r.b); }
    if (span_a) pool.push_back(span_a);
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

namespace {

bool check_desc(const evs_model_desc* d) {
  if (!d || !d->blocks || d->n_blocks < 0 || d->vocab < 2 || d->d_model < 32 || d->d_model % 32) return false;
  if (d->dtype != EVS_BF16 && d->dtype != EVS_F32 && d->dtype != EVS_BF16_FP8W) return false;
  const int kq = d->dtype == EVS_BF16_FP8W ? 64 : 32;   // FP8 fragments hold two 32-wide k-steps
  if (d->d_model % kq) return false;
  if (!(d->norm_eps >= 0.f)) return false;
  if (d->inject_dim < 0 || d->max_slots < 0) return false;
  if (d->inject_dim > 0) {
    if (d->dtype == EVS_BF16_FP8W || d->inject_dim % 32 || d->max_slots < 1 || d->max_slots > 64) return false;
  } else if (d->max_slots != 0) {
    return false;
  }
  for (int i = 0; i < d->n_blocks; ++i) {
    const evs_block_desc& b = d->blocks[i];
    switch (b.kind) {
      case EVS_FIR: if (b.fir_len < 1 || b.fir_len > 4096) return false; break;
      case EVS_IIR: if (b.iir_states < 1 || b.iir_states > 16) return false; break;
      case EVS_ATTN:
        if (b.head_dim != 32 && b.head_dim != 64 && b.head_dim != 128) return false;
        if (b.n_heads < 1 || (long long)b.n_heads * b.head_dim != d->d_model) return false;
        break;
      case EVS_MLP: if (b.d_ff < 32 || b.d_ff % kq) return false; break;
      default: return false;
    }
  }
  return true;
}

// Lay out the packed buffer for `desc` into `m` (no device access).
void plan_model(const evs_model_desc* desc, evs_model* m) {
  m->desc = *desc;
  m->blocks.assign(desc->blocks, desc->blocks + desc->n_blocks);
  m->desc.blocks = m->blocks.data();
  m->es = storage_dtype(desc) == EVS_BF16 ? 2 : 4;
  m->kstep = storage_dtype(desc) == EVS_BF16 ? 32 : 16;
  const int d = desc->d_model, V = desc->vocab, es = m->es;
  const bool w8 = desc->dtype == EVS_BF16_FP8W;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  auto place = [&](Mat& mm) {             // block projections: FP8 in the FP8 variant
    mm.w8 = w8;
    mm.off = take(mm.packed_bytes(m->kstep));
    if (w8) mm.sc_off = take(mm.scale_bytes());
  };
  m->embed = take((size_t)V * d * es);
  m->plan.clear();
  m->max_dff = m->max_heads = m->max_dh = 0;
  for (const auto& b : m->blocks) {
    BlockPlan p;
    p.d = b;
    if (b.kind == EVS_MLP) {
      p.w_gu = Mat{0, 2 * b.d_ff, d, b.d_ff / 16, 2, 1, b.d_ff};
      place(p.w_gu);
      p.w_down = Mat{0, d, b.d_ff, d / 16, 1, 0, 0};
      place(p.w_down);
      m->max_dff = std::max(m->max_dff, b.d_ff);
    } else {
      p.w_in = Mat{0, 3 * d, d, d / 16, 3, 1, d};
      place(p.w_in);
      if (b.kind == EVS_FIR) p.taps = take((size_t)d * b.fir_len * 4);
      if (b.kind == EVS_IIR) { p.lam = take((size_t)d * b.iir_states * 4); p.res = take((size_t)d * b.iir_states * 4); }
      if (b.kind == EVS_ATTN) { m->max_heads = std::max(m->max_heads, b.n_heads); m->max_dh = std::max(m->max_dh, b.head_dim); }
      p.w_out = Mat{0, d, d, d / 16, 1, 0, 0};
      place(p.w_out);
    }
    m->plan.push_back(p);
  }
  m->lm = Mat{0, V, d, (V + 15) / 16, 1, 0, 0};
  m->lm.off = take(m->lm.packed_bytes(m->kstep));
  if (desc->inject_dim > 0) {
    m->inj = Mat{0, d, desc->inject_dim, d / 16, 1, 0, 0};
    m->inj.off = take(m->inj.packed_bytes(m->kstep));
    m->pos = take((size_t)desc->max_slots * d * es);
    m->markov = take((size_t)V * V * 4);
  }
  m->total = off;
}

// canonical tensor list (see evs.h)
struct Canon { int64_t rows, cols; int dtype; };
std::vector<Canon> canon_list(const evs_model_desc* d) {
  std::vector<Canon> v;
  const int64_t D = d->d_model;
  const int mt = storage_dtype(d);
  v.push_back({d->vocab, D, mt});
  for (int i = 0; i < d->n_blocks; ++i) {
    const evs_block_desc& b = d->blocks[i];
    if (b.kind == EVS_FIR) { v.push_back({3 * D, D, mt}); v.push_back({D, b.fir_len, EVS_F32}); v.push_back({D, D, mt}); }
    else if (b.kind == EVS_IIR) {
      v.push_back({3 * D, D, mt}); v.push_back({D, b.iir_states, EVS_F32}); v.push_back({D, b.iir_states, EVS_F32});
      v.push_back({D, D, mt});
    } else if (b.kind == EVS_ATTN) { v.push_back({3 * D, D, mt}); v.push_back({D, D, mt}); }
    else { v.push_back({2LL * b.d_ff, D, mt}); v.push_back({D, b.d_ff, mt}); }
  }
  v.push_back({d->vocab, D, mt});
  if (d->inject_dim > 0) {
    v.push_back({D, d->inject_dim, mt});
    v.push_back({d->max_slots, D, mt});
    v.push_back({d->vocab, d->vocab, EVS_F32});
  }
  return v;
}


struct Slicing { int rows_per_slice, slices, MT; };
Slicing slicing(int nseq, int P) {
  int sps = std::max(1, MAX_ROWS_PER_WG / P);
  sps = std::min(sps, nseq);
  Slicing s;
  s.rows_per_slice = sps * P;
  s.slices = (nseq + sps - 1) / sps;
  s.MT = (s.rows_per_slice + 15) / 16;
  return s;
}


int gemm_bufs(int MT, int NT) { return (4 * NT * MT <= 48) ? 4 : ((2 * NT * MT <= 48) ? 2 : 1); }

// LDS of a gemm_kernel launch: row scales, then either all 8 wave partials
// followed by the epilogue tile (small tiles, one-barrier reduction) or the
// staged-tree buffers overlapped with the epilogue tile.
size_t gemm_lds(int MT, int NT, int scratch_floats) {
  const size_t RS = (size_t)NT * MT * 256;
  if (NT * MT <= 4) return 4 * (MT * 16 + 9 * RS + (size_t)scratch_floats);
  return 4 * (MT * 16 + std::max(gemm_bufs(MT, NT) * RS, RS + (size_t)scratch_floats));
}

void layout_state(evs_state* s) {
  const evs_model* m = s->m;
  const int d = m->desc.d_model, es = m->es, B = s->B;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  s->off_t = take(4 * (size_t)B);
  s->off_ib = take(4 * (size_t)B);
  s->off_is = take(4 * (size_t)B);
  s->off_err = take(4);
  const size_t nb = m->blocks.size();
  s->ring.assign(nb, 0); s->iir.assign(nb, 0); s->kc.assign(nb, 0); s->vt.assign(nb, 0); s->R.assign(nb, 0);
  for (size_t i = 0; i < nb; ++i) {
    const evs_block_desc& b = m->blocks[i];
    if (b.kind == EVS_FIR) {
      s->R[i] = next_pow2(b.fir_len - 1 + s->max_block);
      s->ring[i] = take((size_t)B * s->R[i] * d * 4);
    } else if (b.kind == EVS_IIR) {
      s->iir[i] = take((size_t)B * 2 * s->max_block * d * b.iir_states * 4);
    } else if (b.kind == EVS_ATTN) {
      s->kc[i] = take((size_t)B * b.n_heads * s->cap * b.head_dim * es);
      s->vt[i] = take((size_t)B * b.n_heads * s->cap * b.head_dim * es);
    }
  }
  s->state_total = off;

  // workspace
  const int M = s->M_max;
  off = 0;
  const size_t M16 = align_up((size_t)M, 16);   // activations are stored in whole 16-row tiles
  s->w_x = take(M16 * d * 4);
  s->w_nrm = take((size_t)(d / 16) * M * 4);
  s->w_o = take(M16 * d * es);
  s->w_q = take(M16 * d * es);
  s->w_h = take(M16 * std::max(m->max_dff, 32) * es);
  // logits staging (evs_prefill's last rows): every sequence's block
  s->w_logit = take((size_t)B * s->max_block * m->desc.vocab * es);
  s->w_pre = take(((size_t)B * s->max_block + 3 * (size_t)B + 1) * 4);
  const int H = std::max(m->max_heads, 1), DHm = std::max(m->max_dh, 32);
  s->qtn_max = (s->max_block + 15) / 16;
  s->apart_floats = (size_t)B * s->qtn_max * H * s->S * 16 * (DHm + 2);
  s->w_apart = take(s->apart_floats * 4);
  if (es == 2) {
    s->w_xb = take(M16 * d * 2);
    // split-K partials: 8 ranges x the padded rows of the widest slicing that
    // splits x the widest projection
    size_t rows = 0;
    for (int P = 1; P <= s->max_block; ++P) {
      const Slicing sl = slicing(B, P);
      if (sl.MT >= SPLIT_MT) rows = std::max(rows, (size_t)sl.slices * sl.MT * 16);
    }
    size_t nmax = (size_t)((m->desc.vocab + 15) / 16) * 16;
    for (const auto& p : m->plan) {
      if (p.d.kind == EVS_MLP) nmax = std::max({nmax, (size_t)2 * p.d.d_ff, (size_t)d});
      else nmax = std::max(nmax, (size_t)3 * d);
    }
    s->part_bytes = 8 * rows * nmax * 4;
    if (s->part_bytes) s->w_part = take(s->part_bytes);
  }
  if (m->desc.inject_dim > 0) {
    const size_t B16 = align_up((size_t)B, 16);
    s->w_inj_x = take(B16 * m->desc.inject_dim * es);
    s->w_z = take(B16 * d * es);
  }
  s->ws_total = off;
}

template <typename T> T* sp(evs_state* s, size_t off) { return reinterpret_cast<T*>(s->sb + off); }
template <typename T> T* wp(evs_state* s, size_t off) { return reinterpret_cast<T*>(s->wb + off); }

evs_status hip_ok(hipError_t e) { return e == hipSuccess ? EVS_OK : EVS_E_HIP; }

hipEvent_t pool_event(evs_state* s) {
  if (!s->pool.empty()) { hipEvent_t e = s->pool.back(); s->pool.pop_back(); return e; }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// End the open run of timed launches (if any) with an event on its stream.
hipError_t close_span(evs_state* s) {
  if (!s->span_a) return hipSuccess;
  hipEvent_t b = pool_event(s);
  if (!b) return hipErrorOutOfMemory;
  const hipError_t e = hipEventRecord(b, s->span_st);
  if (e != hipSuccess) return e;
  s->recs.push_back({s->span_a, b, s->span_kc, s->span_bytes, s->span_n});
  s->span_a = nullptr;
  return hipSuccess;
}

// Time a launch when the state's timing is on: `launch` enqueues the kernel.
// Consecutive launches of one class on one stream share a single event pair
// (the run closes at the first launch of another class and at the end of the
// API call), so the events add no gaps inside a run of back-to-back kernels.
template <typename F>
hipError_t timed(evs_state* s, int kc, double bytes, hipStream_t st, F&& launch) {
  if (!s->timing) return launch();
  if (s->span_a && (s->span_kc != kc || s->span_st != st)) {
    const hipError_t e = close_span(s);
    if (e != hipSuccess) return e;
  }
  if (!s->span_a) {
    hipEvent_t a = pool_event(s);
    if (!a) return hipErrorOutOfMemory;
    const hipError_t e = hipEventRecord(a, st);
    if (e != hipSuccess) return e;
    s->span_a = a; s->span_kc = kc; s->span_n = 0; s->span_bytes = 0; s->span_st = st;
  }
  const hipError_t e = launch();
  if (e != hipSuccess) return e;
  ++s->span_n;
  s->span_bytes += bytes;
  return hipSuccess;
}
#define EVS_TRY(x) do { evs_status _st = (x); if (_st != EVS_OK) return _st; } while (0)
#define HIP_TRY(x) do { if ((x) != hipSuccess) return EVS_E_HIP; } while (0)

// ------------------------------------------------------------------ forward
template <typename T>
evs_status gemm_call(evs_model* m, evs_state* s, const Mat& mat, int amode, int epi, const void* A, int lda,
                     int nseq, int P, GemmArgs a, hipStream_t st, int scratch_floats = 0) {
  const Slicing sl = slicing(nseq, P);
  a.W = reinterpret_cast<const uint4*>(m->base + mat.off);
  a.ksteps = mat.steps(m->kstep);   // weight steps (FP8: two k-steps each)
  a.wscale = mat.w8 ? reinterpret_cast<const float*>(m->base + mat.sc_off) : nullptr;
  a.n_groups = mat.n_groups;
  // wave w of a workgroup owns the weight steps [w * per_wave, (w + 1) * per_wave)
  {
    const MatStrides ms = mat_strides(mat);
    a.gstride = ms.g;
    a.wstride = ms.w;
    a.tstride = ms.t;
  }
  a.A = A;
  a.lda = lda;
  a.M = nseq * P;
  a.rows_per_slice = sl.rows_per_slice;
  a.nrm_part = wp<float>(s, s->w_nrm);
  a.n_part = m->desc.d_model / 16;
  a.nrm_ld = m->desc.d_model / 16;   // partials per row
  a.fd = (float)m->desc.d_model;
  a.eps = m->desc.norm_eps;
  // algorithmic bytes: the weights once, the A rows once, the outputs once
  const double bytes = (double)(mat.bytes(m->es) + mat.scale_bytes()) + (double)a.M * mat.K * m->es +
                       (double)a.M * mat.rows_valid * (epi == E_RESID ? 8 : m->es);
  const size_t lds = gemm_lds(sl.MT, mat.NT, scratch_floats);
  if (lds > LDS_MAX) return EVS_E_UNSUPPORTED;
  // multi-tile bf16 launches: k-range partials, then the reduction and
  // epilogue (the same results as one kernel)
  if (m->desc.dtype == EVS_BF16 && !mat.w8 && sl.MT >= SPLIT_MT &&
      (size_t)8 * sl.slices * sl.MT * 16 * mat.n_groups * mat.NT * 16 * 4 <= s->part_bytes) {
    a.part = wp<float>(s, s->w_part);
    // 9 row tiles: range-pair partials (half the partial bytes for twice the
    // activation staging: measured faster there, slower at 7 tiles)
    a.nparts = sl.MT >= SPLIT_PAIR_MT ? 4 : 8;
    return hip_ok(timed(s, EVS_KC_GEMM, bytes, st,
                        [&] { return launch_gemm_split(sl.MT, mat.NT, epi, a, sl.slices, lds, st); }));
  }
  return hip_ok(timed(s, EVS_KC_GEMM, bytes, st,
                      [&] {
                        if constexpr (sizeof(T) == 2)
                          if (mat.w8) return launch_gemm_w8(sl.MT, mat.NT, amode, epi, a, sl.slices, lds, st);
                        return launch_gemm<T>(sl.MT, mat.NT, amode, epi, a, sl.slices, lds, st);
                      }));
}

// The forward over nseq sequences of P positions: the embedding of `tokens`
// (or, with tokens null, input rows the caller already wrote into the
// residual buffer with their norm partials), every block, and the LM head
// into `logits` (if not null). With export_dst, the residual rows after block
// s->export_block are also written out row-major: rows export_m0 ..
// export_m0 + export_n - 1 of the call, or with export_pick (device, one entry
// per sequence) block row export_pick[b] of each sequence into row b.
template <typename T>
evs_status forward(evs_model* m, evs_state* s, int seq0, int nseq, int P, const int32_t* tokens, void* logits,
                   hipStream_t st, float* export_dst = nullptr, int export_m0 = 0, int export_n = -1,
                   const int* export_pick = nullptr) {
  const int d = m->desc.d_model, M = nseq * P;
  if (export_n < 0) export_n = M;
  float* x = wp<float>(s, s->w_x);
  // the residual rows in the storage type: the operand of every normed
  // projection, written by the same producer as x and its norm partials
  bf16* xb = sizeof(T) == 2 ? wp<bf16>(s, s->w_xb) : nullptr;
  float* nrm = wp<float>(s, s->w_nrm);
  int* t = sp<int>(s, s->off_t);
  int* err = sp<int>(s, s->off_err);
  auto normed = [&](int& amode, const void*& A) -> evs_status {
    amode = A_NORM;
    A = sizeof(T) == 2 ? static_cast<const void*>(xb) : static_cast<const void*>(x);
    return EVS_OK;
  };
  if (tokens)
    HIP_TRY(launch_embed<T>(tokens, reinterpret_cast<const T*>(m->base + m->embed), x, xb, nrm, d / 16, M, d,
                            m->desc.vocab, P, seq0, t, s->max_ctx, err, st));
  for (size_t i = 0; i < m->plan.size(); ++i) {
    if (i > 0 && export_dst && (int)i - 1 == s->export_block)
      HIP_TRY(export_pick ? launch_export_pick<T>(x, export_dst, export_pick, nseq, P, d, st)
                          : launch_export_rows<T>(x, export_dst, export_m0, export_n, d, st));
    const BlockPlan& p = m->plan[i];
    GemmArgs a{};
    if (p.d.kind == EVS_MLP) {
      a.out = wp<void>(s, s->w_h);
      a.ldo = p.d.d_ff;
      int am;
      const void* A;
      EVS_TRY(normed(am, A));
      EVS_TRY(gemm_call<T>(m, s, p.w_gu, am, E_GELU, A, d, nseq, P, a, st));
      GemmArgs b{};
      b.x = x; b.ldx = d; b.nrm_out = nrm; b.xb_out = xb;
      EVS_TRY(gemm_call<T>(m, s, p.w_down, A_ACT, E_RESID, wp<void>(s, s->w_h), p.d.d_ff, nseq, P, b, st));
      continue;
    }
    MixArgs& mx = a.mix;
    mx.d = d; mx.P = P; mx.seq0 = seq0; mx.t = t;
    mx.iir_buf = sp<int>(s, s->off_ib); mx.iir_slot = sp<int>(s, s->off_is); mx.err = err;
    int scratch = 0;
    if (p.d.kind == EVS_FIR) {
      mx.kind = MIX_FIR;
      mx.ring = sp<float>(s, s->ring[i]); mx.R = s->R[i]; mx.ring_bs = (long long)s->R[i] * d;
      mx.taps = reinterpret_cast<const float*>(m->base + p.taps); mx.L = p.d.fir_len;
      // taps (odd row stride) + the windows and inputs of fb sequences: the
      // most of a slice's sequences (up to FIR_FB) that fit the workgroup's LDS
      const Slicing sl = slicing(nseq, P);
      const int per_seq = (p.d.fir_len - 1 + P) * 16, taps_f = 16 * (p.d.fir_len | 1);
      mx.fb = std::min(FIR_FB, sl.rows_per_slice / P);
      while (mx.fb > 1 && gemm_lds(sl.MT, p.w_in.NT, taps_f + mx.fb * per_seq) > LDS_MAX) --mx.fb;
      scratch = taps_f + mx.fb * per_seq;
      a.out = wp<void>(s, s->w_o);
    } else if (p.d.kind == EVS_IIR) {
      mx.kind = MIX_IIR;
      mx.iirst = sp<float>(s, s->iir[i]); mx.N = p.d.iir_states;
      mx.iir_buf_s = (long long)s->max_block * d * p.d.iir_states;
      mx.iir_bs = 2 * mx.iir_buf_s;
      mx.lam = reinterpret_cast<const float*>(m->base + p.lam);
      mx.res = reinterpret_cast<const float*>(m->base + p.res);
      scratch = 0;   // the epilogue works in registers and DPP rows
      a.out = wp<void>(s, s->w_o);
    } else {
      mx.kind = MIX_ATTN;
      scratch = MAX_ROWS_PER_WG;   // the slice's committed lengths
      mx.kc = sp<void>(s, s->kc[i]); mx.vt = sp<void>(s, s->vt[i]);
      mx.kv_bs = (long long)p.d.n_heads * s->cap * p.d.head_dim; mx.cap = s->cap; mx.Dh = p.d.head_dim;
      a.out = wp<void>(s, s->w_q);
    }
    a.ldo = d;
    int am;
    const void* A;
    EVS_TRY(normed(am, A));
    EVS_TRY(gemm_call<T>(m, s, p.w_in, am, E_MIXER, A, d, nseq, P, a, st, scratch));
    if (p.d.kind == EVS_ATTN) {
      AttnArgs at{};
      at.q = wp<void>(s, s->w_q); at.out = wp<void>(s, s->w_o);
      at.kc = mx.kc; at.vt = mx.vt; at.kv_bs = mx.kv_bs; at.cap = s->cap;
      at.H = p.d.n_heads; at.Dh = p.d.head_dim; at.d = d; at.P = P; at.QTN = (P + 15) / 16; at.S = s->S; at.LS = s->LS;
      at.seq0 = seq0; at.t = t; at.scale = 1.0f / std::sqrt((float)p.d.head_dim);
      at.part = wp<float>(s, s->w_apart);
      if ((size_t)nseq * at.QTN * at.H * at.S * 16 * (at.Dh + 2) > s->apart_floats) return EVS_E_RANGE;
      // algorithmic bytes: K and V rows up to each sequence's block end (bounded
      // here by the capacity-limited length known on the host: the state's
      // committed lengths live on the device), q in, o out
      const double kvb = (double)nseq * at.H * at.Dh * m->es * 2.0 * (double)s->timing_ctx;
      HIP_TRY(timed(s, EVS_KC_ATTN, kvb + 2.0 * nseq * P * d * m->es, st, [&] { return launch_attn<T>(at, nseq, st); }));
    }
    GemmArgs b{};
    b.x = x; b.ldx = d; b.nrm_out = nrm; b.xb_out = xb;
    EVS_TRY(gemm_call<T>(m, s, p.w_out, A_ACT, E_RESID, wp<void>(s, s->w_o), d, nseq, P, b, st));
  }
  if (export_dst && s->export_block == (int)m->plan.size() - 1)
    HIP_TRY(export_pick ? launch_export_pick<T>(x, export_dst, export_pick, nseq, P, d, st)
                        : launch_export_rows<T>(x, export_dst, export_m0, export_n, d, st));
  if (logits) {
    GemmArgs a{};
    a.N = m->desc.vocab; a.out = logits; a.ldo = m->desc.vocab;
    int am;
    const void* A;
    EVS_TRY(normed(am, A));
    EVS_TRY(gemm_call<T>(m, s, m->lm, am, E_STORE, A, d, nseq, P, a, st));
  }
  return EVS_OK;
}

evs_status forward_any(evs_model* m, evs_state* s, int seq0, int nseq, int P, const int32_t* tokens, void* logits,
                       hipStream_t st, float* export_dst = nullptr, int export_m0 = 0, int export_n = -1,
                       const int* export_pick = nullptr) {
  if (storage_dtype(&m->desc) == EVS_BF16)
    return forward<bf16>(m, s, seq0, nseq, P, tokens, logits, st, export_dst, export_m0, export_n, export_pick);
  return forward<float>(m, s, seq0, nseq, P, tokens, logits, st, export_dst, export_m0, export_n, export_pick);
}

// The drafter's pass (evs_draft): injected prefix, slot rows, the drafter's
// blocks and head over the slots, then the Markov head and draws.
template <typename T>
evs_status draft_pass(evs_model* m, evs_state* s, int B, const float* hidden, int hidden_rows, const int32_t* hidx,
                      const int32_t* last, int gamma, const float* u, float temperature, int top_k, int greedy,
                      void* logits, int32_t* drafts, float* q, hipStream_t st) {
  const int d = m->desc.d_model, K = m->desc.inject_dim, V = m->desc.vocab;
  int* err = sp<int>(s, s->off_err);
  T* xin = wp<T>(s, s->w_inj_x);
  T* z = wp<T>(s, s->w_z);
  HIP_TRY(launch_inject_prep<T>(hidden, hidden_rows, hidx, B, K, m->desc.norm_eps, xin, err, st));
  GemmArgs a{};
  a.N = d; a.out = z; a.ldo = d;
  EVS_TRY(gemm_call<T>(m, s, m->inj, A_ACT, E_STORE, xin, K, B, 1, a, st));
  HIP_TRY(launch_slots<T>(reinterpret_cast<const T*>(m->base + m->embed), reinterpret_cast<const T*>(m->base + m->pos),
                          z, last, B, gamma, d, V, wp<float>(s, s->w_x),
                          sizeof(T) == 2 ? wp<bf16>(s, s->w_xb) : nullptr, wp<float>(s, s->w_nrm), d / 16, err,
                          st));
  EVS_TRY(forward<T>(m, s, 0, B, gamma, nullptr, logits, st));
  DraftArgs da{};
  da.logits = logits; da.markov = reinterpret_cast<const float*>(m->base + m->markov); da.last = last; da.u = u;
  da.gamma = gamma; da.V = V; da.top_k = top_k; da.greedy = greedy ? 1 : 0; da.temperature = temperature;
  da.drafts = drafts; da.q = q; da.err = err;
  HIP_TRY(launch_draft<T>(da, B, st));
  return EVS_OK;
}

}  // namespace

// ------------------------------------------------------------- generation
namespace {

struct GenLayout {
  size_t cand = 0, drafts = 0, logits = 0, q = 0, n_acc = 0, next = 0, n_keep = 0, last = 0, idx = 0, emitted = 0,
         dlogits = 0, total = 0;
};

evs_status gen_check(const evs_model* m, const evs_state* s, const evs_gen_params* p, const evs_draft_source* d) {
  if (!m || !s || !p || s->m != m) return EVS_E_INVALID;
  const int src = d ? d->source : EVS_DRAFT_NONE;
  if (p->n_tokens < 1 || p->gamma < 0 || p->rounds_cap < 1) return EVS_E_INVALID;
  if (p->gamma + 1 > s->max_block) return EVS_E_RANGE;
  if ((long long)(p->gamma + 2) * m->desc.vocab > 15360) return EVS_E_UNSUPPORTED;   // the verifier's LDS rows
  if (!p->greedy) {
    if (!(p->temperature > 0.f && std::isfinite(p->temperature))) return EVS_E_INVALID;
    if (!p->u_first_dev || !p->u_target_dev) return EVS_E_INVALID;
  }
  switch (src) {
    case EVS_DRAFT_NONE:
      if (p->gamma != 0) return EVS_E_INVALID;
      break;
    case EVS_DRAFT_TABLE:
      if (p->gamma < 1 || !d->table_dev || d->table_len < 1) return EVS_E_INVALID;
      break;
    case EVS_DRAFT_MODEL: {
      const evs_model* dm = d->drafter;
      const evs_state* ds = d->drafter_state;
      if (p->gamma < 1 || !dm || !ds || ds->m != dm || dm->desc.inject_dim != m->desc.d_model) return EVS_E_INVALID;
      if (dm->desc.vocab != m->desc.vocab || !ds->wb) return EVS_E_INVALID;
      if (p->gamma > dm->desc.max_slots || p->gamma > ds->max_block || ds->B < s->B) return EVS_E_RANGE;
      if (s->export_block < 0 || !s->export_dst) return EVS_E_STATE;   // the drafter reads the exported rows
      if (!p->greedy && !p->u_draft_dev) return EVS_E_INVALID;
      break;
    }
    default: return EVS_E_INVALID;
  }
  return EVS_OK;
}

GenLayout gen_layout(const evs_model* m, const evs_state* s, const evs_gen_params* p, const evs_draft_source* d) {
  GenLayout g;
  const size_t B = s->B, P = p->gamma + 1, V = m->desc.vocab;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max(bytes, (size_t)4)); return o; };
  g.cand = take(B * P * 4);
  g.drafts = take(B * std::max(p->gamma, 1) * 4);
  g.logits = take(B * P * V * m->es);
  g.q = take(B * p->gamma * V * 4);
  g.n_acc = take(B * 4);
  g.next = take(B * 4);
  g.n_keep = take(B * 4);
  g.last = take(B * 4);
  g.idx = take(B * 4);
  g.emitted = take(B * 4);
  if (d && d->source == EVS_DRAFT_MODEL)
    g.dlogits = take(B * p->gamma * (size_t)d->drafter->desc.vocab * d->drafter->es);
  g.total = off;
  return g;
}

}  // namespace

// ------------------------------------------------------ no-allocation scratch
// The workspace of evs_block_verify_noalloc: one array per GPU, resident for
// the life of the process. Host code never passes `scratch` itself to a
// kernel (on the host it names a stand-in, not device memory): each device's
// address is looked up once with hipGetSymbolAddress, with that device
// current, and that pointer is what the forward uses.
static __device__ __align__(256) unsigned char scratch[EVS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[SCRATCH_MAX_DEVICES] = {};

// The current device's scratch address (looked up on the first call on that device).
evs_status scratch_ptr(char** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return EVS_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EVS_E_HIP;
    scratch_dev[dev] = p;
  }
  *out = reinterpret_cast<char*>(scratch_dev[dev]);
  return EVS_OK;
}
}  // namespace

// =================================================================== C ABI
extern "C" {

const char* evs_status_string(evs_status s) {
  switch (s) {
    case EVS_OK: return "ok";
    case EVS_E_INVALID: return "invalid argument";
    case EVS_E_RANGE: return "size out of range for this state";
    case EVS_E_STATE: return "call out of order";
    case EVS_E_HIP: return "HIP runtime error";
    case EVS_E_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

evs_status evs_canonical_count(const evs_model_desc* desc, int32_t* count) {
  if (!count || !check_desc(desc)) return EVS_E_INVALID;
  *count = (int32_t)canon_list(desc).size();
  return EVS_OK;
}

evs_status evs_canonical_shape(const evs_model_desc* desc, int32_t i, int64_t* rows, int64_t* cols,
                               int32_t* dtype) {
  if (!rows || !cols || !dtype || !check_desc(desc)) return EVS_E_INVALID;
  const auto v = canon_list(desc);
  if (i < 0 || (size_t)i >= v.size()) return EVS_E_RANGE;
  *rows = v[i].rows; *cols = v[i].cols; *dtype = v[i].dtype;
  return EVS_OK;
}

evs_status evs_weights_bytes(const evs_model_desc* desc, size_t* bytes) {
  if (!bytes || !check_desc(desc)) return EVS_E_INVALID;
  evs_model tmp;
  plan_model(desc, &tmp);
  *bytes = tmp.total;
  return EVS_OK;
}

evs_status evs_model_create(const evs_model_desc* desc, void* packed_dev, evs_model** out) {
  if (!out || !packed_dev || !check_desc(desc) || ((uintptr_t)packed_dev % ALIGN)) return EVS_E_INVALID;
  evs_model* m = new (std::nothrow) evs_model();
  if (!m) return EVS_E_INVALID;
  plan_model(desc, m);
  m->base = reinterpret_cast<char*>(packed_dev);
  *out = m;
  return EVS_OK;
}

void evs_model_destroy(evs_model* m) { delete m; }

evs_status evs_pack_weights(evs_model* m, const void* const* canon, void* stream) {
  if (!m || !canon) return EVS_E_INVALID;
  const auto list = canon_list(&m->desc);
  for (size_t i = 0; i < list.size(); ++i)
    if (!canon[i] || ((uintptr_t)canon[i] % 16)) return EVS_E_INVALID;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool bf = storage_dtype(&m->desc) == EVS_BF16;
  auto pack = [&](const void* src, const Mat& mm) -> hipError_t {
    uint4* dst = reinterpret_cast<uint4*>(m->base + mm.off);
    if (mm.w8) {
      float* sc = reinterpret_cast<float*>(m->base + mm.sc_off);
      const bf16* w = reinterpret_cast<const bf16*>(src);
      const hipError_t e = launch_fp8_scales(w, sc, mm.rows_valid, mm.K, mm.n_groups, mm.NT, mm.map_kind,
                                             mm.map_stride, st);
      if (e != hipSuccess) return e;
      return launch_pack_fp8(w, sc, dst, mm.rows_valid, mm.K, mm.n_groups, mm.NT, mm.map_kind, mm.map_stride, st);
    }
    if (bf) return launch_pack<bf16>(reinterpret_cast<const bf16*>(src), dst, mm.rows_valid, mm.K, mm.n_groups, mm.NT,
                                     mm.map_kind, mm.map_stride, st);
    return launch_pack<float>(reinterpret_cast<const float*>(src), dst, mm.rows_valid, mm.K, mm.n_groups, mm.NT,
                              mm.map_kind, mm.map_stride, st);
  };
  auto copy = [&](const void* src, size_t off, size_t bytes) {
    return launch_copy_row(src, m->base + off, bytes, st);
  };
  const int d = m->desc.d_model;
  size_t k = 0;
  HIP_TRY(copy(canon[k++], m->embed, (size_t)m->desc.vocab * d * m->es));
  for (const auto& p : m->plan) {
    if (p.d.kind == EVS_MLP) {
      HIP_TRY(pack(canon[k++], p.w_gu));
      HIP_TRY(pack(canon[k++], p.w_down));
      continue;
    }
    HIP_TRY(pack(canon[k++], p.w_in));
    if (p.d.kind == EVS_FIR) HIP_TRY(copy(canon[k++], p.taps, (size_t)d * p.d.fir_len * 4));
    if (p.d.kind == EVS_IIR) {
      HIP_TRY(copy(canon[k++], p.lam, (size_t)d * p.d.iir_states * 4));
      HIP_TRY(copy(canon[k++], p.res, (size_t)d * p.d.iir_states * 4));
    }
    HIP_TRY(pack(canon[k++], p.w_out));
  }
  HIP_TRY(pack(canon[k++], m->lm));
  if (m->desc.inject_dim > 0) {
    HIP_TRY(pack(canon[k++], m->inj));
    HIP_TRY(copy(canon[k++], m->pos, (size_t)m->desc.max_slots * d * m->es));
    HIP_TRY(copy(canon[k++], m->markov, (size_t)m->desc.vocab * m->desc.vocab * 4));
  }
  return EVS_OK;
}

static evs_status state_setup(const evs_model* m, int32_t batch, int32_t max_ctx, int32_t max_block, evs_state* s) {
  if (!m || batch < 1 || max_ctx < 1 || max_block < 1 || max_block > MAX_ROWS_PER_WG) return EVS_E_INVALID;
  if ((long long)batch * max_block > 4096 || batch > 4096) return EVS_E_RANGE;
  s->m = m;
  s->B = batch;
  s->max_ctx = max_ctx;
  s->max_block = max_block;
  s->cap = (int)align_up((size_t)max_ctx, ATTN_CHUNK);
  // attention splits: contiguous ranges of LS keys (a multiple of 64, so each
  // of a workgroup's 4 waves gets whole 16-key tiles), fixed by the state's
  // capacity and the head count alone: never by the block or the batch, so a
  // sequence's attention sums run in the same order whatever shares the
  // launch. One workgroup per CU for one sequence and one query tile
  // (measured best at 8k and 262k keys with 32 heads); batches add
  // workgroups.
  {
    const int heads = std::max(1, m->max_heads);
    int s0 = ATTN_CUS / heads;
    s0 = std::min(std::min(64, s0), s->cap / 64);
    s0 = std::max(1, s0);
    // mid-size capacities (batches of mixed contexts): ranges of ~2048 keys,
    // so sequences far shorter than the capacity still spread over many
    // workgroups and the longest do not leave a tail
    if (s->cap >= 16384 && s->cap <= 65536) s0 = std::max(s0, std::min(64, s->cap / 2048));
    s->LS = (int)align_up((size_t)((s->cap + s0 - 1) / s0), 64);
    s->S = (s->cap + s->LS - 1) / s->LS;
  }
  s->M_max = batch * max_block;
  layout_state(s);
  return EVS_OK;
}

evs_status evs_state_bytes(const evs_model* m, int32_t batch, int32_t max_ctx, int32_t max_block,
                           size_t* state_bytes, size_t* workspace_bytes) {
  if (!state_bytes || !workspace_bytes) return EVS_E_INVALID;
  evs_state tmp;
  EVS_TRY(state_setup(m, batch, max_ctx, max_block, &tmp));
  *state_bytes = tmp.state_total;
  *workspace_bytes = tmp.ws_total;
  return EVS_OK;
}

evs_status evs_state_create(const evs_model* m, int32_t batch, int32_t max_ctx, int32_t max_block, void* state_dev,
                            void* workspace_dev, void* stream, evs_state** out) {
  // (workspace_dev NULL: a state with no workspace of its own, for
  // evs_block_verify_noalloc)
  if (!out || !state_dev || ((uintptr_t)state_dev % ALIGN) || ((uintptr_t)workspace_dev % ALIGN))
    return EVS_E_INVALID;
  evs_state* s = new (std::nothrow) evs_state();
  if (!s) return EVS_E_INVALID;
  evs_status stt = state_setup(m, batch, max_ctx, max_block, s);
  if (stt != EVS_OK) { delete s; return stt; }
  s->sb = reinterpret_cast<char*>(state_dev);
  s->wb = reinterpret_cast<char*>(workspace_dev);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (e == hipSuccess) e = launch_fill_i32(sp<int>(s, s->off_t), 0, batch, st);
  if (e == hipSuccess) e = launch_fill_i32(sp<int>(s, s->off_ib), 0, batch, st);
  if (e == hipSuccess) e = launch_fill_i32(sp<int>(s, s->off_is), -1, batch, st);
  if (e == hipSuccess) e = launch_fill_i32(sp<int>(s, s->off_err), 0, 1, st);
  if (e != hipSuccess) { delete s; return EVS_E_HIP; }
  *out = s;
  return EVS_OK;
}

void evs_state_destroy(evs_state* s) { delete s; }

evs_status evs_state_tensor(const evs_state* s, int32_t what, int32_t block, evs_tensor_desc* o) {
  if (!s || !o) return EVS_E_INVALID;
  std::memset(o, 0, sizeof(*o));
  const evs_model* m = s->m;
  const int B = s->B, d = m->desc.d_model;
  const int dt = storage_dtype(&m->desc);
  auto need_block = [&](int kind) {
    return block >= 0 && (size_t)block < m->blocks.size() && m->blocks[block].kind == kind;
  };
  auto set = [&](uint64_t off, int dtype, std::initializer_list<int64_t> shape) {
    o->offset = off; o->dtype = dtype; o->ndim = (int32_t)shape.size();
    int i = 0;
    for (int64_t v : shape) o->shape[i++] = v;
    int64_t st = 1;
    for (int k = o->ndim - 1; k >= 0; --k) { o->strides[k] = st; st *= o->shape[k]; }
  };
  switch (what) {
    case EVS_ST_T: set(s->off_t, EVS_I32, {B}); return EVS_OK;
    case EVS_ST_IIR_BUF: set(s->off_ib, EVS_I32, {B}); return EVS_OK;
    case EVS_ST_IIR_SLOT: set(s->off_is, EVS_I32, {B}); return EVS_OK;
    case EVS_ST_ERROR: set(s->off_err, EVS_I32, {1}); return EVS_OK;
    case EVS_ST_FIR_RING:
      if (!need_block(EVS_FIR)) return EVS_E_INVALID;
      set(s->ring[block], EVS_F32, {B, s->R[block], d});
      return EVS_OK;
    case EVS_ST_IIR:
      if (!need_block(EVS_IIR)) return EVS_E_INVALID;
      set(s->iir[block], EVS_F32, {B, 2, s->max_block, d, m->blocks[block].iir_states});
      return EVS_OK;
    case EVS_ST_K:
      if (!need_block(EVS_ATTN)) return EVS_E_INVALID;
      set(s->kc[block], dt, {B, m->blocks[block].n_heads, s->cap, m->blocks[block].head_dim});
      return EVS_OK;
    case EVS_ST_VT:
      if (!need_block(EVS_ATTN)) return EVS_E_INVALID;
      set(s->vt[block], dt, {B, m->blocks[block].n_heads, s->cap / 16, m->blocks[block].head_dim, 16});
      return EVS_OK;
    default: return EVS_E_INVALID;
  }
}

evs_status evs_state_error(evs_state* s, int32_t* host_word, int32_t clear, void* stream) {
  if (!s || !host_word) return EVS_E_INVALID;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(hipStreamSynchronize(st));
  HIP_TRY(hipMemcpy(host_word, sp<int>(s, s->off_err), 4, hipMemcpyDeviceToHost));
  if (clear) {
    HIP_TRY(launch_fill_i32(sp<int>(s, s->off_err), 0, 1, st));
    HIP_TRY(hipStreamSynchronize(st));
  }
  return EVS_OK;
}

evs_status evs_prefill(evs_model* m, evs_state* s, const int32_t* tokens, const int32_t* offs, void* last_logits,
                       void* stream) {
  if (!m || !s || !tokens || !offs || s->m != m) return EVS_E_INVALID;
  if (s->pending || !s->wb) return EVS_E_STATE;
  for (int b = 0; b < s->B; ++b)
    if (offs[b + 1] < offs[b] || offs[b] < 0) return EVS_E_INVALID;
  for (int b = 0; b < s->B; ++b)
    if (offs[b + 1] - offs[b] > s->max_ctx) return EVS_E_RANGE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int V = m->desc.vocab;
  if (s->B > 1) {
    // All sequences advance together, P positions per round (one forward and
    // one weight read per round for the whole batch), prompts right-aligned
    // so every last prompt row falls in the final round. Block verify equals
    // sequential decoding bit for bit whatever the chunking, so the state and
    // the last logits are those of per-sequence prefill.
    const int P = std::min(s->max_block, s->max_ctx);
    int R = 0;
    for (int b = 0; b < s->B; ++b) R = std::max(R, (offs[b + 1] - offs[b] + P - 1) / P);
    if (R == 0) return EVS_OK;
    int32_t* pre = wp<int32_t>(s, s->w_pre);
    int32_t *cand = pre, *n_keep = pre + (size_t)s->B * s->max_block, *pick = n_keep + s->B, *doffs = pick + s->B;
    // the offsets are the caller's host memory: the copy has completed when
    // the call returns (a pageable source may be read after an async copy returns)
    HIP_TRY(hipMemcpyAsync(doffs, offs, (size_t)(s->B + 1) * 4, hipMemcpyHostToDevice, st));
    HIP_TRY(hipStreamSynchronize(st));
    for (int j = 0; j < R; ++j) {
      const bool last = j == R - 1;
      HIP_TRY(launch_prefill_round(tokens, doffs, s->B, P, R, j, cand, n_keep, pick, st));
      void* lg = (last && last_logits) ? wp<void>(s, s->w_logit) : nullptr;
      float* ex = (last && s->export_block >= 0) ? s->export_dst : nullptr;
      EVS_TRY(forward_any(m, s, 0, s->B, P, cand, lg, st, ex, 0, -1, pick));
      HIP_TRY(close_span(s));
      HIP_TRY(launch_commit(sp<int>(s, s->off_t), sp<int>(s, s->off_ib), sp<int>(s, s->off_is), n_keep, 0, s->B, P,
                            sp<int>(s, s->off_err), st));
      if (lg) HIP_TRY(launch_pick_rows(lg, last_logits, pick, s->B, P, (size_t)V * m->es, st));
    }
    return EVS_OK;
  }
  const int chunk = s->max_block;
  for (int b = 0; b < s->B; ++b) {
    const int n = offs[b + 1] - offs[b];
    for (int a = 0; a < n; a += chunk) {
      const int P = std::min(chunk, n - a);
      const bool last = a + P == n;
      void* lg = (last && last_logits) ? wp<void>(s, s->w_logit) : nullptr;
      // with the export on, the last chunk also writes the sequence's last
      // prompt row to row b of the export buffer
      float* ex = (last && s->export_block >= 0) ? s->export_dst + (size_t)b * m->desc.d_model : nullptr;
      EVS_TRY(forward_any(m, s, b, 1, P, tokens + offs[b] + a, lg, st, ex, P - 1, 1));
      HIP_TRY(close_span(s));
      HIP_TRY(launch_commit(sp<int>(s, s->off_t) + b, sp<int>(s, s->off_ib) + b, sp<int>(s, s->off_is) + b,
                            nullptr, P, 1, P, sp<int>(s, s->off_err), st));
      if (lg)
        HIP_TRY(launch_copy_row(wp<char>(s, s->w_logit) + (size_t)(P - 1) * V * m->es,
                                reinterpret_cast<char*>(last_logits) + (size_t)b * V * m->es, (size_t)V * m->es, st));
    }
  }
  return EVS_OK;
}

evs_status evs_block_verify(evs_model* m, evs_state* s, const int32_t* cand, int32_t gamma, void* logits,
                            void* stream) {
  if (!m || !s || !cand || !logits || s->m != m) return EVS_E_INVALID;
  if (gamma < 0 || gamma + 1 > s->max_block) return EVS_E_RANGE;
  if (!s->wb) return EVS_E_STATE;
  s->pending = false;   // a pending block is discarded (rollback to 0 changes nothing on device)
  EVS_TRY(forward_any(m, s, 0, s->B, gamma + 1, cand, logits, reinterpret_cast<hipStream_t>(stream),
                      s->export_block >= 0 ? s->export_dst : nullptr));
  HIP_TRY(close_span(s));
  s->pending = true;
  s->pending_P = gamma + 1;
  return EVS_OK;
}

evs_status evs_rollback(evs_state* s, const int32_t* n_keep, void* stream) {
  if (!s) return EVS_E_INVALID;
  if (!s->pending) return EVS_E_STATE;
  HIP_TRY(launch_commit(sp<int>(s, s->off_t), sp<int>(s, s->off_ib), sp<int>(s, s->off_is), n_keep, s->pending_P,
                        s->B, s->pending_P, sp<int>(s, s->off_err), reinterpret_cast<hipStream_t>(stream)));
  s->pending = false;
  return EVS_OK;
}

evs_status evs_block_verify_noalloc(evs_model* m, evs_state* s, const int32_t* cand, int32_t gamma, void* logits,
                                    void* stream) {
  if (!m || !s || !cand || !logits || s->m != m) return EVS_E_INVALID;
  if (gamma < 0 || gamma + 1 > s->max_block) return EVS_E_RANGE;
  if (s->ws_total > (size_t)EVS_NOALLOC_SCRATCH_BYTES) return EVS_E_RANGE;
  char* ws = nullptr;
  EVS_TRY(scratch_ptr(&ws));
  // the same forward over the device scratch; no timing events (creating
  // them could allocate)
  char* own = s->wb;
  const bool timing = s->timing;
  s->wb = ws;
  s->timing = false;
  s->pending = false;
  const evs_status r = forward_any(m, s, 0, s->B, gamma + 1, cand, logits, reinterpret_cast<hipStream_t>(stream),
                                   s->export_block >= 0 ? s->export_dst : nullptr);
  s->wb = own;
  s->timing = timing;
  if (r != EVS_OK) return r;
  s->pending = true;
  s->pending_P = gamma + 1;
  return EVS_OK;
}

evs_status evs_verify_sample(int32_t batch, int32_t gamma, int32_t vocab, const void* target, int32_t kind,
                             const float* q, const int32_t* draft, const float* u, float temperature, int32_t top_k,
                             int32_t greedy, int32_t* n_acc, int32_t* next, int32_t* n_keep, int32_t* err,
                             void* stream) {
  if (batch < 1 || gamma < 0 || gamma > 63 || vocab < 2 || !target || !n_acc || !next) return EVS_E_INVALID;
  if (kind != EVS_TARGET_LOGITS_BF16 && kind != EVS_TARGET_LOGITS_F32 && kind != EVS_TARGET_PROBS_F32)
    return EVS_E_INVALID;
  if (gamma > 0 && !draft) return EVS_E_INVALID;
  if (!greedy && (!u || (gamma > 0 && !q))) return EVS_E_INVALID;
  if (!greedy && kind != EVS_TARGET_PROBS_F32 && !(temperature > 0.f && std::isfinite(temperature)))
    return EVS_E_INVALID;
  if ((long long)(gamma + 2) * vocab > 15360) return EVS_E_UNSUPPORTED;   // LDS: about 60 KB of fp32 rows
  VerifyArgs a{};
  a.gamma = gamma; a.V = vocab; a.kind = kind; a.top_k = top_k; a.greedy = greedy ? 1 : 0;
  a.temperature = temperature; a.target = target; a.q = q; a.draft = draft; a.u = u;
  a.n_acc = n_acc; a.next = next; a.n_keep = n_keep; a.err = err;
  return hip_ok(launch_verify(a, batch, reinterpret_cast<hipStream_t>(stream)));
}

evs_status evs_state_export(evs_state* s, int32_t block, float* dst) {
  if (!s) return EVS_E_INVALID;
  if (block < 0 || !dst) {
    s->export_block = -1;
    s->export_dst = nullptr;
    return EVS_OK;
  }
  if (block >= (int)s->m->plan.size() || ((uintptr_t)dst % 16)) return EVS_E_INVALID;
  s->export_block = block;
  s->export_dst = dst;
  return EVS_OK;
}

evs_status evs_draft(evs_model* m, evs_state* s, int32_t batch, const float* hidden, int32_t hidden_rows,
                     const int32_t* hidden_index, const int32_t* last, int32_t gamma, const float* u,
                     float temperature, int32_t top_k, int32_t greedy, void* logits, int32_t* drafts, float* q,
                     void* stream) {
  if (!m || !s || s->m != m || m->desc.inject_dim <= 0) return EVS_E_INVALID;
  if (!hidden || hidden_rows < 1 || !last || !logits || !drafts || (!greedy && !u)) return EVS_E_INVALID;
  if (!s->wb) return EVS_E_STATE;
  if (!(temperature > 0.f && std::isfinite(temperature))) return EVS_E_INVALID;
  if (batch < 1 || batch > s->B || gamma < 1 || gamma > m->desc.max_slots) return EVS_E_RANGE;
  if (gamma > s->max_block) return EVS_E_RANGE;
  if (m->desc.vocab > 15360) return EVS_E_UNSUPPORTED;   // one fp32 row in LDS
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  evs_status r;
  if (storage_dtype(&m->desc) == EVS_BF16)
    r = draft_pass<bf16>(m, s, batch, hidden, hidden_rows, hidden_index, last, gamma, u, temperature, top_k, greedy,
                         logits, drafts, q, st);
  else
    r = draft_pass<float>(m, s, batch, hidden, hidden_rows, hidden_index, last, gamma, u, temperature, top_k, greedy,
                          logits, drafts, q, st);
  HIP_TRY(close_span(s));
  return r;
}

evs_status evs_generate_workspace_bytes(const evs_model* m, const evs_state* s, const evs_gen_params* p,
                                        const evs_draft_source* d, size_t* bytes) {
  if (!bytes) return EVS_E_INVALID;
  EVS_TRY(gen_check(m, s, p, d));
  *bytes = gen_layout(m, s, p, d).total;
  return EVS_OK;
}

evs_status evs_generate(evs_model* m, evs_state* s, const void* last_logits, const evs_gen_params* p,
                        const evs_draft_source* d, void* work, int32_t* ids, int32_t* stats, int32_t* n_rounds,
                        void* stream) {
  EVS_TRY(gen_check(m, s, p, d));
  if (!last_logits || !work || !ids || !stats || !n_rounds || ((uintptr_t)work % ALIGN)) return EVS_E_INVALID;
  if (s->pending || !s->wb) return EVS_E_STATE;
  *n_rounds = 0;
  const GenLayout L = gen_layout(m, s, p, d);
  char* w = reinterpret_cast<char*>(work);
  auto wi = [&](size_t off) { return reinterpret_cast<int32_t*>(w + off); };
  int32_t *cand = wi(L.cand), *drafts = wi(L.drafts), *n_acc = wi(L.n_acc), *next = wi(L.next),
          *n_keep = wi(L.n_keep), *last = wi(L.last), *idx = wi(L.idx), *emitted = wi(L.emitted);
  void* logits = w + L.logits;
  float* q = reinterpret_cast<float*>(w + L.q);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int B = s->B, g = p->gamma, P = g + 1, V = m->desc.vocab;
  const int src = d ? d->source : EVS_DRAFT_NONE;
  const int kind = storage_dtype(&m->desc) == EVS_BF16 ? EVS_TARGET_LOGITS_BF16 : EVS_TARGET_LOGITS_F32;
  int32_t* err = sp<int>(s, s->off_err);
  const float T = p->temperature;
  // the first token, from the last prompt position's logits
  EVS_TRY(evs_verify_sample(B, 0, V, last_logits, kind, nullptr, nullptr, p->greedy ? nullptr : p->u_first_dev, T,
                            p->top_k, p->greedy, n_acc, next, nullptr, err, stream));
  HIP_TRY(launch_gen_start(next, B, p->n_tokens, ids, last, idx, emitted, stats, st));
  auto round = [&](int r) -> evs_status {
    if (src == EVS_DRAFT_MODEL) {
      // the exported rows: one per sequence after the prefill, the block's after a round
      EVS_TRY(evs_draft(d->drafter, d->drafter_state, B, s->export_dst, r == 0 ? 1 : P, idx, last, g,
                        p->greedy ? nullptr : p->u_draft_dev + (size_t)r * B * g, T, p->top_k, p->greedy,
                        w + L.dlogits, drafts, p->greedy ? nullptr : q, stream));
    }
    const bool table = src == EVS_DRAFT_TABLE;
    HIP_TRY(launch_gen_cand(last, emitted, B, g, table ? d->table_dev : nullptr, table ? d->table_len : 0,
                            (table && d->replace_dev) ? d->replace_dev + (size_t)r * B * g : nullptr, drafts, cand,
                            (table && !p->greedy) ? q : nullptr, V, st));
    EVS_TRY(evs_block_verify(m, s, cand, g, logits, stream));
    EVS_TRY(evs_verify_sample(B, g, V, logits, kind, (p->greedy || g == 0) ? nullptr : q, g > 0 ? drafts : nullptr,
                              p->greedy ? nullptr : p->u_target_dev + (size_t)r * B * P, T, p->top_k, p->greedy,
                              n_acc, next, nullptr, err, stream));
    HIP_TRY(launch_gen_emit(drafts, g, n_acc, next, B, p->n_tokens, ids, emitted, n_keep, last, idx, stats, st));
    return evs_rollback(s, n_keep, stream);
  };
  // Rounds go out in batches without a host read: the sequence furthest from
  // n_tokens needs at least ceil(remaining / (gamma + 1)) more rounds, so a
  // batch of that many never overshoots it; sequences that finish earlier
  // keep nothing in the remaining rounds of the batch.
  std::vector<int32_t> em(B);
  int rounds = 0;
  while (true) {
    HIP_TRY(hipMemcpyAsync(em.data(), emitted, (size_t)B * 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    const int rem = p->n_tokens - *std::min_element(em.begin(), em.end());
    if (rem <= 0) break;
    if (rounds >= p->rounds_cap) {
      *n_rounds = rounds;
      return EVS_E_RANGE;
    }
    const int k = std::min((rem + g) / (g + 1), p->rounds_cap - rounds);
    for (int i = 0; i < k; ++i) {
      EVS_TRY(round(rounds));
      ++rounds;
    }
  }
  *n_rounds = rounds;
  return EVS_OK;
}

evs_status evs_measure_weight_stream(const evs_model* m, int32_t block, int32_t which, void* sink_dev,
                                     size_t sink_bytes, double* bytes_host, void* stream) {
  if (!m || !sink_dev || !bytes_host) return EVS_E_INVALID;
  if (m->desc.dtype != EVS_BF16) return EVS_E_UNSUPPORTED;
  const Mat* mat = nullptr;
  if (which == EVS_W_LM) {
    mat = &m->lm;
  } else {
    if (block < 0 || (size_t)block >= m->plan.size()) return EVS_E_INVALID;
    const BlockPlan& p = m->plan[block];
    const bool mlp = p.d.kind == EVS_MLP;
    if (which == EVS_W_IN && !mlp) mat = &p.w_in;
    else if (which == EVS_W_OUT && !mlp) mat = &p.w_out;
    else if (which == EVS_W_GU && mlp) mat = &p.w_gu;
    else if (which == EVS_W_DOWN && mlp) mat = &p.w_down;
    else return EVS_E_INVALID;
  }
  if (sink_bytes < (size_t)mat->n_groups * 512 * 4) return EVS_E_RANGE;
  // the chunk depth gemm_kernel streams this matrix with at one row tile
  const int CH = mat->NT == 3 ? 1 : 2;
  const MatStrides ms = mat_strides(*mat);
  *bytes_host = (double)mat->bytes(m->es);
  return hip_ok(launch_stream(mat->NT, CH, reinterpret_cast<const uint4*>(m->base + mat->off), ms.g, ms.w, ms.t,
                              mat->steps(m->kstep), mat->n_groups, reinterpret_cast<unsigned*>(sink_dev),
                              reinterpret_cast<hipStream_t>(stream)));
}

evs_status evs_state_timing(evs_state* s, int32_t enable, int64_t context_hint) {
  if (!s) return EVS_E_INVALID;
  HIP_TRY(close_span(s));
  s->timing = enable != 0;
  s->timing_ctx = context_hint;
  return EVS_OK;
}

evs_status evs_state_timing_read(evs_state* s, int32_t kernel_class, double* total_ms, int64_t* launches,
                                 double* bytes, void* stream) {
  if (!s || !total_ms || !launches || !bytes) return EVS_E_INVALID;
  HIP_TRY(close_span(s));
  HIP_TRY(hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)));
  double ms = 0, by = 0;
  int64_t n = 0;
  std::vector<evs_state::Rec> keep;
  for (auto& r : s->recs) {
    if (r.kc != kernel_class) { keep.push_back(r); continue; }
    float e = 0.f;
    HIP_TRY(hipEventElapsedTime(&e, r.a, r.b));
    ms += e;
    by += r.bytes;
    n += r.n;
    s->pool.push_back(r.a);
    s->pool.push_back(r.b);
  }
  s->recs.swap(keep);
  *total_ms = ms;
  *launches = n;
  *bytes = by;
  return EVS_OK;
}

}  // extern "C"
