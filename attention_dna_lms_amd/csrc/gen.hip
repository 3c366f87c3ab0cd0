// Device side of the generation loop (evs_generate): the first token's
// bookkeeping, the candidate block of each round, and the emission of each
// round's tokens with the truncation at n_tokens. Every decision that depends
// on the verifier's output stays on the device, so rounds are enqueued back
// to back without the host reading anything.
#include "evs_dev.h"

namespace evs {

// After the first draw (next = the token drawn from the last prompt
// position's logits): it is the first emitted token and the last, not yet
// consumed one.
__global__ void gen_start_kernel(const int* next, int B, int n_tokens, int* ids, int* last, int* idx, int* emitted,
                                 int* stats) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int x = next[b];
  ids[(size_t)b * n_tokens] = x;
  last[b] = x;
  idx[b] = 0;
  emitted[b] = 1;
  stats[2 * b] = 0;
  stats[2 * b + 1] = 0;
}

hipError_t launch_gen_start(const int* next, int B, int n_tokens, int* ids, int* last, int* idx, int* emitted,
                            int* stats, hipStream_t st) {
  gen_start_kernel<<<(B + 255) / 256, 256, 0, st>>>(next, B, n_tokens, ids, last, idx, emitted, stats);
  return hipGetLastError();
}

// The round's candidate block [x_last, d_1 .. d_gamma] per sequence. Table
// drafts: after e emitted tokens draft i is table[b][e + i - 1] (clamped to
// the table's end), replaced by replace[b][i] where that is >= 0; q (if not
// null) is one-hot at each table draft. Model drafts are already in `drafts`.
// One workgroup per sequence.
__global__ void gen_cand_kernel(const int* last, const int* emitted, int gamma, const int* table, int table_len,
                                const int* replace, int* drafts, int* cand, float* q, int V) {
  const int b = blockIdx.x, P = gamma + 1;
  const int e = emitted[b];
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    int tok;
    if (i == 0) {
      tok = last[b];
    } else {
      if (table) {
        const int k = min(e + i - 1, table_len - 1);
        tok = table[(size_t)b * table_len + k];
        if (replace) {
          const int r = replace[(size_t)b * gamma + i - 1];
          tok = r >= 0 ? r : tok;
        }
        drafts[(size_t)b * gamma + i - 1] = tok;
      } else {
        tok = drafts[(size_t)b * gamma + i - 1];
      }
    }
    cand[(size_t)b * P + i] = tok;
  }
  if (q && table) {
    __syncthreads();   // the drafts of this sequence are written
    for (int j = threadIdx.x; j < gamma * V; j += blockDim.x) {
      const int i = j / V, y = j % V;
      q[(size_t)b * gamma * V + j] = y == drafts[(size_t)b * gamma + i] ? 1.f : 0.f;
    }
  }
}

hipError_t launch_gen_cand(const int* last, const int* emitted, int B, int gamma, const int* table, int table_len,
                           const int* replace, int* drafts, int* cand, float* q, int V, hipStream_t st) {
  gen_cand_kernel<<<B, 256, 0, st>>>(last, emitted, gamma, table, table_len, replace, drafts, cand, q, V);
  return hipGetLastError();
}

// A round's emission: d_1 .. d_{n_acc} and the verifier's next token, cut at
// n_tokens. A sequence with r tokens still to emit takes the first
// take = min(n_acc + 1, r) of them and keeps take positions of the block
// (x_last, d_1 .. d_{take-1}); its new x_last is the last token taken, and
// the drafter reads the residual row at block position take - 1 next. A
// finished sequence keeps nothing. stats[b] = (rounds, tokens the rounds
// emitted before truncation).
__global__ void gen_emit_kernel(const int* drafts, int gamma, const int* n_acc, const int* next, int B, int n_tokens,
                                int* ids, int* emitted, int* n_keep, int* last, int* idx, int* stats) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int e = emitted[b], rem = n_tokens - e;
  if (rem <= 0) {
    n_keep[b] = 0;
    return;
  }
  const int na = min(max(n_acc[b], 0), gamma), out = na + 1;
  const int take = min(out, rem);
  int tok = 0;
  for (int j = 0; j < take; ++j) {
    tok = j < na ? drafts[(size_t)b * gamma + j] : next[b];
    ids[(size_t)b * n_tokens + e + j] = tok;
  }
  emitted[b] = e + take;
  n_keep[b] = take;
  last[b] = tok;
  idx[b] = take - 1;
  stats[2 * b] += 1;
  stats[2 * b + 1] += out;
}

hipError_t launch_gen_emit(const int* drafts, int gamma, const int* n_acc, const int* next, int B, int n_tokens,
                           int* ids, int* emitted, int* n_keep, int* last, int* idx, int* stats, hipStream_t st) {
  gen_emit_kernel<<<(B + 255) / 256, 256, 0, st>>>(drafts, gamma, n_acc, next, B, n_tokens, ids, emitted, n_keep,
                                                   last, idx, stats);
  return hipGetLastError();
}

// Batched prefill, round j of R lockstep rounds of P positions over all
// sequences. The prompts are right-aligned: sequence b with n tokens covers
// positions [max(e - P, 0), max(e, 0)) in round j, e = n - (R - 1 - j) * P, so
// its first chunk is the partial one and its last token falls in round R - 1.
// Its block is those tokens followed by copies of the last one (the commit
// keeps only n_keep = their count); pick = the block row of its last token in
// this round, -1 if it has none. One workgroup per sequence.
__global__ void prefill_round_kernel(const int* tokens, const int* offs, int P, int R, int j, int* cand, int* n_keep,
                                     int* pick) {
  const int b = blockIdx.x;
  const int o = offs[b], n = offs[b + 1] - o;
  const int e = n - (R - 1 - j) * P;
  const int s0 = max(e - P, 0), v = max(e, 0) - s0;
  for (int i = threadIdx.x; i < P; i += blockDim.x) cand[(size_t)b * P + i] = v > 0 ? tokens[o + s0 + min(i, v - 1)] : 0;
  if (threadIdx.x == 0) {
    n_keep[b] = v;
    pick[b] = v - 1;
  }
}

hipError_t launch_prefill_round(const int* tokens, const int* offs, int B, int P, int R, int j, int* cand,
                                int* n_keep, int* pick, hipStream_t st) {
  prefill_round_kernel<<<B, 64, 0, st>>>(tokens, offs, P, R, j, cand, n_keep, pick);
  return hipGetLastError();
}

// dst row b = src row b * P + pick[b] (row_bytes each), for the sequences with
// pick[b] >= 0 (the last prompt row's logits of a batched prefill)
__global__ void pick_rows_kernel(const unsigned char* src, unsigned char* dst, const int* pick, int P,
                                 size_t row_bytes) {
  const int b = blockIdx.x, r = pick[b];
  if (r < 0) return;
  const unsigned char* sr = src + ((size_t)b * P + r) * row_bytes;
  unsigned char* dr = dst + (size_t)b * row_bytes;
  for (size_t i = threadIdx.x; i < row_bytes; i += blockDim.x) dr[i] = sr[i];
}

hipError_t launch_pick_rows(const void* src, void* dst, const int* pick, int B, int P, size_t row_bytes,
                            hipStream_t st) {
  pick_rows_kernel<<<B, 256, 0, st>>>(reinterpret_cast<const unsigned char*>(src),
                                      reinterpret_cast<unsigned char*>(dst), pick, P, row_bytes);
  return hipGetLastError();
}

}  // namespace evs
