/*
 * evs.h — C ABI of the block-verification hot path for hybrid (FIR / IIR /
 * attention) DNA language models, on CDNA4 (gfx950).
 *
 * The operations follow the EvSpark pages:
 *   - block-verification forward over gamma+1 candidate tokens keeping the
 *     inference state of every position, for all three state classes (FIR
 *     sliding windows, IIR modal recurrences, append-only KV caches)
 *     [EvSpark preprint, abstract (i); Evo2 discussion #232, "What we
 *     implemented" and the state-slicing contract, item 1];
 *   - rollback by slicing that state to the accepted boundary, with no replay
 *     and per-sequence boundaries in a batch [same; state-slicing contract,
 *     item 2];
 *   - the exact rejection-sampling verifier and greedy verification
 *     [preprint abstract (iii); discussion #232, "A few other observations";
 *     model card, "Library"].
 *
 * Conventions
 *   Memory   — every buffer is caller-owned device memory passed as a plain
 *              pointer; the library never allocates device memory. Host
 *              handles (evs_model, evs_state) are small host objects.
 *   Streams  — `stream` is a hipStream_t (NULL = default stream). Calls only
 *              enqueue work; none synchronises except evs_state_error,
 *              evs_state_timing_read, evs_generate (between batches of rounds)
 *              and evs_prefill with several sequences (once, for the offsets).
 *   Errors   — argument and state-machine checks run on the host before
 *              anything is enqueued: on failure nothing is enqueued and a
 *              negative evs_status is returned. A failed kernel launch returns
 *              EVS_E_HIP. Conditions only the device can see (a token id out
 *              of range, a context overflow, a device-side n_keep out of
 *              range) are clamped so every access stays in bounds, and set a
 *              bit in the state's sticky error word (evs_state_error).
 *   Threads  — handles are not thread-safe; distinct states may be used on
 *              distinct streams.
 *   Layout   — "storage type" below is bf16 for EVS_BF16 models and fp32 for
 *              EVS_F32 models. Matrices are row-major with y = x W^T.
 */
#ifndef EVS_H
#define EVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EVS_OK = 0,
  EVS_E_INVALID = -1,     /* bad argument (null pointer, bad size, bad descriptor) */
  EVS_E_RANGE = -2,       /* a size exceeds what the state was created for */
  EVS_E_STATE = -3,       /* call out of order (e.g. rollback with nothing pending) */
  EVS_E_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  EVS_E_UNSUPPORTED = -5  /* valid request outside what the library implements */
} evs_status;

/* block kinds */
enum { EVS_FIR = 1, EVS_IIR = 2, EVS_ATTN = 3, EVS_MLP = 4 };
/* storage types; EVS_BF16_FP8W is a model dtype only: a bf16 model whose block
 * projection matrices (w_in, w_out, w_gu, w_down) are held as OCP FP8 E4M3 with
 * one power-of-two scale per output row, the smallest s with max|w| <= 448 s
 * (Evo2 discussion #232, author reply, "Regime overlap": FP8 weights shrink
 * the weight read further; the E4M3 format and the row scaling are this
 * library's choice, the page names neither). evs_pack_weights quantises the
 * bf16 canonical tensors (round to nearest, ties to even); activations,
 * states, embedding and LM head stay bf16 and the accumulation stays fp32. */
enum { EVS_BF16 = 1, EVS_F32 = 2, EVS_I32 = 3, EVS_BF16_FP8W = 4 };
/* target kinds for evs_verify_sample */
enum { EVS_TARGET_LOGITS_BF16 = 1, EVS_TARGET_LOGITS_F32 = 2, EVS_TARGET_PROBS_F32 = 3 };
/* sticky error-word bits */
enum { EVS_ERR_TOKEN = 1, EVS_ERR_CONTEXT = 2, EVS_ERR_NKEEP = 4, EVS_ERR_DRAFT = 8, EVS_ERR_INDEX = 16 };

/* One residual block (pre-norm). FIR: causal depthwise filter of fir_len
 * taps on h = k*v (state: the last fir_len-1 inputs). IIR: diagonal real modal
 * recurrence with iir_states (<= 16) modes per channel (state: the modes).
 * ATTN: causal multi-head attention, n_heads * head_dim = d_model, head_dim a
 * multiple of 32, no positional encoding (state: K and V rows). MLP: gated
 * GELU with d_ff hidden units. */
typedef struct {
  int32_t kind, fir_len, iir_states, n_heads, head_dim, d_ff;
} evs_block_desc;

/* d_model and every d_ff are multiples of 32 (of 64 for EVS_BF16_FP8W);
 * vocab >= 2. inject_dim > 0 makes the model a drafter (EvSpark preprint,
 * abstract (ii); model card, "Drafter checkpoints"): its input rows are built
 * from an injected target hidden state of inject_dim (a multiple of 32)
 * columns, a token embedding and max_slots (1..64) position embeddings, and a
 * full [V, V] Markov matrix follows its head (see evs_draft). Drafters are
 * EVS_BF16 or EVS_F32. inject_dim = max_slots = 0 for a plain model. */
typedef struct {
  int32_t d_model, vocab, n_blocks, dtype;
  float norm_eps;
  const evs_block_desc* blocks;
  int32_t inject_dim, max_slots;
} evs_model_desc;

typedef struct evs_model evs_model;
typedef struct evs_state evs_state;

/* Where a state tensor lives inside the caller's state buffer. */
typedef struct {
  uint64_t offset;      /* byte offset from the start of the state buffer */
  int32_t dtype;        /* EVS_BF16 | EVS_F32 | EVS_I32 */
  int32_t ndim;
  int64_t shape[6];
  int64_t strides[6];   /* in elements */
} evs_tensor_desc;

/* state tensors (evs_state_tensor `what`) */
enum {
  EVS_ST_T = 1,         /* i32 [B]: committed length of each sequence */
  EVS_ST_IIR_BUF = 2,   /* i32 [B]: which IIR buffer holds the committed state */
  EVS_ST_IIR_SLOT = 3,  /* i32 [B]: its position slot, -1 = the zero state */
  EVS_ST_FIR_RING = 4,  /* f32 [B, R, d] (FIR block): row (pos mod R) holds the
                           filter input h at position pos */
  EVS_ST_IIR = 5,       /* f32 [B, 2, max_block, d, N] (IIR block): the state after
                           each position of a block, double-buffered */
  EVS_ST_K = 6,         /* storage [B, H, cap, Dh] (ATTN block): key rows */
  EVS_ST_VT = 7,        /* storage [B, H, cap/16, Dh, 16] (ATTN block): value rows in
                           blocks of 16 positions, each block dimension-major:
                           [b, h, pos/16, e, pos%16] holds V[pos][h][e] */
  EVS_ST_ERROR = 8      /* i32 [1]: sticky error word (EVS_ERR_* bits) */
};

const char* evs_status_string(evs_status s);

/* ------------------------------------------------------------------ model */

/* Number of canonical weight tensors and the shape of tensor i, in the order
 * evs_pack_weights expects them:
 *   embed [V, d];
 *   per block: FIR  w_in [3d, d], taps [d, L] (f32), w_out [d, d];
 *              IIR  w_in [3d, d], lam [d, N] (f32), res [d, N] (f32), w_out [d, d];
 *              ATTN w_in [3d, d] (rows: q, k, v), w_out [d, d];
 *              MLP  w_gu [2 d_ff, d] (gate rows first), w_down [d, d_ff];
 *   lm_head [V, d];
 *   drafters only: inject [d, inject_dim], pos [max_slots, d], markov [V, V] (f32).
 * Matrices are in the storage type; taps/lam/res/markov are always f32. */
evs_status evs_canonical_count(const evs_model_desc* desc, int32_t* count);
evs_status evs_canonical_shape(const evs_model_desc* desc, int32_t i, int64_t* rows,
                               int64_t* cols, int32_t* dtype);

/* Bytes of the packed weight buffer for `desc`. */
evs_status evs_weights_bytes(const evs_model_desc* desc, size_t* bytes);

/* Create a model over a caller-owned packed weight buffer (evs_weights_bytes
 * bytes, 256-byte aligned). The descriptor is copied. */
evs_status evs_model_create(const evs_model_desc* desc, void* packed_dev, evs_model** out);

/* Fill the packed buffer from the canonical tensors (device pointers, order
 * and shapes as in evs_canonical_shape). Enqueued on `stream`; the canonical
 * tensors may be freed once the stream has passed this point. */
evs_status evs_pack_weights(evs_model* m, const void* const* canonical_dev, void* stream);

void evs_model_destroy(evs_model* m);

/* ------------------------------------------------------------------ state */

/* Sizes of the state buffer (persistent across calls) and the workspace
 * (scratch, reused by every call on this state) for `batch` sequences of up
 * to `max_ctx` positions each, processed `max_block` positions per call
 * (max_block = gamma_max + 1 for verification; it also bounds prefill chunks;
 * batch * max_block <= 4096). */
evs_status evs_state_bytes(const evs_model* m, int32_t batch, int32_t max_ctx,
                           int32_t max_block, size_t* state_bytes, size_t* workspace_bytes);

/* Create a state over caller-owned buffers (256-byte aligned) and enqueue their
 * initialisation on `stream`: every sequence empty (t = 0, zero IIR state),
 * error word cleared (the workspace needs no initialisation).
 * workspace_dev may be NULL: the state then has no workspace of its own, and
 * evs_prefill, evs_block_verify and evs_draft on it return EVS_E_STATE; use
 * evs_block_verify_noalloc (and evs_rollback with all positions kept to
 * consume a prompt chunk). */
evs_status evs_state_create(const evs_model* m, int32_t batch, int32_t max_ctx,
                            int32_t max_block, void* state_dev, void* workspace_dev,
                            void* stream, evs_state** out);

void evs_state_destroy(evs_state* s);

/* Location of a state tensor (see EVS_ST_*); `block` selects the block for
 * per-block tensors and is ignored otherwise. Lets a caller inspect the
 * per-position state or import a committed state it synthesised. */
evs_status evs_state_tensor(const evs_state* s, int32_t what, int32_t block,
                            evs_tensor_desc* out);

/* Synchronise `stream`, then read (and with `clear` != 0, reset) the sticky
 * error word. */
evs_status evs_state_error(evs_state* s, int32_t* host_word, int32_t clear, void* stream);

/* --------------------------------------------------------------- hot path */

/* Consume prompt tokens into committed sequences (model card, "Library":
 * generation starts from a prompt, which is consumed before the first round). tokens_dev holds the concatenated
 * prompts (i32); seq_offsets_host[B+1] delimits sequence b's tokens. With
 * several sequences the offsets are copied to the workspace and the call
 * synchronises `stream` once, so the host array may be reused on return. Each sequence's tokens are appended after its
 * committed length. With one sequence, the prompt goes in chunks of at most
 * max_block positions. With several, all sequences advance together in
 * rounds of P = min(max_block, max_ctx) positions, one forward per round for
 * the whole batch. The prompts are right-aligned so that every last prompt
 * token falls in the final round. A sequence's block in a round is its
 * tokens of that round followed by copies of the last one, of which the
 * commit keeps only the tokens. The committed state and the logits equal
 * per-sequence prefill bit for bit. last_logits_dev [B, V] (storage type; may
 * be NULL) receives the logits after each sequence's last token. With the
 * hidden-state export on, row b of the export buffer receives that token's
 * residual row. Rows of sequences with no tokens are left untouched.
 * Requires no pending block. */
evs_status evs_prefill(evs_model* m, evs_state* s, const int32_t* tokens_dev,
                       const int32_t* seq_offsets_host, void* last_logits_dev, void* stream);

/* Block-verification forward. cand_dev [B, gamma+1] (i32) holds, per sequence,
 * the last emitted (not yet consumed) token followed by gamma draft tokens.
 * logits_dev [B, gamma+1, V] (storage type) receives the logits of every
 * candidate position: row i is the next-token distribution after cand[i], so
 * draft i+1 is judged by row i. The state of every position (FIR window rows,
 * IIR modes, KV rows) is written beyond each sequence's committed boundary; the
 * block stays pending until evs_rollback. A call on a pending state first
 * discards the pending block (rollback to 0). 0 <= gamma < max_block. */
evs_status evs_block_verify(evs_model* m, evs_state* s, const int32_t* cand_dev,
                            int32_t gamma, void* logits_dev, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * evs_block_verify with the call's workspace taken from a library-owned device
 * array of EVS_NOALLOC_SCRATCH_BYTES per GPU (resident until the process
 * ends) instead of the state's own workspace, so the state may have been
 * created with workspace_dev = NULL. Results are those of evs_block_verify bit
 * for bit (same kernels, same order). Allocates nothing: no hipMalloc, no
 * hipFree, no event creation (the state's timing is not recorded for it).
 * Errors: as evs_block_verify; EVS_E_RANGE if the state's workspace (see
 * evs_state_bytes) exceeds EVS_NOALLOC_SCRATCH_BYTES; EVS_E_HIP if the scratch
 * address of the current device cannot be looked up. The scratch is shared by
 * every call on one GPU and keeps the last call's contents (nothing in it has
 * to start at zero): calls that overlap on one GPU (other streams, other
 * threads, other states) race and must be serialised by the caller. The state
 * and all pointers must live on the current device. */
#define EVS_NOALLOC_SCRATCH_BYTES (32u << 20)
evs_status evs_block_verify_noalloc(evs_model* m, evs_state* s, const int32_t* cand_dev,
                                    int32_t gamma, void* logits_dev, void* stream);

/* Commit the pending block: sequence b keeps the first n_keep_dev[b] positions
 * (0 .. gamma+1; n_accepted + 1 after a verification). Zero bytes of state are
 * copied: lengths advance and the IIR slot index moves to the kept position.
 * n_keep_dev may be NULL to keep all gamma+1 positions. Device-side values out
 * of range are clamped and flagged (EVS_ERR_NKEEP). */
evs_status evs_rollback(evs_state* s, const int32_t* n_keep_dev, void* stream);

/* Verify a drafted block for `batch` sequences (stateless).
 *   target_dev  [B, gamma+1, V]: logits (bf16 or f32) or probabilities (f32)
 *   q_dev       [B, gamma, V] f32: draft distributions (unused if greedy)
 *   draft_dev   [B, gamma] i32: draft tokens d_1 .. d_gamma
 *   u_dev       [B, gamma+1] f32 in [0,1): u[i] for the accept test of draft
 *               i+1, u[gamma] for the final draw (unused if greedy)
 *   temperature (finite, > 0; checked when sampling from logits) and top_k
 *               (0 or >= V keeps all) apply to logits targets.
 * NaN entries: a NaN logit reads as -inf; a NaN probability (target or draft,
 * greedy or sampling) reads as 0. A target row with no positive probability
 * falls back to its argmax (lowest id on ties).
 * Sampling: accept draft i+1 iff u[i] < p_i[x] / q_i[x] (iff p_i[x] > 0 when
 * q_i[x] = 0); at the first reject draw from max(0, p_i - q_i) normalised
 * (p_i if that is all zero); if all are accepted draw a bonus token from
 * p_gamma. A draw is the inverse CDF with the running fp32 sum in token order.
 * Greedy: accept while the draft equals the argmax (lowest id on ties); emit
 * the argmax at the first mismatch or after the last row.
 * Outputs (i32 [B]): n_accepted, next_token, and n_keep = n_accepted + 1 (may
 * be NULL). Draft ids out of range are clamped and set EVS_ERR_DRAFT in
 * *error_dev if given. Requires gamma <= 63 and (gamma + 2) * V <= 15360. */
evs_status evs_verify_sample(int32_t batch, int32_t gamma, int32_t vocab, const void* target_dev,
                             int32_t target_kind, const float* q_dev, const int32_t* draft_dev,
                             const float* u_dev, float temperature, int32_t top_k, int32_t greedy,
                             int32_t* n_accepted_dev, int32_t* next_token_dev,
                             int32_t* n_keep_dev, int32_t* error_dev, void* stream);

/* ---------------------------------------------------------------- drafter */

/* Hidden-state export for a drafter's prefix (EvSpark preprint, abstract
 * (ii): the drafter reads the target's hidden state; model card, "Drafter
 * checkpoints": injected from layer 27). From now on, every evs_block_verify
 * on `s` also writes the fp32 residual rows after block `block` (0-based
 * index into the descriptor's blocks; for a [mixer, MLP] layer stack, layer L
 * ends at block 2L + 1) to dst_dev [B, gamma+1, d] (row-major f32; row i of
 * sequence b is candidate position i). block = -1 (dst_dev NULL) turns it off.
 * dst_dev must hold B * max_block * d floats and outlive its use. While the
 * export is on, evs_prefill writes each sequence's last prompt row (after
 * block `block`) to dst_dev[b, 0, :] ([B, 1, d]). */
evs_status evs_state_export(evs_state* s, int32_t block, float* dst_dev);

/* Draft gamma tokens for each of B sequences with a drafter model (inject_dim
 * > 0) and its own state `ds` (created for this drafter with batch >= B and
 * max_block >= gamma; never committed: the slots always start at position 0).
 * Steps:
 *   h_b   = hidden_dev[b, idx_b, :] (f32 [B, hidden_rows, inject_dim];
 *           idx_b = hidden_index_dev[b], or 0 if that is NULL; an index outside
 *           0 .. hidden_rows-1 is clamped and sets EVS_ERR_INDEX);
 *   z_b   = rmsnorm(h_b) inject^T, rounded to the storage type;
 *   x_b,i = (embed[last_b] + pos[i]) + z_b for the slots i = 0 .. gamma-1
 *           (last_dev [B] i32: the token each sequence continues from; out of
 *           range reads as 0 and sets EVS_ERR_TOKEN);
 *   the drafter's blocks over the slots (causal), final norm and head -> l_b,i
 *   (written to logits_dev [B, gamma, V], storage type);
 *   Markov head and draws, one slot after another: l' = fp32(l_b,i) +
 *   markov[prev], prev = last_b then each draft; q_b,i = softmax of the top_k
 *   largest of l' / temperature (ties to the lower id; 0 keeps all) with the
 *   verifier's fp32 arithmetic; the draft is the inverse-CDF draw of q_b,i
 *   with u_dev[b, i] (f32 [B, gamma]; the argmax of l' if q has no positive
 *   entry), or the argmax of l' (lowest id) when greedy != 0 (u unused).
 * Outputs: drafts_dev [B, gamma] i32, q_dev [B, gamma, V] f32 (may be NULL).
 * 1 <= gamma <= max_slots; temperature finite and > 0; V <= 15360; errors go
 * to the drafter state's word.
 * The drafter state's timing covers its GEMM and attention launches. */
evs_status evs_draft(evs_model* drafter, evs_state* ds, int32_t batch, const float* hidden_dev,
                     int32_t hidden_rows, const int32_t* hidden_index_dev, const int32_t* last_dev,
                     int32_t gamma, const float* u_dev, float temperature, int32_t top_k, int32_t greedy,
                     void* logits_dev, int32_t* drafts_dev, float* q_dev, void* stream);

/* ------------------------------------------------------------- generation */

/* Where a speculative round's drafts come from. */
enum { EVS_DRAFT_NONE = 0, EVS_DRAFT_MODEL = 1, EVS_DRAFT_TABLE = 2 };

typedef struct {
  int32_t source;               /* EVS_DRAFT_NONE (native decoding: gamma 0), _MODEL or _TABLE */
  /* EVS_DRAFT_MODEL: a drafter (inject_dim = the target's d_model, same vocab)
   * and its own state (batch >= B, max_block >= gamma), run through
   * evs_draft on the target's exported residual rows. The target state's
   * export must be on (evs_state_export) before the prompt's evs_prefill, so
   * that the first round reads each sequence's last prompt row. */
  evs_model* drafter;
  evs_state* drafter_state;
  /* EVS_DRAFT_TABLE: proposals table_dev [B, table_len] (i32) by generated
   * position: after e emitted tokens, draft i (1 .. gamma) is
   * table[b][min(e + i - 1, table_len - 1)]; replace_dev (may be NULL)
   * [rounds_cap, B, gamma] (i32): where an entry is >= 0 it replaces that
   * round's draft. The drafts' q is one-hot (a deterministic drafter). With
   * the target's own greedy continuation as the table this is the identity
   * drafter. */
  const int32_t* table_dev;
  int32_t table_len;
  const int32_t* replace_dev;
} evs_draft_source;

typedef struct {
  int32_t n_tokens;             /* tokens to emit per sequence, >= 1 */
  int32_t gamma;                /* drafts per round (0 .. max_block - 1; 0 with EVS_DRAFT_NONE) */
  int32_t greedy;               /* greedy verification (and greedy drafts) */
  float temperature;            /* finite, > 0 (sampling) */
  int32_t top_k;                /* 0 or >= V keeps all */
  int32_t rounds_cap;           /* rounds the uniform (and replace) arrays cover, >= 1 */
  const float* u_first_dev;     /* [B]: draw of the first token (sampling) */
  const float* u_target_dev;    /* [rounds_cap, B, gamma + 1]: each round's verifier uniforms (sampling) */
  const float* u_draft_dev;     /* [rounds_cap, B, gamma]: each round's drafter uniforms (EVS_DRAFT_MODEL, sampling) */
} evs_gen_params;

/* Bytes of the caller-owned work buffer evs_generate needs. */
evs_status evs_generate_workspace_bytes(const evs_model* m, const evs_state* s, const evs_gen_params* p,
                                        const evs_draft_source* d, size_t* bytes);

/* Generation by speculative rounds (EvSpark model card, "Library": generate,
 * and generate_native with gamma = 0 and EVS_DRAFT_NONE; preprint, abstract
 * (i)). Starts from a state whose prompts were just consumed by evs_prefill,
 * with last_logits_dev [B, V] (storage type) the logits that call returned.
 * The first token of each sequence is drawn from them (argmax when greedy,
 * else the inverse CDF of the target distribution at u_first). Each round r
 * then, on the device: drafts gamma tokens after the last emitted token
 * x_last; runs evs_block_verify on [x_last, drafts]; verifies them
 * (evs_verify_sample, uniforms u_target[r]); emits d_1 .. d_{n_accepted} and
 * the next token, cut at n_tokens (a sequence with r tokens left takes the
 * first r and keeps r block positions); rolls back to the kept positions.
 * Outputs: ids_dev [B, n_tokens] (i32), stats_dev [B, 2] (i32: rounds the
 * sequence took part in, tokens those rounds emitted before the cut, so their
 * ratio is the mean tokens per round), *n_rounds_host. work_dev: at least
 * evs_generate_workspace_bytes bytes, 256-byte aligned. Afterwards the state
 * holds the prompt and every emitted token but the last. Each round needs
 * gamma + 1 free positions past the committed length, so max_ctx must cover
 * the prompt plus n_tokens + gamma; a block that would pass it sets
 * EVS_ERR_CONTEXT in the sticky error word (and is clamped in bounds). Unlike the other
 * calls this one synchronises `stream`: the host reads the emitted counts
 * between batches of rounds to decide how many more to enqueue. Errors:
 * argument checks as listed (EVS_E_STATE: a pending block, a state without a
 * workspace, or a model drafter without the target's export on);
 * EVS_E_RANGE if rounds_cap rounds do not reach n_tokens (the outputs then
 * hold what was emitted). */
evs_status evs_generate(evs_model* m, evs_state* s, const void* last_logits_dev, const evs_gen_params* p,
                        const evs_draft_source* d, void* work_dev, int32_t* ids_dev, int32_t* stats_dev,
                        int32_t* n_rounds_host, void* stream);

/* ------------------------------------------------------------ measurement */

/* kernel classes for per-launch timing */
enum { EVS_KC_GEMM = 1, EVS_KC_ATTN = 2 };

/* Measurement aid: with timing enabled, the GEMM and attention launches made
 * for this state are timed with HIP events on the call's stream and their
 * algorithmic bytes are noted (weights + input rows + output rows for a GEMM;
 * K/V rows up to `context_hint` positions + q + o for attention). Each run of
 * consecutive launches of one class within one API call shares one event
 * pair, so a run's time covers its kernels back to back (including the short
 * gaps between them). Leave it off for headline timing. */
evs_status evs_state_timing(evs_state* s, int32_t enable, int64_t context_hint);

/* projections for evs_measure_weight_stream */
enum { EVS_W_IN = 1, EVS_W_OUT = 2, EVS_W_GU = 3, EVS_W_DOWN = 4, EVS_W_LM = 5 };

/* Measurement aid: enqueue a kernel that reads the packed weights of one
 * projection exactly as the projection's GEMM does (same workgroups, the
 * same contiguous per-wave fragment runs, 16-byte non-temporal loads, the
 * same chunk pipeline at one row tile) and nothing else, so its duration is
 * the weight-read floor of that projection. `block` selects the block (a
 * mixer block for EVS_W_IN / EVS_W_OUT, an MLP block for EVS_W_GU /
 * EVS_W_DOWN; ignored for EVS_W_LM; EVS_E_INVALID if the block has no such
 * projection). sink_dev receives one word per thread, the XOR of every 32-bit
 * word that thread loaded (n_groups * 512 * 4 bytes, workgroup-major;
 * EVS_E_RANGE if sink_bytes is smaller), which keeps the loads from being
 * removed and lets a caller check that exactly the matrix's bytes were read;
 * *bytes_host the weight bytes read. EVS_BF16 models only
 * (EVS_E_UNSUPPORTED otherwise). */
evs_status evs_measure_weight_stream(const evs_model* m, int32_t block, int32_t which, void* sink_dev,
                                     size_t sink_bytes, double* bytes_host, void* stream);

/* Synchronise `stream`, then sum the recorded launches of one kernel class:
 * total device time (ms), number of launches and algorithmic bytes. The
 * records read are cleared. */
evs_status evs_state_timing_read(evs_state* s, int32_t kernel_class, double* total_ms,
                                 int64_t* launches, double* bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EVS_H */
