/*
 * gdn_spec.h -- C ABI of the MI355X (gfx950) GatedDeltaNet speculative
 * verify / commit library (libgdn_spec.so).
 *
 * The step: for every request, the target model scores k+1 verify rows (the
 * pending token and k draft tokens, k <= 8) through each GatedDeltaNet layer,
 * then keeps the first n of them (FreeToken PR #844 "MTP drafts for the
 * Qwen3.5 family and Flash-Next", Summary and Design). n, the accept length,
 * counts the rows a request keeps from one verify, so it never exceeds k+1
 * (same page, End-to-end). Per layer this library does:
 *
 *   gdn_spec_verify  the spec-decode causal conv over [history | rows], SiLU,
 *                    per-key-head L2 norm of q and k, and the gated delta rule
 *                        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *                        o_t = scale * S_t q_t
 *                    on every value head, for all rows; the committed state is
 *                    only read (FreeToken issue #828 "Speculative decoding: MTP
 *                    and DFlash", Design: a verify is a uniform extend of k+1
 *                    rows and only reads the GatedDeltaNet state);
 *   gdn_spec_commit  once the accept lengths are known, writes each request's
 *                    conv history and state as they stand after its n accepted
 *                    rows: by replaying the accepted rows (same Design section)
 *                    or by selecting the state the verify saved after row n-1
 *                    (LightLLM PR #1330 "Qwen3.5 / Qwen3.5-MoE MTP speculative
 *                    decoding", Summary: snapshot/restore of committed state).
 *
 * Conventions carried from the pages:
 *  - per-request state lives in a pool of slots addressed through a slot-id
 *    table (FreeToken PR #844, Design: pools keyed by the target's slot ids;
 *    one upload of the slot and count indices shared by every handler);
 *  - verify request i's scratch is row i of the scratch buffer (same page,
 *    "Flash-Next target verify");
 *  - accept lengths stay on the device and nothing here reads device memory on
 *    the host, so both calls are capture-safe (LightLLM PR #1330, Summary: no
 *    device-to-host syncs, accept_len passed by device pointer);
 *  - arguments that cannot work are refused before anything is launched
 *    (FreeToken PR #844, Summary: rejection at config time).
 *
 * Readings where the pages are silent: x holds the mixed channels
 * [q (HK*d_k) | k (HK*d_k) | v (HV*d_v)]; the conv is depthwise with no bias,
 * conv_w[c][W-1] multiplying the newest input; the conv history holds the
 * last W-1 raw inputs, oldest first; q and k are normalised as
 * x / sqrt(sum x^2 + l2_eps) per key head; value head h uses key head
 * h / (HV/HK); alpha and beta arrive already activated, per (row, value head).
 *
 * Ownership: the caller allocates every buffer (device memory unless stated);
 * the library allocates nothing, keeps no state between calls, never
 * synchronises and never reads device memory on the host. All work is
 * enqueued on `stream` (a hipStream_t; NULL = the null stream).
 */
#ifndef GDN_SPEC_H
#define GDN_SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,       /* null pointer, bad count, misaligned buffer */
    GDN_ERR_UNSUPPORTED = 2,       /* a shape the library has no kernel for */
    GDN_ERR_SCRATCH_TOO_SMALL = 3, /* scratch_bytes below gdn_spec_scratch_bytes() */
    GDN_ERR_HIP = 4                /* the HIP runtime refused a launch */
} gdn_status;

/* Storage type of x, conv history, conv weights, alpha, beta and out. The SSM
 * state is always fp32. bf16 is the upper half of an IEEE fp32 word. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum { GDN_COMMIT_REPLAY = 0, GDN_COMMIT_SNAPSHOT = 1 } gdn_commit_mode;

typedef enum { GDN_ACT_SILU = 0, GDN_ACT_NONE = 1 } gdn_act;

typedef struct {
    int32_t num_k_heads;  /* HK >= 1 */
    int32_t num_v_heads;  /* HV, a multiple of HK */
    int32_t d_k;          /* key head dim; supported: d_k == d_v in {32, 64, 128} */
    int32_t d_v;          /* value head dim */
    int32_t conv_width;   /* W; supported: 4 */
    int32_t dtype;        /* gdn_dtype */
    int32_t act;          /* gdn_act applied after the conv */
    float scale;          /* o = scale * S q */
    float l2_eps;         /* q / sqrt(sum q^2 + l2_eps) */
} gdn_layer_desc;

/*
 * One layer's state pool.
 *  ssm   fp32 [num_slots][HV][d_k][d_v]: head h of slot s stores its d_v x d_k
 *        state S transposed, S[i][j] at ssm[((s*HV + h)*d_k + j)*d_v + i]
 *        (d_v contiguous). 16-byte aligned.
 *  conv  dtype [num_slots][W-1][C], C = 2*HK*d_k + HV*d_v, oldest input first.
 *        16-byte aligned.
 */
typedef struct {
    float *ssm;
    void *conv;
    int32_t num_slots;
} gdn_pool;

/*
 * Bytes of scratch a verify of `batch` requests x `rows` rows needs in `mode`
 * (the commit reads the same buffer). Request b's part is row b. Host only.
 * Returns GDN_ERR_INVALID_ARG / GDN_ERR_UNSUPPORTED for arguments the verify
 * would refuse.
 */
gdn_status gdn_spec_scratch_bytes(const gdn_layer_desc *desc, int32_t batch, int32_t rows,
                                  gdn_commit_mode mode, size_t *bytes);

/*
 * Verify `rows` rows (1..9) of `batch` requests; the pool is only read.
 *  conv_w    dtype [C][W], 16-byte aligned
 *  x         dtype [batch][rows][C]      pre-conv inputs of the verify rows,
 *                                        16-byte aligned
 *  alpha     dtype [batch][rows][HV]     decay gate a_t
 *  beta      dtype [batch][rows][HV]     write strength b_t
 *  slot_ids  int32 [batch]               slot of each request, -1 = padding;
 *                                        distinct within one call
 *  scratch   device buffer of scratch_bytes >= gdn_spec_scratch_bytes(), 16-byte
 *            aligned, left untouched by the caller until the commit
 *  out       dtype [batch][rows][HV][d_v] o of every row (zeros for padding and
 *            bad slots)
 *  err_flag  int32, nullable: bit 0 is OR-ed in when a slot id is outside
 *            [-1, num_slots); that request is skipped.
 */
gdn_status gdn_spec_verify(const gdn_layer_desc *desc, const gdn_pool *pool, const void *conv_w,
                           const void *x, const void *alpha, const void *beta,
                           const int32_t *slot_ids, int32_t batch, int32_t rows,
                           gdn_commit_mode mode, void *scratch, size_t scratch_bytes, void *out,
                           int32_t *err_flag, void *stream);

/*
 * Commit accept_len[b] rows (0..rows; 0 = nothing) of each request verified by
 * the last gdn_spec_verify on this scratch, which must have used the same
 * desc, batch, rows, mode and slot_ids. Writes the pool's conv history and
 * state of each request's slot. Bad slot ids (bit 0) and accept lengths
 * outside [0, rows] (bit 1) are OR-ed into *err_flag and leave that slot
 * untouched. The result is the same in both modes, bit for bit.
 */
gdn_status gdn_spec_commit(const gdn_layer_desc *desc, const gdn_pool *pool,
                           const int32_t *slot_ids, const int32_t *accept_len, int32_t batch,
                           int32_t rows, gdn_commit_mode mode, const void *scratch,
                           size_t scratch_bytes, int32_t *err_flag, void *stream);

/*
 * Commit the previous step's accepted rows and verify this step's rows, in one
 * launch. A layer's commit of step s and its verify of step s+1
 * are adjacent in a serving loop: the verify must read the committed state,
 * and nothing else reads that layer's state in between (FreeToken issue
 * #828, Design: the verify only reads the state and the commit replays the
 * accepted rows; lmdeploy PR #5006, Verification path: a gated-delta-rule
 * verify-and-commit kernel mode). Here each state chunk takes the pending
 * rows' update on its way into the verify (replay mode), or is the previous
 * step's saved S_n to begin with (snapshot mode), and goes back to the pool
 * from there, so the state is read once per step instead of twice. The pool,
 * the outputs and the new scratch are bit for bit those of gdn_spec_commit
 * (previous step) followed by gdn_spec_verify (this step) in the same mode.
 *
 * Arguments as for gdn_spec_verify (batch, rows, mode, slot_ids, x, alpha,
 * beta, scratch, out), plus the previous step's verify:
 *  src_row        int32 [batch]: the previous batch row whose accepted rows
 *                 are still to be committed to slot_ids[b], or -1 (nothing
 *                 pending: the state is read as it is). Ignored for padding
 *                 requests. Distinct within one call.
 *  prev_scratch   the scratch of the previous step's verify (same desc and
 *                 rows, batch prev_batch), prev_scratch_bytes long; must not
 *                 overlap `scratch`. Each buffer holds at least its batch's
 *                 gdn_spec_scratch_bytes(..., mode).
 *  prev_slot_ids  int32 [prev_batch], the previous step's slot table;
 *                 prev_slot_ids[src_row[b]] must equal slot_ids[b].
 *  prev_accept_len int32 [prev_batch], its accept lengths (0..rows).
 *  err_flag       bit 0: slot id outside [-1, num_slots); bit 1: accept
 *                 length outside [0, rows]; bit 2: src_row[b] outside
 *                 [-1, prev_batch) or naming another slot. Such a request is
 *                 skipped: no commit, zero outputs.
 * Rows of the previous batch that no src_row names are not committed here
 * (gdn_spec_commit does that). The previous step must have been a
 * gdn_spec_verify or gdn_spec_commit_verify in the same mode: their scratch
 * also keeps the conv history they read, from which the committed history is
 * built, so no workgroup reads pool history that another is rewriting.
 * Requires bf16 storage, d_k = d_v = 128 and an even number of value heads
 * per key head (GDN_ERR_UNSUPPORTED otherwise).
 */
gdn_status gdn_spec_commit_verify(const gdn_layer_desc *desc, const gdn_pool *pool, const void *conv_w,
                                  const void *x, const void *alpha, const void *beta,
                                  const int32_t *slot_ids, int32_t batch, int32_t rows, gdn_commit_mode mode,
                                  void *scratch, size_t scratch_bytes, const int32_t *src_row,
                                  const void *prev_scratch, size_t prev_scratch_bytes, const int32_t *prev_slot_ids,
                                  const int32_t *prev_accept_len, int32_t prev_batch, void *out, int32_t *err_flag,
                                  void *stream);

/*
 * Commit every GDN layer of a hybrid stack in one launch. Layer l's pool is
 * pools[l] and scratch[l] is the scratch its last gdn_spec_verify used; all
 * layers were verified with the same desc, batch, rows, mode and slot_ids,
 * and share slot_ids and accept_len (FreeToken PR #844, Design: the commit
 * restores the GDN state and every other slot state with one upload of the
 * slot and count indices). The result is that of gdn_spec_commit on each
 * layer in turn, bit for bit.
 *
 *  pools    host array of `layers` pools (device pointers inside; each may
 *           have its own num_slots)
 *  scratch  host array of `layers` device scratch pointers, each at least
 *           scratch_bytes >= gdn_spec_scratch_bytes(desc, batch, rows, mode)
 *  layers   1..64
 * Errors as gdn_spec_commit; any bad layer refuses the whole call before a
 * launch.
 */
gdn_status gdn_spec_commit_layers(const gdn_layer_desc *desc, const gdn_pool *pools,
                                  void *const *scratch, int32_t layers, const int32_t *slot_ids,
                                  const int32_t *accept_len, int32_t batch, int32_t rows,
                                  gdn_commit_mode mode, size_t scratch_bytes, int32_t *err_flag,
                                  void *stream);

/*
 * Another per-slot state a commit restores after the accepted rows: a window
 * of the last `length` entries of a stream (FreeToken PR #844 "MTP drafts for
 * the Qwen3.5 family and Flash-Next", Design: besides the GDN state a slot
 * carries a second conv history and an n-gram context of token ids; the
 * verify stages, per verify row, the entry that row appends, and the commit
 * restores each state as it stands after the accepted rows, with the same
 * upload of the slot and count indices). For request b with slot s and accept
 * length n >= 1, state[s] becomes entries n .. n+length-1 of
 * [state[s] (length entries, oldest first) | rows[b][0..n-1]]; n = 0 leaves it
 * as it is. The GDN conv history is such a window (entries of C channels,
 * length W-1).
 *
 *  state        [num_slots][length][entry_bytes], device, 4-byte aligned,
 *               updated in place
 *  rows         [batch][rows][entry_bytes], device, 4-byte aligned: row t of
 *               request b is the entry verify row t appends
 *  entry_bytes  a positive multiple of 4
 */
typedef struct {
    void *state;
    const void *rows;
    int32_t num_slots;
    int32_t length;
    int32_t entry_bytes;
} gdn_slot_window;

/*
 * Commit every GDN layer of a hybrid stack and every window state in one
 * launch, all sharing slot_ids and accept_len (FreeToken PR #844, Design: the
 * GDN commit and then every other slot state's commit, with one upload of the
 * slot and count indices). The GDN layers are as in gdn_spec_commit_layers
 * (0..64 of them; with none, desc, pools and scratch are not read); the
 * windows (0..16, at least one layer or window in all) follow the rule above.
 * Per request, a slot id outside [-1, num_slots) of a window sets bit 0 of
 * *err_flag and an accept length outside [0, rows] bit 1, and that window of
 * that request is left as it is. No window may overlap a pool, a scratch
 * buffer or another window. Host checks return a status before any launch:
 * GDN_ERR_INVALID_ARG for counts out of range, missing or misaligned
 * pointers, entry_bytes not a positive multiple of 4; GDN_ERR_UNSUPPORTED for
 * a window whose words do not fit an int32 index.
 */
gdn_status gdn_spec_commit_all(const gdn_layer_desc *desc, const gdn_pool *pools, void *const *scratch,
                               int32_t layers, const gdn_slot_window *windows, int32_t num_windows,
                               const int32_t *slot_ids, const int32_t *accept_len, int32_t batch, int32_t rows,
                               gdn_commit_mode mode, size_t scratch_bytes, int32_t *err_flag, void *stream);

/*
 * Greedy acceptance on the device, producing the accept_len that
 * gdn_spec_commit reads. Verify row 0 of request b holds the pending token and
 * row t (1 <= t < rows) the draft token draft[b][t-1]; target[b][t] is the
 * target's greedy token after row t (FreeToken PR #844, Design: the target
 * scores [pending, d1..dk] and n tokens are accepted; FreeToken issue #828,
 * Design: speculative decoding must reproduce greedy decoding token for
 * token). Draft t is accepted while draft[b][t-1] == target[b][t-1] holds for
 * it and every earlier draft, so
 *     accept_len[b] = 1 + (number of leading drafts accepted), in [1, rows],
 *     next_token[b] = target[b][accept_len[b] - 1], the new pending token.
 * A request whose slot id is -1 (padding) gets accept_len 0 and next_token -1.
 *
 *  draft       int32 [batch][rows-1] (may be NULL when rows == 1)
 *  target      int32 [batch][rows]
 *  slot_ids    int32 [batch], nullable (NULL: no padding)
 *  accept_len  int32 [batch], written
 *  next_token  int32 [batch], nullable, written
 * All device memory. Returns GDN_ERR_INVALID_ARG for rows outside [1, 9], a
 * negative batch or a missing required pointer; batch 0 launches nothing.
 */
gdn_status gdn_spec_accept_greedy(const int32_t *draft, const int32_t *target,
                                  const int32_t *slot_ids, int32_t batch, int32_t rows,
                                  int32_t *accept_len, int32_t *next_token, void *stream);

/*
 * Speculative (rejection) sampling on the device: the accept_len that
 * gdn_spec_commit reads, and the next pending token (FreeToken issue #828
 * "Speculative decoding: MTP and DFlash", Plan: target-side verify with
 * rejection sampling and per-row presence and frequency penalties; lmdeploy
 * PR #5006, What's included, Verification path: speculative sampling).
 *
 * Row t of request b (0 <= t < rows) holds the pending token (t = 0) or draft
 * d_t = draft[b][t-1]; its logits give the target distribution of the token
 * after it,
 *     p_t = softmax((l_t - frequency * c_t - presence * [c_t > 0]) / temperature),
 * where c_t[v] = prior_counts[b][v] plus the number of rows 0..t whose token
 * is v (the pending token counts only when given). For t = 0..rows-2, draft
 * d_{t+1} is accepted when u_t * q_t(d_{t+1}) <= p_t(d_{t+1}), i.e. with
 * probability min(1, p/q); q_t is draft_probs[b][t] or, without it, one on
 * d_{t+1} (a greedy drafter). At the first rejection (row t) accept_len is
 * t + 1 and the next token is drawn from max(0, p_t - q_t); with no rejection
 * accept_len is rows and the next token is drawn from p_{rows-1}. The emitted
 * tokens are then distributed as the target's own sampling.
 *
 * Draws are Gumbel-max, argmax_v (log w_v + G_v) with G = -log(-log U). The
 * uniforms come from Philox4x32-10 (Salmon et al., SC'11) with key (seed low
 * word, seed high word): G of row t at entry v from counter (v >> 2, t, b, 0),
 * word v & 3; u_t from counter (0, t, b, 1), word 0; U = (2 (word >> 9) + 1)
 * / 2^24. Pass a new seed for every call.
 *
 * Inputs (device memory; vocab V, at most 2^20):
 *  logits        [batch][rows][V], logits_dtype (GDN_F32 or GDN_BF16), finite
 *  draft_probs   fp32 [batch][rows-1][V], nullable (greedy drafter)
 *  draft         int32 [batch][rows-1] (nullable when rows == 1)
 *  pending       int32 [batch], nullable: the token of row 0, for the counts
 *  prior_counts  int32 [batch][V], nullable: occurrences in the earlier output
 *  temperature   fp32 [batch], finite and > 0
 *  presence, frequency  fp32 [batch], nullable (0)
 *  slot_ids      int32 [batch], nullable: -1 marks padding (accept_len 0,
 *                next_token -1)
 * Outputs: accept_len, next_token int32 [batch]. A request with a temperature
 * that is not finite and > 0, or a draft or pending token outside [0, V), gets
 * accept_len 0 and next_token -1, and bit 3 is OR-ed into *err_flag.
 * scratch: gdn_spec_sample_scratch_bytes() bytes, 16-byte aligned, used
 * within the call only; it needs no clearing (the call resets what it uses),
 * and calls in flight at the same time need buffers of their own. Host checks
 * return a status before any launch.
 */
typedef struct {
    const void *logits;
    const float *draft_probs;
    const int32_t *draft;
    const int32_t *pending;
    const int32_t *prior_counts;
    const float *temperature;
    const float *presence;
    const float *frequency;
    const int32_t *slot_ids;
} gdn_sample_inputs;

gdn_status gdn_spec_sample_scratch_bytes(int32_t batch, int32_t rows, int32_t vocab, size_t *bytes);

gdn_status gdn_spec_accept_sample(const gdn_sample_inputs *in, int32_t logits_dtype, int32_t batch,
                                  int32_t rows, int32_t vocab, uint64_t seed, void *scratch,
                                  size_t scratch_bytes, int32_t *accept_len, int32_t *next_token,
                                  int32_t *err_flag, void *stream);

/* Static description of a status code. */
const char *gdn_strerror(gdn_status status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_SPEC_H */
