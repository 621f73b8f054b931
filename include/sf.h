/*
 * sf.h - C ABI of the speculative-decoding verify library for MI355X (gfx950).
 *
 * One decoder stack scores a draft of K tokens in a single pass over K+1
 * positions, takes its own greedy choice at every position, accepts the longest
 * agreeing prefix and rewinds its static KV cache in place.
 *
 * Sources (cited by page title and section):
 *   [ShardFlow] "I Got 28 TPS Out of Free Kaggle GPUs: Here's What It Took"
 *   [Sangama]   "Qwen3.5-397B on 20 GPUs, through a relay"
 *
 * Conventions for every call:
 *   - Returns sf_status: SF_OK (0) or a negative error code.  No C++ exception
 *     crosses this boundary.  sf_last_error() gives a message for the calling
 *     thread's most recent failure.
 *   - Arguments are checked on the host before any device work is enqueued; a
 *     call that fails leaves the committed length and pending token of every
 *     sequence unchanged.
 *   - "host" pointers are ordinary CPU memory owned by the caller and only read
 *     or written during the call.  "device" pointers are HIP device memory owned
 *     by the caller.  Everything else (packed weights, KV pool, scratch,
 *     counters, captured graphs) is owned by the library.
 *   - The library allocates device memory only in sf_model_create(_nf4) and
 *     sf_cache_alloc; every later call reuses fixed addresses, so captured graph
 *     replays stay valid ([ShardFlow] "Why It Kept Breaking (and How I Fixed
 *     It)": captured addresses must not change; fixes 1 and 2).
 *   - All device work runs on the stream given to sf_model_create.  Caller device
 *     buffers are read and written in that stream's order only: work the caller issued
 *     on other streams that writes them (a fill, a copy) must be complete, or ordered
 *     before that stream, when the call is made (sf_kv_write and sf_kv_read excepted:
 *     they wait for the whole device first).
 *   - bf16 = 16-bit brain float stored as uint16 bit patterns.
 */
#ifndef SF_H
#define SF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sf_status;
#define SF_OK          0
#define SF_E_ARG      -1  /* bad argument: null pointer, size, token id, k > k_max, flags */
#define SF_E_CAPACITY -2  /* the pass would write past the cache capacity */
#define SF_E_STATE    -3  /* call not valid in the current state (e.g. rollback past length) */
#define SF_E_HIP      -4  /* a HIP runtime call failed; see sf_last_error() */
#define SF_E_NOMEM    -5  /* device or pinned host allocation failed */

typedef struct sf_model sf_model;   /* opaque, library-owned */
typedef struct sf_cache sf_cache;   /* opaque, library-owned */
typedef struct sf_round sf_round;   /* opaque, library-owned */

/* Decoder shape (Qwen2.5 decoder layer: pre-norm RMSNorm, rotate-half RoPE,
 * grouped-query attention, SwiGLU FFN, optional q/k/v biases). */
typedef struct sf_model_desc {
    int32_t n_layers;
    int32_t hidden;       /* H; multiple of 32 */
    int32_t n_q_heads;
    int32_t n_kv_heads;   /* divides n_q_heads */
    int32_t head_dim;     /* 64 or 128 */
    int32_t ffn;          /* F; multiple of 32 */
    int32_t vocab;        /* V; multiple of 32 */
    float rope_base;
    float rms_eps;
    int32_t has_head;     /* 1: final RMSNorm + LM head + argmax; 0: stack emits hidden states */
    int32_t tied_head;    /* 1: the LM head is the embedding matrix */
    int32_t qkv_bias;     /* 1: q/k/v projections have biases */
} sf_model_desc;

/* sf_model_create: pack the weights into library-owned device memory.
 *   desc     host, read during the call.
 *   weights  host array of device pointers to bf16 tensors in this order
 *            ([out][in] row-major for linear layers):
 *              embed[V][H];
 *              per layer i: ln1[H], wq[nq*dh][H], bq[nq*dh] (if qkv_bias),
 *                wk[nkv*dh][H], bk (if qkv_bias), wv[nkv*dh][H], bv (if qkv_bias),
 *                wo[H][nq*dh], ln2[H], wg[F][H], wu[F][H], wd[H][F];
 *              final_norm[H] (if has_head); lm_head[V][H] (if has_head and not tied_head).
 *            The tensors are copied; the caller may free them after the call.
 *   stream   a hipStream_t (NULL: the library creates its own non-blocking stream).
 *   out      receives the model handle.
 * Errors: SF_E_ARG for unsupported shapes, SF_E_NOMEM, SF_E_HIP. */
sf_status sf_model_create(const sf_model_desc* desc, const void* const* weights, void* stream,
                          sf_model** out);

/* sf_model_create_nf4: as sf_model_create, with the seven projections of every layer (wq,
 * wk, wv, wo, wg, wu, wd) in 4-bit NormalFloat ([ShardFlow] "The Numbers": the 14.7B model
 * run with 4-bit NF4 quantization).  Each projection takes two consecutive entries of
 * `weights` in place of one:
 *   codes   device uint8 [out][in/2]: the 4-bit code of input k of a row in byte k/2, the
 *           even input in the low nibble;
 *   scales  device bf16 [out][in/64]: one scale per 64 consecutive inputs of a row.
 * The weight of code c in block b is level[c] * scale[b], level[] the table sf_nf4_levels
 * returns.  Embedding, norms, biases and the LM head stay bf16.  The library packs each
 * 32-row x 64-input block as 1 KB of codes in MFMA operand order plus the 32 row scales and
 * turns codes into bf16 levels inside the GEMM (weights are read once per pass at about
 * 0.53 bytes per weight).  Needs hidden, ffn and n_q_heads*head_dim to be multiples of 64;
 * caches of an NF4 model run passes of at most 64 rows (n_seqs*(k_max+1) <= 64, prefill
 * passes of 64 positions).  Errors as sf_model_create. */
sf_status sf_model_create_nf4(const sf_model_desc* desc, const void* const* weights, void* stream,
                              sf_model** out);

/* sf_nf4_levels: the 16 NF4 levels the library decodes codes 0..15 to (host float out[16]):
 * quantiles of the standard normal distribution at evenly spaced probabilities, 8 positive
 * and 7 negative plus an exact zero, normalised to [-1, 1] (the QLoRA paper's 4-bit
 * NormalFloat), each rounded to bf16.  Callers quantize with this table.  Errors: SF_E_ARG. */
sf_status sf_nf4_levels(float* out);

sf_status sf_model_free(sf_model* model);

/* sf_cache_alloc: static KV pool for n_seqs sequences of `capacity` positions
 * each, plus all scratch, device counters and the captured verify (T = k_max+1)
 * and single-token draft (T = 1) graphs ([ShardFlow] "Why It Kept Breaking":
 * fix 1, a pre-allocated fixed-size cache).  Every sequence starts with length 0
 * and pending token 0.  KV layout: [layer][seq][kv_head][position][head_dim] bf16;
 * K is stored after RoPE.
 * Scratch is sized for passes of max(n_seqs*(k_max+1), prefill pass size) rows.
 * Limits: 1 <= n_seqs <= 64, n_seqs * (k_max+1) <= 512, 0 <= k_max <= 15,
 * k_max+1 <= capacity <= 16384. */
sf_status sf_cache_alloc(sf_model* model, int32_t n_seqs, int32_t capacity, int32_t k_max,
                         sf_cache** out);
sf_status sf_cache_free(sf_cache* cache);

/* sf_prefill: score the prompt tokens[0..n) of sequence `seq` from position 0
 * (any previous content of that sequence is discarded) and commit all of them.
 * Afterwards length = n and the pending token is the greedy choice after the
 * last prompt token, returned in *next_token (host, may be NULL; hidden-state
 * stacks return 0).  [Sangama] "What made it faster", item 4, splits long prompts into
 * 64-token pieces so that pipeline stages work on different pieces at once; on one GPU
 * there is no pipeline to fill, so up to eight such pieces (512 positions) go through
 * one pass together, which lets each weight byte serve 512 rows.  Not graph-captured.  The
 * pass size (1..512) can be lowered for a cache by setting SF_PREFILL_CHUNK in the
 * environment before sf_cache_alloc; results are bit-identical
 * for any pass size.  Only the last position's logits are computed: earlier passes skip
 * the LM head, and the last one runs it for the rows it needs.
 * Errors: SF_E_ARG (token id outside [0,V), n < 1), SF_E_CAPACITY (n > capacity). */
sf_status sf_prefill(sf_cache* cache, int32_t seq, const int32_t* tokens, int32_t n,
                     int32_t* next_token);

/* Flags of sf_verify / sf_verify_device. */
#define SF_NO_COMMIT     1u  /* do not advance length / pending token (the pass still writes KV past length) */
#define SF_FORCE_ACCEPT  2u  /* accept all k drafts (feed known tokens) */
#define SF_DEBUG_LOGITS  4u  /* eager launch that also writes fp32 logits to dev_out */

/* sf_verify: one verify pass for every sequence of the cache ([ShardFlow]
 * "Speculative Decoding: The Idea": all K guesses checked in one pass;
 * [Sangama] "Speculative decoding: correct, but slower (for now)": the model's
 * own choice is returned at every position).
 *   draft     host int32 [n_seqs][k_max]: d_1..d_k of each sequence (slots past k ignored).
 *   k         host int32 [n_seqs] drafts per sequence (0..k_max), or NULL for k_max.
 *   flags     SF_* above.
 *   accepted  host int32 [n_seqs] (may be NULL): M, the number of leading drafts
 *             equal to the model's greedy choice, capped at k.
 *   target    host int32 [n_seqs][k_max+1] (may be NULL): the greedy choice at
 *             positions L..L+k_max, where L is the length before the call; slot j
 *             is the choice for the token after draft j (slot 0: after the pending token).
 *   dev_out   device pointer or NULL.  Hidden-state stacks: bf16 [n_seqs][k_max+1][H]
 *             residual stream after the last layer.  With SF_DEBUG_LOGITS: fp32
 *             [n_seqs][k_max+1][V] logits.
 * The pass feeds [pending, d_1..d_k, 0...] at positions L..L+k_max.  On commit
 * (default) a stack with a head sets length = L+M+1 and pending = target[M]
 * (M accepted drafts plus the model's own token at the first mismatch); a
 * hidden-state stack sets length = L+k+1 and leaves the decision to the caller
 * (sf_rollback + sf_set_next).  Positions past the new length keep stale KV that
 * later passes overwrite.  Replays a captured graph unless SF_DEBUG_LOGITS is set.
 * Returns after the results have been copied back.
 * Errors: SF_E_ARG, SF_E_CAPACITY (L + k_max + 1 > capacity for some sequence). */
sf_status sf_verify(sf_cache* cache, const int32_t* draft, const int32_t* k, uint32_t flags,
                    int32_t* accepted, int32_t* target, void* dev_out);

/* sf_verify_device: enqueue one verify pass whose drafts are already in device
 * memory, without waiting (inputs resident in HBM; results stay on the device).
 *   dev_draft  device int32 [n_seqs][k_max]; dev_k device int32 [n_seqs] or NULL (k_max).
 *   Drafts are copied into the library's fixed staging buffer on the stream, then
 *   the captured graph is replayed.  Token ids are not range-checked here (they
 *   are never read on the host); ids outside [0,V) are clamped by the kernels, and a k
 *   outside 0..k_max by the accept step (the checking build records both: sf_debug_checks).
 *   Results: see sf_results_device.  Host-side length bookkeeping assumes the
 *   worst case (length + k_max + 1 per committing call) until sf_sync.
 * Errors: SF_E_ARG, SF_E_CAPACITY. */
sf_status sf_verify_device(sf_cache* cache, const int32_t* dev_draft, const int32_t* dev_k,
                           uint32_t flags);

/* sf_verify_device_static: sf_verify_device's pass for callers that cannot allocate device
 * memory or call anything that does (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels, enqueued eagerly on the model stream
 * without waiting, with the pass's working memory (activations, split-K partials and
 * counters, attention partials, LM-head maxima, staging block) taken from one static device
 * array of 16 MiB per GPU instead of the cache's own scratch; no hipMalloc, hipFree or other
 * allocating call is made (the array's device address is looked up once per device, on the
 * first call there).
 *   dev_draft, dev_k, flags  as sf_verify_device (SF_NO_COMMIT, SF_FORCE_ACCEPT).
 *   dev_result  device int32 [n_seqs + n_seqs*(k_max+1)], caller-owned: accepted[n_seqs]
 *               then target[n_seqs][k_max+1], written by the pass (results are not placed at
 *               sf_results_device's address).
 * The cache's KV pool, lengths and pending tokens are read and committed exactly as by
 * sf_verify_device, and the results are bit-identical to it.  Limit: the pass's working
 * memory must fit the array (a single-sequence 7B-shape K=8 verify at capacity 8208 needs
 * about 9.4 MB; 32-sequence batches do not fit) -- larger passes fail with SF_E_CAPACITY
 * before any work is enqueued.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents: calls whose passes overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.
 * Errors: SF_E_ARG, SF_E_CAPACITY, SF_E_HIP. */
sf_status sf_verify_device_static(sf_cache* cache, const int32_t* dev_draft, const int32_t* dev_k,
                                  uint32_t flags, int32_t* dev_result);

/* sf_results_device: device addresses (fixed for the cache's lifetime) of the
 * last pass's results: accepted int32 [n_seqs] and target int32 [n_seqs][k_max+1]. */
sf_status sf_results_device(sf_cache* cache, int32_t** dev_accepted, int32_t** dev_target);

/* sf_rollback: in-place rewind of sequence `seq` to length `pos` (0 <= pos <=
 * length).  An index write only: no KV data moves ([ShardFlow] "Why It Kept
 * Breaking": fix 4, in-place KV rewind).  The pending token is unchanged.
 * Errors: SF_E_ARG (bad seq), SF_E_STATE (pos > length or pos < 0). */
sf_status sf_rollback(sf_cache* cache, int32_t seq, int32_t pos);

/* sf_snapshot_save: record, for every sequence, its length, pending token and the K/V
 * rows of every layer at positions [length, length+k_max+1): the state one verify pass
 * overwrites.  sf_snapshot_restore puts all of it back.  Together with a replay of the
 * accepted drafts (sf_verify with SF_FORCE_ACCEPT and k = accepted count) this is the
 * pages' other rollback ([Sangama] "Speculative decoding: correct, but slower (for now)":
 * each worker saves a snapshot of its state before checking the guesses and, when some
 * were wrong, restores it and replays only the accepted tokens locally), the form needed by
 * stacks whose state cannot be rewound by an index.  For this attention-only stack it
 * reaches bit-identical state to sf_rollback's index rewind at the cost of the replay
 * pass.  Both calls are enqueued on the model stream without waiting; restore marks the
 * host view of the state stale.  One snapshot per cache; a save replaces the previous one.
 * Errors: SF_E_ARG (NULL), SF_E_STATE (restore before any save), SF_E_HIP. */
sf_status sf_snapshot_save(sf_cache* cache);
sf_status sf_snapshot_restore(sf_cache* cache);

/* sf_set_next: set the pending token of `seq` (the token the next pass places at
 * position `length`).  Errors: SF_E_ARG (bad seq or token outside [0,V)). */
sf_status sf_set_next(sf_cache* cache, int32_t seq, int32_t token);

/* sf_cache_state: waits for the stream, then returns the committed length and
 * pending token of `seq` (host outputs, either may be NULL). */
sf_status sf_cache_state(sf_cache* cache, int32_t seq, int32_t* length, int32_t* next_token);

/* sf_draft_step: n_steps greedy single-token passes for every sequence, each a
 * replay of the captured T = 1 graph (whole forward + LM head + argmax + commit:
 * [ShardFlow] "CUDA Graphs: What They Are and Why They Helped").  tokens: host
 * int32 [n_seqs][n_steps] receives the generated tokens (may be NULL).  Each step
 * commits: length += 1, pending = the new token.
 * Errors: SF_E_STATE (hidden-state stack), SF_E_ARG (n_steps < 1 or > 256),
 * SF_E_CAPACITY (length + n_steps > capacity). */
sf_status sf_draft_step(sf_cache* cache, int32_t n_steps, int32_t* tokens);

/* sf_round_create: a device-resident speculative round over a drafter cache `drafter` and a
 * verifier cache `verifier` holding the same sequences ([ShardFlow] "Speculative Decoding: The
 * Idea": a small model guesses k tokens, the large one checks them in one pass and the agreed
 * prefix is committed; "CUDA Graphs: What They Are and Why They Helped": the whole round is one
 * captured graph, with no host round trip between its steps).  One round, for every sequence:
 *   1. k greedy drafter steps (as sf_draft_step) from the shared pending token;
 *   2. one verifier pass over [pending, d_1..d_k] (as sf_verify), accepting M drafts and
 *      committing length += M+1, pending = target[M];
 *   3. the drafter rewound in place to the committed stream ([ShardFlow] "Why It Kept
 *      Breaking", fix 4): length L+M+1 and pending target[M]; when all k drafts were accepted
 *      it first feeds its last draft d_k (one non-committing step counted afterwards).
 * Both models must share one stream (the stream given to sf_model_create), both stacks need
 * an LM head, the drafter's vocabulary may not exceed the verifier's (shared token ids; a
 * verifier token beyond the drafter's table, a padding row that a trained head never picks,
 * embeds as the drafter's last row), the caches hold the same n_seqs, and 1 <= k <= the
 * verifier's k_max.  The round object holds the graph and 2*n_seqs ints of device scratch;
 * it does not own the caches, which must outlive it.
 * Errors: SF_E_ARG, SF_E_STATE (a stack without a head), SF_E_NOMEM, SF_E_HIP. */
sf_status sf_round_create(sf_cache* drafter, sf_cache* verifier, int32_t k, sf_round** out);

/* sf_round_run: enqueue n_rounds rounds (graph replays) without waiting.  Before the first,
 * every sequence's drafter and verifier must be at the same point (equal length and pending
 * token, e.g. after the same sf_prefill on both).  Afterwards the verifier's last results are
 * at sf_results_device(verifier) and sf_cache_state reads either cache's position.
 * Errors: SF_E_ARG, SF_E_STATE (caches not at the same point), SF_E_CAPACITY (n_rounds*(k+1)
 * more positions, plus one verify, might not fit a cache). */
sf_status sf_round_run(sf_round* round, int32_t n_rounds);

/* sf_round_free: waits for the stream, then releases the round (not the caches). */
sf_status sf_round_free(sf_round* round);

/* sf_ngram_propose: prompt-lookup drafter ([Sangama] "Speculative decoding:
 * correct, but slower (for now)": if the last 2-4 tokens appeared earlier, guess
 * what followed them then).  Host only.  For n = max_n down to min_n, finds the
 * most recent earlier start j < n_hist-n with hist[j..j+n) equal to the last n
 * tokens and writes hist[j+n .. min(j+n+k_max, n_hist)) to out (host int32
 * [k_max]).  Returns the number of proposed tokens (0..k_max), or SF_E_ARG. */
int32_t sf_ngram_propose(const int32_t* hist, int32_t n_hist, int32_t min_n, int32_t max_n,
                         int32_t k_max, int32_t* out);

/* sf_kv_write / sf_kv_read: copy positions [0, n_pos) of sequence `seq` between
 * the KV pool and caller device buffers k, v laid out bf16
 * [n_layers][n_kv_heads][src_positions][head_dim] (src_positions >= n_pos).
 * sf_kv_write also sets length = n_pos (pending token unchanged).  Both first wait for
 * all work on the device (the buffers may have been written or filled on any stream),
 * copy on the model stream, and return when the copy is done.
 * Errors: SF_E_ARG, SF_E_CAPACITY (n_pos > capacity). */
sf_status sf_kv_write(sf_cache* cache, int32_t seq, const void* dev_k, const void* dev_v,
                      int32_t n_pos, int32_t src_positions);
sf_status sf_kv_read(sf_cache* cache, int32_t seq, void* dev_k, void* dev_v, int32_t n_pos,
                     int32_t dst_positions);

/* sf_sync: wait for all work on the stream; refresh host-side length bookkeeping. */
sf_status sf_sync(sf_cache* cache);

/* Kernels that sf_time_kernel can time, each at the verify shape (rows =
 * n_seqs*(k_max+1)), cycling through the layers so weights come from HBM. */
#define SF_KERNEL_QKV        0
#define SF_KERNEL_ATTENTION  1
#define SF_KERNEL_OPROJ      2
#define SF_KERNEL_GATEUP     3
#define SF_KERNEL_DOWN       4
#define SF_KERNEL_LMHEAD     5
/* The whole verify pass as captured (a replay of the verify graph with commit off). */
#define SF_KERNEL_VERIFY     6

/* sf_time_kernel: launch one kernel of the verify pass `iters` times back to back
 * on the library stream between two HIP events and return the mean time per
 * launch in microseconds (host *avg_us) and the algorithmic bytes one launch
 * must move (host *bytes: weights once, activations once, KV once; for
 * SF_KERNEL_VERIFY: every weight once, K/V of positions 0..len+k_max read once per
 * layer and the new positions written once).
 * Overwrites scratch and the staged drafts (SF_KERNEL_VERIFY stages k = 0 with commit
 * off), so call it between passes only. */
sf_status sf_time_kernel(sf_cache* cache, int32_t kernel, int32_t iters, float* avg_us,
                         double* bytes);

/* sf_debug_counters: waits for the stream, then reports the sum and the largest value of
 * the cache's k-split arrival counters (host *sum, *max).  The last of the workgroups
 * splitting an output block resets its counter, so both are 0 between passes; a test reads
 * them to check that no counter grows from pass to pass.  Errors: SF_E_ARG, SF_E_HIP. */
sf_status sf_debug_counters(sf_cache* cache, int64_t* sum, int32_t* max);

/* Bits of sf_debug_checks: invariants the kernels of a checking build record when violated
 * (they still clamp or skip as the regular build does; nothing traps). */
#define SF_CHECK_TOKEN   1u   /* a token id outside [0, vocab) reached the embedding (clamped) */
#define SF_CHECK_K       2u   /* a staged draft count outside [0, k_max] (clamped by the accept) */
#define SF_CHECK_POS     4u   /* a K/V append or attention row at or past the capacity (skipped) */
#define SF_CHECK_COMMIT  8u   /* a commit that would move a length past the capacity */
#define SF_CHECK_NAN    16u   /* a NaN logit in the LM head's output */

/* sf_debug_checks: the checking build (libsf_checks.so, built by `build.py --checks` and by
 * the package build) records the SF_CHECK_* invariants above in one word per device instead
 * of only clamping; this waits for the device, returns the word of the current device (host
 * *bits) and with clear != 0 sets it to zero.  For callers that feed device-resident inputs
 * (sf_verify_device, sf_round_run) which the host cannot check.  The regular build returns
 * SF_E_STATE ("built without device checks") and *bits = 0.  Errors: SF_E_ARG, SF_E_HIP. */
sf_status sf_debug_checks(uint32_t* bits, int32_t clear);

/* Error injection for tests of the failure path: with SF_FAULT=alloc in the environment every
 * device allocation of sf_model_create(_nf4), sf_cache_alloc and sf_round_create fails as an
 * out-of-memory hipMalloc would (SF_E_NOMEM, nothing left allocated); with SF_FAULT=launch
 * every graph replay and eager pass fails as a failed launch would (SF_E_HIP), before the
 * call changes any sequence's length or pending token.  Read at every use. */

/* sf_last_error: message of the calling thread's last failed call ("" if none). */
const char* sf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SF_H */
