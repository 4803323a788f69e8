/*
 * idlm_isd.h -- C ABI of libidlm_isd.so, the MI355X (gfx950) ISD step.
 *
 * One Introspective Strided Decoding (ISD) step verifies the previous
 * step's drafts and proposes new ones in a single forward.  The library
 * implements the data-parallel part of that step on one GPU:
 *
 *   1. idlm_isd_paged_attn: strictly causal grouped-query attention of the
 *      2N-1 step rows of every sequence over a paged KV cache.  Causal
 *      attention over all positions is what lets the model run in an
 *      autoregressive serving stack ("Introspective Diffusion Language
 *      Models", sections "Training" and "Serving (SGLang)"); a forward
 *      carries 2N-1 queries (section "How do DLMs perform as they approach
 *      compute-bound?"); the cache is paged ("Serving (SGLang)").
 *   2. idlm_isd_accept: the acceptance stage.  Clean rows give the anchor
 *      distribution p, MASK rows the proposal distribution q; draft x is
 *      kept with probability min(1, p(x)/q(x)), the first rejection is
 *      resampled from normalize(max(0, p - q)), and the committed prefix is
 *      truncated there ("Introspective Diffusion Language Models", section
 *      "Inference & ISD"; GeekNews summary, section "Inference & ISD").
 *   3. idlm_isd_step: 1 and 2 side by side (they are independent).
 *   4. idlm_isd_propose: the next step's drafts from this forward's MASK
 *      rows, or a fresh step after a rejection; it can record the MASK
 *      rows' statistics, which the next acceptance then does not recompute.
 *      idlm_isd_loop_step: 3 and 4 in one call, the proposals beside the
 *      attention.
 *   5. idlm_isd_gated_lora: R-ISD's adapter on MASK rows after the base
 *      projection (verify rows untouched).
 *   6. idlm_isd_kv_append / idlm_isd_kv_rollback: the cache writes around a
 *      step (new rows in before attention, back to the accepted prefix
 *      after acceptance).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked [device] are caller-owned device memory; [host] are
 *   caller-owned host memory, read during the call only.  The library
 *   allocates nothing; per-call scratch lives in the caller's workspace.
 * - Everything is enqueued on `stream` (a hipStream_t passed as void*;
 *   NULL = the default stream) and returns without synchronising, except
 *   idlm_isd_read_status.  idlm_isd_step also uses one stream of the
 *   library's own per device (default priority, non-blocking, made by
 *   idlm_isd_workspace_init or the first step), forked from `stream` and
 *   joined back to it with events before the call returns, so work enqueued
 *   on `stream` afterwards sees the whole step.  The enqueued work is kernel
 *   launches only, plus that fork's event records and waits (no memset or
 *   copy nodes, no host synchronisation, no allocation), so every entry
 *   point but idlm_isd_read_status can be captured into a HIP graph and
 *   replayed; scalar arguments (seed, T) are fixed at capture.
 * - A nonzero return is an idlm_status; nothing was enqueued when a call
 *   fails host-side validation.  Host validation needs no GPU.
 * - Bad *device data* (a page id outside [0, num_pages), a context length
 *   outside [2N-1, 16*max_pages], a draft id outside [-1, V)) cannot be seen
 *   on the host: kernels clamp the value, set a sticky status word in the
 *   workspace and leave that sequence's outputs unspecified.  Read it with
 *   idlm_isd_read_status.
 * - Calls on one workspace must not overlap (they share its partial
 *   softmax states, row statistics and sampling plans); use one workspace
 *   per concurrent stream.  The kernels use no atomic counters: launch
 *   boundaries order every hand-over, so results do not depend on
 *   scheduling.
 * - Workspace: the first idlm_isd_workspace_state_bytes(d) bytes are state
 *   kept between calls (the sticky status word); idlm_isd_workspace_init
 *   zeroes them.  The rest is scratch that every call writes before it
 *   reads, so its contents between calls do not matter.
 *
 * Symbols: B batch, N stride, R = 2N-1 query rows, K = N-1 drafts, Hq / Hkv
 * query / KV heads, G = Hq/Hkv, D head dim, V vocabulary, P pool pages.
 *
 * Paged KV layout
 * ---------------
 * kv_pages is [P][2][Hkv][16*D] elements of qkv_dtype: for every physical
 * page a K block ([.][0][h]) and a V block ([.][1][h]) per KV head, each
 * holding 16 token slots.
 *   K block: 16-byte column chunks.  With x = 16 / sizeof(element) (8 for
 *            bf16, 4 for f32), (slot s, dim d) is at ((d/x)*16 + s)*x + d%x.
 *   V block: transposed, (slot s, dim d) is at d*16 + s.
 * Logical token t of sequence b is slot t%16 of page page_table[b][t/16].
 * ctx_lens[b] counts the R new rows, whose K/V the caller has already
 * written; step row r sits at position ctx_lens[b]-R+r and attends to tokens
 * 0..ctx_lens[b]-R+r.  Scores are q.k/sqrt(D); query head h reads KV head
 * h/G; q and k arrive with rotary embedding applied.
 */
#ifndef IDLM_ISD_H
#define IDLM_ISD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { IDLM_BF16 = 0, IDLM_F32 = 1 } idlm_dtype;

typedef enum {
  IDLM_OK = 0,
  IDLM_ERR_NULL = 1,        /* a required pointer is NULL */
  IDLM_ERR_DIMS = 2,        /* a size is out of range or inconsistent */
  IDLM_ERR_UNSUPPORTED = 3, /* valid but not built: D, dtype or tile shape */
  IDLM_ERR_TEMPERATURE = 4, /* T < 0 or not finite */
  IDLM_ERR_WORKSPACE = 5,   /* workspace too small or misaligned */
  IDLM_ERR_HIP = 6,         /* a HIP runtime call failed */
  IDLM_ERR_DEVICE_DATA = 7, /* kernels saw bad device data (read_status) */
  IDLM_ERR_SCRATCH = 8      /* sizes exceed idlm_isd_accept_noalloc's scratch */
} idlm_status;

/* Sizes of one step.  Passed by [host] pointer. */
typedef struct {
  int32_t B;            /* sequences, >= 0 (0 is a no-op)                    */
  int32_t N;            /* stride, 1..16; R = 2N-1 rows, K = N-1 drafts      */
  int32_t Hq, Hkv;      /* query / KV heads; Hq % Hkv == 0; R*Hq/Hkv <= 128  */
  int32_t D;            /* head dim: 64 or 128                               */
  int32_t V;            /* vocabulary, >= 1                                  */
  int32_t page_size;    /* tokens per page: must be 16                       */
  int32_t max_pages;    /* row stride of page_table, >= 1                    */
  int32_t num_pages;    /* pages in the pool (device range check), >= 1     */
  int32_t qkv_dtype;    /* idlm_dtype of q, kv_pages and attn_out            */
  int32_t logits_dtype; /* idlm_dtype of logits_clean and logits_mask        */
} idlm_isd_dims;

/* Bytes of workspace every entry point below needs for these sizes; 0 for
 * invalid sizes.  Host only. */
size_t idlm_isd_workspace_bytes(const idlm_isd_dims* d);

/* Leading bytes of that workspace holding state kept between calls (see
 * the conventions above); 0 for invalid sizes.  Host only. */
size_t idlm_isd_workspace_state_bytes(const idlm_isd_dims* d);

/* Check sizes and temperature without touching the GPU.  Returns IDLM_OK,
 * IDLM_ERR_NULL, IDLM_ERR_DIMS, IDLM_ERR_UNSUPPORTED (also for sizes whose
 * grids would not fit one dispatch: more than 2^32 - 1 work-items) or
 * IDLM_ERR_TEMPERATURE (T < 0, not finite, or 0 < T < 2^-126).  Host only. */
int32_t idlm_isd_validate(const idlm_isd_dims* d, float T);

/* Prepare a workspace for first use: zeroes it (the sticky status word
 * included) with a fill kernel on `stream`, never a memset node.  Must run
 * once after allocating the workspace, and again to clear a reported device
 * data error; the step kernels need nothing else zeroed between calls. */
int32_t idlm_isd_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* Causal paged GQA attention of the R step rows (see the header comment).
 *   q          [device] [B][R][Hq][D] qkv_dtype
 *   kv_pages   [device] [P][2][Hkv][16*D] qkv_dtype, layout above
 *   page_table [device] int32 [B][max_pages]
 *   ctx_lens   [device] int32 [B]
 *   attn_out   [device] [B][R][Hq][D] qkv_dtype, written
 * bf16 runs bf16 MFMA with float32 accumulation and softmax; f32 runs float32
 * FMA.  Output rows are the softmax-weighted sums rounded once to
 * qkv_dtype. */
int32_t idlm_isd_paged_attn(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                            const int32_t* page_table, const int32_t* ctx_lens, void* attn_out,
                            void* workspace, size_t ws_bytes, void* stream);

/* Bytes of a MASK-row statistics record for these sizes (0 for invalid
 * sizes).  idlm_isd_propose fills one (its mask_stats argument) with the
 * statistics of the MASK rows it proposes from and the drafts it makes; the
 * next step's idlm_isd_accept (or idlm_isd_step) on those drafts takes it
 * as its mask_stats and then reduces only the N clean rows: in a decode
 * loop, MASK rows propose with q ("Introspective Diffusion Language
 * Models", section "Inference & ISD") and that same q tests the drafts one
 * step later.  Caller-owned device memory, 256-byte aligned.  Host only. */
size_t idlm_isd_mask_stats_bytes(const idlm_isd_dims* d);

/* Acceptance stage.
 *   logits_clean   [device] [B][N][V] logits_dtype.  Clean row i (i < K)
 *                  gives p_i, which verifies draft i; row K gives the bonus
 *                  distribution used when every draft is kept.
 *   logits_mask    [device] [B][K][V] logits_dtype.  MASK row i gives q_i,
 *                  the distribution draft i was proposed from.  May be NULL
 *                  when N == 1.
 *   draft_tokens   [device] int32 [B][K]; a -1 ends sequence b's list early
 *                  (k < K drafts; the bonus then comes from clean row k).
 *                  May be NULL when N == 1.
 *   seed           Philox4x64-10 key word 0; key word 1 is b; counter
 *                  (i,0,0,0) gives u_i (word 0, ratio test) and u'_i (word 1,
 *                  sampling) as (word >> 40) * 2^-24.
 *   T              temperature: 0 (greedy: one-hot argmax, lowest index on
 *                  ties) or 2^-126 <= T < inf; p = softmax(clean/T),
 *                  q = softmax(mask/T).
 *   out_tokens     [device] int32 [B][N]: kept drafts, then the resampled or
 *                  bonus token, then -1 padding.
 *   out_accept_len [device] int32 [B]: tokens committed, in 1..N.
 *   out_debug      [device] double [B][N+1][4] or NULL.  Row i < N holds
 *                  (p_i(x_i), q_i(x_i), u_i, u'_i) for every draft tested
 *                  (NaN elsewhere); row N holds (sum of sampling weights,
 *                  threshold t, u' used, committed token).
 *   mask_stats     [device] or NULL: the record idlm_isd_propose wrote when
 *                  it made draft_tokens from logits_mask at this T.  The MASK
 *                  rows' maxima and sums and the drafts' logits then come
 *                  from it, and logits_mask is read only for a rejected
 *                  draft's residual.  The record's sums are float64
 *                  weights at the float64 scale log2(e)/T; the
 *                  acceptance's own reduction sums float32 exponentials
 *                  at that scale rounded to float32, so q from either
 *                  agrees to about 1e-7 relative.
 * Draft i is kept iff p_i(x) > 0 and (p_i(x) >= q_i(x) or u_i*q_i(x) <
 * p_i(x)), in float64.  At the first rejected index j the token is the
 * smallest v whose running sum of w = max(0, p_j - q_j) exceeds
 * t = u'_j * sum(w) (sum(w) == 0 falls back to w = p_j); with no rejection
 * w = p_k (bonus row).  The sampling weights, their sums and the row sums
 * they are normalised by are float64 (exponentials included).
 * Device-data errors: a draft id outside [-1, V); a mask_stats record made
 * for other drafts, another T or other sizes (that sequence's outputs are
 * unspecified). */
int32_t idlm_isd_accept(const idlm_isd_dims* d, const void* logits_clean, const void* logits_mask,
                        const int32_t* draft_tokens, uint64_t seed, float T, int32_t* out_tokens,
                        int32_t* out_accept_len, double* out_debug, const void* mask_stats,
                        void* workspace, size_t ws_bytes, void* stream);

/* Debug dump of what the last idlm_isd_accept or idlm_isd_step on
 * `workspace` computed, with the same sizes, logits and T passed again:
 *   out_p    [device] double [B][N][V] or NULL: p over the whole vocabulary
 *            for each clean row, exp((l - M)/T)/S from that call's row
 *            maximum M and sum S (greedy: one-hot at the argmax), the same
 *            expression the acceptance evaluates at the drafts.  Rows the
 *            call did not reduce hold NaN: clean rows past the listed
 *            drafts, and the bonus row (clean row k) unless it was sampled.
 *   out_q    [device] double [B][K][V] or NULL: q likewise for MASK rows.
 *   out_subw [device] double [B][ceil(V/2048)] or NULL: the sampled
 *            distribution (residual, bonus, or p_j when the residual
 *            vanished) summed over each 2048-entry sub-chunk and normalised
 *            to total 1; NaN when greedy.
 * Reads the workspace only; enqueued on `stream`. */
int32_t idlm_isd_accept_probs(const idlm_isd_dims* d, const void* logits_clean,
                              const void* logits_mask, float T, const void* workspace,
                              size_t ws_bytes, double* out_p, double* out_q, double* out_subw,
                              void* stream);

/* idlm_isd_accept without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * idlm_isd_accept (bit-identical outputs for the same inputs), except:
 *   out_status  [device] int32 or NULL: cleared, then set nonzero when the
 *               kernels see bad device data (a draft id outside [-1, V)).
 * Scratch: a static device array of IDLM_ISD_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's load on that device until the process ends; the
 * call allocates and frees nothing (no hipMalloc, no allocating library
 * routine).  The acceptance's buffers take 256 bytes plus seven regions,
 * each rounded up to a multiple of 256 bytes: B*64, B*R*16*ceil(V/8192),
 * B*32*ceil(V/2048), B*R*4, B*256, B*R*32 and B*8*ceil(V/2048) (R = 2N-1;
 * B = 64, N = 4, V = 151936: 0.37 MB; up to B = 1471 at that N and V).
 * Larger sizes are rejected with IDLM_ERR_SCRATCH before anything is
 * enqueued.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call clears the one word it needs cleared): calls that
 * overlap on one GPU (different streams, or host threads without ordering
 * between them) race and must not be issued.  idlm_isd_accept_probs does
 * not read this scratch. */
#define IDLM_ISD_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int32_t idlm_isd_accept_noalloc(const idlm_isd_dims* d, const void* logits_clean,
                                const void* logits_mask, const int32_t* draft_tokens,
                                uint64_t seed, float T, int32_t* out_tokens,
                                int32_t* out_accept_len, double* out_debug,
                                const void* mask_stats, int32_t* out_status, void* stream);

/* One ISD step: idlm_isd_paged_attn and idlm_isd_accept, which read
 * different inputs, run side by side: the attention on `stream`, the
 * acceptance on the library's second stream of this device (forked from
 * `stream` with an event and joined back to it).  The results equal the
 * two calls in sequence.  Small steps (B*R*V < 2^23 logits, where the
 * event hand-over costs more than the overlap saves), or a device where the
 * second stream cannot be created, run the two in sequence on `stream`.
 * Steps from several host threads on one device share that stream (their
 * enqueues are serialised); while one thread captures a step into a graph,
 * no other thread may run a step on the same device.  N must equal d->N (it
 * is repeated to keep the step's own argument list); mask_stats as for
 * idlm_isd_accept. */
int32_t idlm_isd_step(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                      const int32_t* page_table, const int32_t* ctx_lens,
                      const void* logits_clean, const void* logits_mask,
                      const int32_t* draft_tokens, uint64_t seed, int32_t N, float T,
                      int32_t* out_tokens, int32_t* out_accept_len, void* attn_out,
                      const void* mask_stats, void* workspace, size_t ws_bytes, void* stream);

/* One step of the decode loop: idlm_isd_step, then, on the acceptance's
 * stream (beside the attention when the step forks), idlm_isd_propose of the
 * next step's drafts from this forward's MASK rows:
 *   logits_mask, draft_tokens, mask_stats   as for idlm_isd_step (the
 *                  previous forward's MASK rows, the drafts made from them,
 *                  and their record or NULL)
 *   logits_next    [device] [B][K][V]: this forward's MASK rows
 *   next_drafts    [device] int32 [B][K], written (as idlm_isd_propose)
 *   mask_stats_next [device] or NULL, written: the record of next_drafts;
 *                  may be the mask_stats buffer itself (the proposals run
 *                  after the acceptance has read it)
 * The proposals use the step's seed (their counters, (i, 1, 0, 0), are
 * apart from the acceptance's) and T.  Results equal idlm_isd_step followed
 * by idlm_isd_propose(d, logits_next, draft_tokens, out_accept_len, seed, T,
 * next_drafts, mask_stats_next, ...). */
int32_t idlm_isd_loop_step(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                           const int32_t* page_table, const int32_t* ctx_lens,
                           const void* logits_clean, const void* logits_mask,
                           const int32_t* draft_tokens, const void* mask_stats,
                           const void* logits_next, uint64_t seed, int32_t N, float T,
                           int32_t* out_tokens, int32_t* out_accept_len, void* attn_out,
                           int32_t* next_drafts, void* mask_stats_next, void* workspace,
                           size_t ws_bytes, void* stream);

/* Drafts for the next step.  MASK rows propose the next tokens from q
 * ("Introspective Diffusion Language Models", section "Inference & ISD").
 * A sequence whose listed drafts were all kept (accept_len == k + 1, k the
 * drafts before the first -1; k = 0 is a fresh step) keeps verifying: draft
 * i of its next step is drawn from softmax(logits_next[b][i] / T) by inverse
 * CDF (ascending vocabulary, smallest v whose running sum exceeds u * sum)
 * with u = word 0 of the Philox4x64-10 block at counter (i, 1, 0, 0) under
 * key (seed, b), or the argmax (lowest index) when T == 0; the weights are
 * float64 (exponentials included), as are the running sums.  Otherwise the
 * next step is fresh and all its drafts are -1.  No-op when N == 1.
 *   logits_next  [device] [B][K][V] logits_dtype: this forward's MASK rows
 *   draft_tokens [device] int32 [B][K]: this step's list
 *   accept_len   [device] int32 [B]: idlm_isd_accept's output
 *   next_drafts  [device] int32 [B][K], written
 *   mask_stats   [device] or NULL, written: the MASK rows' statistics and
 *                the drafts, for the next step's idlm_isd_accept (see
 *                idlm_isd_mask_stats_bytes)
 * Rows of sequences that start a fresh step are not read. */
int32_t idlm_isd_propose(const idlm_isd_dims* d, const void* logits_next,
                         const int32_t* draft_tokens, const int32_t* accept_len, uint64_t seed,
                         float T, int32_t* next_drafts, void* mask_stats, void* workspace,
                         size_t ws_bytes, void* stream);

/* Sizes of a gated-LoRA call.  Passed by [host] pointer. */
typedef struct {
  int32_t B, N;   /* rows: B blocks of R = 2N-1; row r of a block is a MASK row iff r >= N */
  int32_t H;      /* input features, multiple of 32                        */
  int32_t O;      /* output features, >= 1                                 */
  int32_t rank;   /* adapter rank, multiple of 16, <= 256                  */
} idlm_isd_lora_dims;

/* Workspace bytes idlm_isd_gated_lora needs (0 for invalid sizes).  Host only. */
size_t idlm_isd_lora_workspace_bytes(const idlm_isd_lora_dims* L);

/* R-ISD's gated LoRA, applied after the base projection: the adapter is
 * active only at MASK rows and verify rows keep the base weights alone, which
 * makes the output bit-for-bit the base model's ("Introspective Diffusion
 * Language Models", section "Lossless R-ISD").
 *   y_base [device] float32 [M][O], M = B*(2N-1): the base projection's
 *          accumulator, before rounding
 *   x      [device] bf16 [M][H] (16-byte aligned): the projection's input rows
 *   lora_a [device] bf16 [rank][H], lora_b [device] bf16 [O][rank] (aligned)
 *   y_out  [device] bf16 [M][O], written
 * Verify rows: y_out = bf16(y_base), nothing else (bit-identical to the
 * base-only output).  MASK rows: y_out = bf16(y_base + scale * (x A^T) B^T),
 * the adapter products accumulated in float32, rounded once to nearest even.
 * Workspace: idlm_isd_lora_workspace_bytes, 256-byte aligned, no init
 * needed (split partials of x A^T and their sum).  All buffers are the
 * caller's; y_out must not overlap y_base, x or the workspace.  Kernels are
 * enqueued on `stream`; nothing is synchronised.
 * Errors (nothing enqueued): IDLM_ERR_NULL for a null pointer,
 * IDLM_ERR_DIMS for sizes out of range or a non-finite scale,
 * IDLM_ERR_UNSUPPORTED for H not a multiple of 32, rank not a multiple of
 * 16 or above 256, or x / lora_a / lora_b not 16-byte aligned,
 * IDLM_ERR_WORKSPACE for a short or misaligned workspace.  B = 0 is a no-op. */
int32_t idlm_isd_gated_lora(const idlm_isd_lora_dims* L, const float* y_base, const void* x,
                            const void* lora_a, const void* lora_b, float scale, void* y_out,
                            void* workspace, size_t ws_bytes, void* stream);

/* KV append, before attention.  Writes the R step rows' keys and values into
 * the paged cache at positions ctx_before[b] .. ctx_before[b]+R-1 (the cache
 * is paged and serves continuous batching: "Introspective Diffusion Language
 * Models", section "Serving (SGLang)").
 *   k_new, v_new [device] [B][R][Hkv][D] qkv_dtype (keys rotated already)
 *   ctx_before   [device] int32 [B]: tokens already cached
 *   ctx_after    [device] int32 [B], written: ctx_before + R (the ctx_lens
 *                of idlm_isd_paged_attn); may be the same array as ctx_before
 *   kv_pages     [device] pool, layout above; rows written in place
 *   page_table   [device] int32 [B][max_pages]; entries of new pages written
 *   free_pages   [device] int32 [num_pages]: a stack of free page ids, the
 *                first *free_count entries valid
 *   free_count   [device] int32 scalar, updated
 * The call takes T pages in total, the top T stack entries, sequence by
 * sequence in batch order and each sequence's pages in page order (no
 * atomics: the same inputs give the same assignment).  Device-data errors
 * (read_status): a ctx_before outside [0, 16*max_pages - R] (that sequence is
 * left unchanged), too few free pages or a free-list id outside
 * [0, num_pages) (the whole call is left unchanged). */
int32_t idlm_isd_kv_append(const idlm_isd_dims* d, const void* k_new, const void* v_new,
                           const int32_t* ctx_before, int32_t* ctx_after, void* kv_pages,
                           int32_t* page_table, int32_t* free_pages, int32_t* free_count,
                           void* workspace, size_t ws_bytes, void* stream);

/* KV rollback, after acceptance.  Only the anchor and the accepted drafts
 * stay context (the first rejection ends the kept prefix: "Introspective
 * Diffusion Language Models", section "Inference & ISD"), so sequence b keeps
 * ctx_lens[b] - R + accept_len[b] tokens; page-table entries past that are
 * set to -1 and their pages pushed on the free stack in batch order, page
 * order.  Freed pages keep their stale contents.
 *   ctx_lens   [device] int32 [B]: the step's context (R rows included)
 *   accept_len [device] int32 [B]: idlm_isd_accept's output, in [1, R]
 *              (clamped otherwise and reported)
 *   ctx_after  [device] int32 [B], written; may be the same array as ctx_lens
 *   page_table, free_pages, free_count as for idlm_isd_kv_append
 * Device-data errors: a ctx_lens outside [R, 16*max_pages] (sequence left
 * unchanged), a stack overflow past num_pages (call left unchanged). */
int32_t idlm_isd_kv_rollback(const idlm_isd_dims* d, const int32_t* ctx_lens,
                             const int32_t* accept_len, int32_t* ctx_after, int32_t* page_table,
                             int32_t* free_pages, int32_t* free_count, void* workspace,
                             size_t ws_bytes, void* stream);

/* Synchronise `stream`, then copy the workspace's sticky device status into
 * *host_code (IDLM_OK or IDLM_ERR_DEVICE_DATA).  Cleared only by
 * idlm_isd_workspace_init. */
int32_t idlm_isd_read_status(const void* workspace, void* stream, int32_t* host_code);

/* Static description of a status code. */
const char* idlm_isd_strerror(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* IDLM_ISD_H */
