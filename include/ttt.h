/*
 * ttt.h - C ABI of the TTT-E2E prefill library (libttt.so, gfx950 / MI355X).
 *
 * What the library computes is the causal prefill with inner adaptation of
 * "End-to-End Test-Time Training for Long Context" as described in the
 * zhongzhuzhou.org reading notes (section 7, Algorithm 1; section 5, Eq. 9;
 * section 3, Eq. 3): a context is read in chunks of b positions through a
 * pre-norm Transformer with causal sliding-window attention (window k) and
 * QK-norm.  Each chunk's per-token next-token losses are recorded with the
 * current fast weights W; then the mean loss of the chunk is differentiated
 * with respect to W only - the fast SwiGLU MLPs of the last n_update blocks,
 * each summed with a frozen static SwiGLU on the same pre-MLP norm (notes,
 * section 6) - and one SGD step W <- W - eta * grad is taken before the next
 * chunk.  Keys and values of earlier chunks are kept in a bounded ring of the
 * window and are constants of each step.  Every prefill starts from W_init
 * (notes, section 7: state of independent documents is never shared).
 *
 * All compute runs in the library's own HIP kernels on the given stream.
 *
 * Conventions for every entry point:
 *   - Device pointers point to GPU memory of the current HIP device; host
 *     pointers are marked "host".
 *   - Row-major layouts.  "[R,C]" means R rows of C contiguous elements.
 *   - Element types: tensors marked "wt" are float32 when cfg.dtype ==
 *     TTT_FP32 and bfloat16 (raw 16-bit storage) when cfg.dtype == TTT_BF16.
 *   - The caller owns every buffer it passes; the library never frees them.
 *   - Return value: TTT_OK or a negative ttt_status.  On TTT_EINVAL nothing
 *     was enqueued.  ttt_last_error() gives a text for the last failure.
 *   - A handle is not thread-safe; use one handle per stream.
 */
#ifndef TTT_H
#define TTT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTT_OK = 0,
  TTT_EINVAL = -1,        /* bad argument: sizes, null pointers, unsupported combination */
  TTT_ENOMEM = -2,        /* device allocation failed */
  TTT_EHIP = -3,          /* a HIP runtime call failed (text in ttt_last_error) */
  TTT_EUNSUPPORTED = -4,  /* shape not supported by the compiled kernels (e.g. head_dim) */
  TTT_ENONFINITE = -5     /* a recorded loss or an updated fast weight was NaN or infinite
                             (checked after the prefill, see ttt_check_finite) */
} ttt_status;

typedef enum { TTT_FP32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* Flags for ttt_prefill (and defaults in ttt_config.flags). */
enum {
  TTT_NO_UPDATE = 1u << 0,  /* forward-only sliding-window prefill: no backward, no SGD.
                               Losses equal those of eta = 0. */
  TTT_NO_GRAPH = 1u << 1    /* launch kernels one by one instead of replaying the
                               captured per-chunk HIP graph (same results, bit for bit) */
};

/*
 * Model and run shape.  Constraints checked by ttt_create (TTT_EINVAL otherwise):
 *   n_layers >= 1; 0 <= n_update <= n_layers; d_model == n_heads * head_dim;
 *   d_model, d_ff, vocab multiples of 16; head_dim in {16, 32, 64, 80, 96, 128};
 *   chunk and window multiples of 64 with window >= chunk (the notes, section 5:
 *   the window covers at least one chunk); max_tokens >= 1.
 * Shapes outside the compiled kernels give TTT_EUNSUPPORTED: head_dim not in the
 * set above, head_dim > 64 with fp32, d_model > 8192, and in bf16 mode d_model
 * or d_ff not a multiple of 64, or an updated block's fast or static MLP weight
 * that is not finite or not below 8192 in magnitude (their fp16 forward copies
 * are stored scaled by a power of two chosen from the largest magnitude).
 */
typedef struct {
  int32_t n_layers;     /* L */
  int32_t d_model;      /* d */
  int32_t n_heads;      /* H */
  int32_t head_dim;     /* hd */
  int32_t d_ff;         /* F: hidden size of each SwiGLU (fast and static alike) */
  int32_t vocab;        /* V */
  int32_t window;       /* k: query p attends keys j with p-k < j <= p */
  int32_t chunk;        /* b: positions per inner update */
  int32_t n_update;     /* n_u: blocks L-n_u .. L-1 carry fast MLPs */
  float eta;            /* inner SGD step size */
  float rms_eps;        /* epsilon inside every RMSNorm (block, final, QK-norm) */
  float rope_theta;     /* rotary base; angle_i = p * theta^(-2i/hd), pairs (i, i+hd/2) */
  int32_t dtype;        /* ttt_dtype of weights and activations */
  int64_t max_tokens;   /* largest T accepted by ttt_prefill; sizes the rotary table */
  uint32_t flags;       /* default flags OR-ed into every ttt_prefill call */
  int32_t n_seq;        /* B: independent sequences per ttt_prefill (0 or 1: one; at most 256).
                           Each has its own fast weights and window; they share the frozen
                           weights, and every frozen-weight product runs once over all B chunks */
} ttt_config;

/*
 * Weights.  The pointer ARRAYS are host memory (one entry per layer, or per
 * updated block); every tensor they point to is device memory, read only
 * during ttt_create (the library copies and repacks everything it needs).
 * Linear maps follow y = x W^T with W stored [out, in].
 */
typedef struct {
  const void *tok_emb;             /* wt [V, d] */
  const void *lm_head;             /* wt [V, d] (untied output head) */
  const void *final_norm;          /* wt [d] */
  const void *const *attn_norm;    /* host array of L; each wt [d] */
  const void *const *wq;           /* host array of L; each wt [d, d] (heads contiguous in rows) */
  const void *const *wk;           /* host array of L; each wt [d, d] */
  const void *const *wv;           /* host array of L; each wt [d, d] */
  const void *const *wo;           /* host array of L; each wt [d, d] */
  const void *const *q_norm;       /* host array of L; each wt [hd] (shared by heads) */
  const void *const *k_norm;       /* host array of L; each wt [hd] */
  const void *const *mlp_norm;     /* host array of L; each wt [d] */
  const void *const *w_gate;       /* host array of L; each wt [F, d]  (static SwiGLU) */
  const void *const *w_up;         /* host array of L; each wt [F, d] */
  const void *const *w_down;       /* host array of L; each wt [d, F] */
  const float *const *fast_gate;   /* host array of n_u; each float32 [F, d]: W_init of block L-n_u+u */
  const float *const *fast_up;     /* host array of n_u; each float32 [F, d] */
  const float *const *fast_down;   /* host array of n_u; each float32 [d, F] */
} ttt_weights;

typedef struct ttt_handle ttt_handle;

/*
 * Creates a handle on the current HIP device: validates cfg, allocates the
 * bounded state (per-layer key/value rings of k+b rows, or k+G rows for the
 * blocks below the updated ones, which run ahead over groups of G tokens;
 * activations of one chunk and of two groups, the current one and the next,
 * whose frozen-block pass runs beside the current one's chunks; the exponentiated logits of
 * one vocabulary slab when n_update > 0 - no [b, V] logits are kept; fp32
 * master fast weights) and copies/repacks the weights.  It reads the head and
 * final-norm weights once to decide how the head runs: one pass over the
 * vocabulary for losses and gradient when the weights bound how far any
 * logit can lie from its row's label logit, 2.02 sqrt(d) max|final_norm|
 * max_v |lm_head row v|, by 126 - ln V; else a cross-entropy pass first and
 * a second pass for the gradient (same results up to rounding).
 * G is 8192 to 16384 rows over all sequences (the count for which a model of the
 * frozen pass over max_tokens tokens, in whole rounds of GEMM tiles and attention
 * work-groups, is fastest), at most max_tokens rounded up to a chunk, and 0 (no
 * group pass) when that is not more than one chunk.
 * `stream` is a hipStream_t (NULL = default stream); the call synchronises it
 * before returning.  *out receives the handle (NULL on failure).
 */
ttt_status ttt_create(const ttt_config *cfg, const ttt_weights *w, void *stream, ttt_handle **out);

/*
 * Algorithm 1 of the notes on each of the handle's B = n_seq sequences (each
 * starts from W_init with its own fast weights and window; they advance chunk
 * by chunk together, all of length T).
 *   d_tokens   device int32 [B][T+1]: ids x_0..x_T of each sequence, each in [0, V).
 *   T          number of scored positions, 0 <= T <= cfg.max_tokens.  The last
 *              chunk may be short (T % b != 0); its update averages over its own size.
 *   d_losses   device float32 [B][T] out: d_losses[s][p] = -ln p(x_{p+1} | x_0..x_p)
 *              of sequence s under its fast weights current at p's chunk,
 *              recorded before that chunk's update.
 *   d_fast_out host array of 3*n_u*B device float32 pointers, or NULL.  If given,
 *              receives each sequence's W_N after all ceil(T/b) updates, in the
 *              order gate[F,d], up[F,d], down[d,F] for block L-n_u, then
 *              L-n_u+1, ..., sequence 0 first.
 *   flags      TTT_NO_UPDATE / TTT_NO_GRAPH, OR-ed with cfg.flags.
 *   stream     hipStream_t to enqueue on (NULL = default stream).  With graph
 *              replay the frozen blocks' pass over the next group of G tokens runs
 *              on a stream the handle owns, ordered against `stream` by events;
 *              all of the call's work is complete when `stream` reaches its end.
 * Starts from W_init and an empty ring every call.  Returns after enqueueing
 * (no host synchronisation) unless the non-finite check is requested with
 * ttt_check_finite().  Token ids are not range-checked on the device; ids
 * outside [0, V) are undefined behaviour.
 */
ttt_status ttt_prefill(ttt_handle *h, const int32_t *d_tokens, int64_t T, float *d_losses,
                       float *const *d_fast_out, uint32_t flags, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): ttt_prefill with the
 * same arguments, results and errors, except that
 *   - the partial results of split-K products and of key-range-split attention
 *     go to a static device array of the library (160 MiB per device, held from
 *     the library's load until the process ends: 96 MiB for the product
 *     partials, 64 MiB for the attention partials) instead of the handle's
 *     workspaces; TTT_EUNSUPPORTED, with nothing enqueued, when the handle's
 *     shapes need more (the 2.7B workload needs 80 and 41 MiB);
 *   - every kernel is launched one by one on `stream` (no HIP graph is captured
 *     or instantiated) and no event is recorded, so the call allocates nothing
 *     and ttt_get_stats reports no duration for it (0 ms);
 *   - TTT_EINVAL when kernel timing is on or the current device is not the
 *     handle's.
 * The handle's own state (created by ttt_create) is used as by ttt_prefill.
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (on different streams, or from several threads) race and
 * give undefined results.  The HIP runtime may load the kernels' code on their
 * first launch; a caller that must not see that does one ttt_prefill first.
 */
ttt_status ttt_prefill_noalloc(ttt_handle *h, const int32_t *d_tokens, int64_t T, float *d_losses,
                               float *const *d_fast_out, uint32_t flags, void *stream);

/*
 * Algorithm 3 of the notes (generation with periodic updates), continuing the
 * sequence that the last ttt_prefill (given tokens), or ttt_decode, on this
 * handle left: its fast weights, its window of keys/values and its length P
 * (positions 0..P-1 processed; the id at position P, the prefill's last label,
 * is known).
 *   n_steps       positions fed, P + n_steps <= cfg.max_tokens.
 *   d_forced      device int32 [n_steps] or NULL.  NULL: each next id is the
 *                 argmax of the current prediction (greedy; lowest id among equal
 *                 logits).  Otherwise id j is taken as the next token whatever the
 *                 prediction (teacher forcing, for evaluation and tests).
 *   d_tokens_out  device int32 [n_steps] out: the ids at positions P+1..P+n_steps.
 *   d_losses_out  device float32 [n_steps] out: -ln p(next id | prefix) at each
 *                 fed position, under the fast weights current at that position.
 *   d_fast_out    as for ttt_prefill: the fast weights after the call, or NULL.
 * Decode chunks are [P, P+b), [P+b, P+2b), ... counted from the length the
 * prefill left.  Once every target of the open chunk is known (after the step
 * that produces id s+b), the chunk's forward is run again and its mean loss
 * back-propagated into the fast weights with one SGD step, exactly as a
 * prefill chunk (no update with TTT_NO_UPDATE or n_update = 0); the next
 * position then uses the new weights.  A partial chunk is kept open for the
 * next call.  Returns after enqueueing; ttt_check_finite covers these losses
 * too.  TTT_EINVAL when no prefill with tokens preceded it or the length
 * would pass max_tokens; TTT_EUNSUPPORTED for a handle of more than one sequence.
 */
ttt_status ttt_decode(ttt_handle *h, int64_t n_steps, const int32_t *d_forced, int32_t *d_tokens_out,
                      float *d_losses_out, float *const *d_fast_out, uint32_t flags, void *stream);

/* Synchronises `stream` and returns TTT_ENONFINITE if, in the last prefill or
 * decode on this handle, any recorded loss was NaN or infinite or any fast
 * weight after its inner updates was (Algorithm 1 steps 3.3-3.5: the fp32
 * master copies hold W_0 - eta * the sum of every step's gradient, so a
 * non-finite gradient of any chunk leaves a non-finite weight behind; they are
 * checked after the last update), TTT_OK otherwise.  The kernels finish
 * normally either way; only the status reports the condition. */
ttt_status ttt_check_finite(ttt_handle *h, void *stream);

/* Host values of the last prefill: its duration in ms between events recorded on
 * its stream at the start and at the end of ttt_prefill's work (waits for the
 * end event; 0 before any prefill), the number of chunks and the kernel launches
 * of one chunk step.  Each out pointer may be NULL. */
ttt_status ttt_get_stats(ttt_handle *h, double *ms_last, int64_t *chunks_last, int64_t *launches_per_chunk);

/*
 * Kernel timing (diagnostics).  While enabled, ttt_prefill launches kernel by
 * kernel (no graph replay), brackets every kernel group of a class with HIP
 * events on the prefill's stream and synchronises after each chunk to add the
 * elapsed times to per-class totals.  Enabling or disabling clears the totals.
 * Results are bit-identical to a run without timing.
 */
ttt_status ttt_set_kernel_timing(ttt_handle *h, int enable);

/* Number of kernel classes (embed, rmsnorm, gemm_qkv, attn_fwd, ...). */
int ttt_kernel_class_count(void);

/* Name, summed duration (ms) and launch count of class `cls` since timing was
 * enabled.  *name points to a static string. */
ttt_status ttt_get_kernel_time(const ttt_handle *h, int cls, const char **name, double *total_ms, int64_t *count);

/* Text of the last error on this handle (or of the calling thread if h is NULL). */
const char *ttt_last_error(const ttt_handle *h);

/* Frees everything the handle owns.  Synchronises the device first. NULL is a no-op. */
void ttt_destroy(ttt_handle *h);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H */
