/*
 * qwen2.h - C ABI of the MI355X (gfx950) Qwen2 / Qwen2.5 decoder forward pass.
 *
 * One library, libqwen2_mi355x.so, computes the decoder forward pass of the
 * Qwen2 family on one AMD Instinct MI355X:
 *
 *   embedding -> per layer [RMSNorm -> fused WQ/WK/WV + bias -> RoPE(q, k)
 *   (NonInterleaved / rotate_half) -> KV store -> causal GQA attention ->
 *   WO + residual -> RMSNorm -> fused gate/up + SwiGLU -> down + residual]
 *   -> final RMSNorm -> lm_head (tied or untied) -> argmax on the device.
 *
 * The layer dataflow is the one on the minfer page "Qwen2 / Qwen2.5
 * Architecture Support", section 1; bias placement, GQA mapping, readout and
 * shapes follow the nnterp encyclopedia page "qwen2" (Notes, Printout,
 * Config); the dtype policy (f16 matmul weights and lm_head, f32 biases,
 * norms and activations) follows xinfer "Module 7", section 7.4.
 *
 * Conventions shared by every call:
 *  - Matrices are IEEE binary16 bit patterns (uint16_t), row-major
 *    [out_features, in_features] like a PyTorch Linear weight.
 *  - Biases, norm weights, activations, logits and the KV cache are float32.
 *  - Token ids, positions, sequence ids and argmax results are int32.
 *  - "host" pointers are ordinary CPU memory read before the call returns;
 *    "device" pointers are HIP device memory owned by the caller.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *    only enqueue work; the caller synchronises the stream before reading
 *    device outputs.
 *  - Calls on one context share its scratch and KV cache: the caller keeps
 *    them ordered (one stream, or synchronised between streams).
 *  - Every call returns QWEN2_OK (0) or a negative QWEN2_E_* code.  All
 *    checks that can be done on the host run before anything is enqueued, so
 *    a rejected call changes neither the KV cache nor any other state.
 *    qwen2_last_error() gives a message for the last failure on a context.
 */
#ifndef QWEN2_MI355X_H
#define QWEN2_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QWEN2_OK = 0,
  QWEN2_E_ARG = -1,     /* null pointer, n <= 0, bad `which`, out-of-range layer */
  QWEN2_E_HPARAMS = -2, /* hyperparameters the library does not support */
  QWEN2_E_POS = -3,     /* position < 0 or >= n_ctx (hard error, never truncated) */
  QWEN2_E_TOKEN = -4,   /* token id outside [0, n_vocab) */
  QWEN2_E_SEQ = -5,     /* sequence slot outside [0, n_seq) or repeated in one batch */
  QWEN2_E_ORDER = -6,   /* positions of one prefill not strictly increasing */
  QWEN2_E_HIP = -7,     /* a HIP runtime call failed (message has the HIP error) */
  QWEN2_E_OOM = -8,     /* device or host allocation failed */
  QWEN2_E_DEBUG = -9,   /* a debug check failed (contexts loaded with QWEN2_DEBUG_CHECKS=1) */
};

/* Model and cache hyperparameters (HParams of the minfer page, section 2;
 * QwenConfig of xinfer Module 7, section 7.1).
 * Supported: n_embd == n_head * head_dim, n_embd % 64 == 0, n_embd <= 8192,
 * n_ctx <= 131072, n_head % n_head_kv == 0 with n_head / n_head_kv <= 8,
 * head_dim in {16, 64, 128}, rope_style 0 (NonInterleaved: dimension d pairs
 * with d + head_dim/2, the Qwen2 convention) or 1 (Interleaved: 2d pairs with
 * 2d + 1), a model-level flag (minfer page, section 3), rope_theta > 0,
 * rope_freq_scale > 0, rms_eps >= 0, every size > 0. */
typedef struct qwen2_hparams {
  int32_t n_layer, n_embd, n_head, n_head_kv, head_dim, n_ff, n_vocab;
  int32_t n_ctx;      /* KV slots per sequence (the --n-ctx of the minfer page,
                         section 6), not the model's training context */
  int32_t n_seq;      /* independent sequence slots in the KV cache */
  int32_t tied;       /* 1: lm_head is the token embedding (xinfer 7.3) */
  int32_t rope_style; /* 0 = NonInterleaved, 1 = Interleaved; else rejected */
  float rope_theta;   /* RoPE base; angle = pos * freq_scale * theta^(-2d/head_dim) */
  float rope_freq_scale;
  float rms_eps;      /* y = w * x / sqrt(mean(x^2) + rms_eps) */
} qwen2_hparams;

/* Host pointers to one layer's weights (LayerWeights of the minfer page,
 * section 2).  Shapes with H = n_embd, I = n_ff, hd = head_dim:
 *   attn_norm, ffn_norm [H] f32;  bq [n_head*hd], bk, bv [n_head_kv*hd] f32;
 *   wq [n_head*hd, H], wk/wv [n_head_kv*hd, H], wo [H, n_head*hd],
 *   w_gate/w_up [I, H], w_down [H, I]   (binary16, row-major [out, in]). */
typedef struct qwen2_layer_weights {
  const float *attn_norm, *bq, *bk, *bv, *ffn_norm;
  const uint16_t *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
} qwen2_layer_weights;

typedef struct qwen2_weights {
  const uint16_t *tok_embd;           /* [n_vocab, H] binary16 */
  const uint16_t *lm_head;            /* [n_vocab, H]; ignored (may be NULL) when tied */
  const float *out_norm;              /* [H] */
  const qwen2_layer_weights *layers;  /* [n_layer] */
} qwen2_weights;

typedef struct qwen2_ctx qwen2_ctx;

typedef struct qwen2_info_t {
  uint64_t weight_bytes_f16;   /* binary16 matrices as the model defines them
                                  (the tied lm_head counted once) */
  uint64_t weight_bytes_f32;   /* biases and norm weights */
  uint64_t weight_bytes_alloc; /* device bytes of the weight store incl. padding */
  uint64_t kv_bytes_per_pos;   /* K+V bytes of one position over all layers */
  uint64_t kv_bytes;           /* whole KV cache: n_seq * n_ctx * kv_bytes_per_pos */
  uint64_t scratch_bytes;      /* activations and attention partials */
  int32_t n_ctx, n_seq, max_rows; /* max_rows: rows per prefill pass (longer
                                     prompts are processed in passes) */
} qwen2_info_t;

/* Checks hyperparameters without touching a GPU.  QWEN2_OK or QWEN2_E_HPARAMS
 * / QWEN2_E_ARG. */
int qwen2_check_hparams(const qwen2_hparams *hp);

/* Host-side validation of a prefill, exactly as qwen2_prefill performs it
 * (no GPU needed).  Order of checks: E_ARG (n <= 0 or a null pointer),
 * E_SEQ, E_TOKEN, E_POS, E_ORDER. */
int qwen2_check_prefill(const qwen2_hparams *hp, int32_t seq, const int32_t *tokens,
                        const int32_t *positions, int32_t n);

/* Host-side validation of a batched prefill, as qwen2_prefill_batch performs
 * it.  Order: E_ARG (n_batch <= 0, a null pointer, a length <= 0, more than
 * 2^31 - 1 rows), E_SEQ (range, then repeats), then each sequence in turn as
 * qwen2_check_prefill checks it. */
int qwen2_check_prefill_batch(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                              const int32_t *lens, const int32_t *tokens,
                              const int32_t *positions);

/* Host-side validation of a decode batch, as qwen2_decode performs it.
 * Order: E_ARG, E_SEQ (range, then repeats), E_POS. */
int qwen2_check_decode(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                       const int32_t *positions);

/* Creates a context on the current HIP device: copies the host weights into
 * a library-owned device weight store (repacked for the kernels; the caller
 * may free its copies on return), allocates a zero-filled f32 KV cache
 * [n_layer][n_seq][n_head_kv][n_ctx][head_dim] for K and for V, scratch
 * activations and the RoPE cos/sin table.  Synchronous.  On failure *out is
 * NULL and nothing stays allocated.
 * Debug checks (the GPU guards of the minfer page, section 7, that fail with
 * the offending values): with the environment variable QWEN2_DEBUG_CHECKS=1
 * at load, every prefill, batched prefill and decode of the context also
 * hashes every KV-cache word (f32 K and V and both binary16 mirrors) outside
 * the (sequence, position) slots the call may write, before and after the
 * call, and scans the K / V it wrote, its read-out hidden rows and its
 * logits (when given) for non-finite values.  Such a call waits for its
 * stream and returns QWEN2_E_DEBUG, with the place and the value in
 * qwen2_last_error, if the cache changed outside those slots or a value is
 * not finite.  Slow (two passes over the whole cache per call); off by
 * default. */
int qwen2_load(const qwen2_hparams *hp, const qwen2_weights *w, void *stream, qwen2_ctx **out);

/* Runs the prompt (or a continuation) of one sequence.
 *   seq        sequence slot in [0, n_seq)
 *   tokens     host [n] token ids, positions host [n] strictly increasing,
 *              each in [0, n_ctx) (minfer page, section 6: a position >= n_ctx
 *              is a hard error)
 *   logits_dev device [n_vocab] f32 or NULL: logits of the last row
 *   argmax_dev device [1] int32 or NULL: lowest index of the largest logit
 * The K/V of every row is stored in the sequence's slots at its position
 * before any row attends; a row at position p attends to slots 0..p (slots
 * never written hold zeros).  Only the last row is read out (the tail-row
 * cut of the minfer page, section 3). */
int qwen2_prefill(qwen2_ctx *ctx, int32_t seq, const int32_t *tokens, const int32_t *positions,
                  int32_t n, float *logits_dev, int32_t *argmax_dev, void *stream);

/* Runs the prompts (or continuations) of n_batch distinct sequences in one
 * call (positions are data, so prefill, decode and continuation are one
 * computation: minfer page, section 6).  The rows of all sequences share each projection's matrix product
 * (passes of up to max_rows rows; a sequence may straddle two passes) and
 * attention runs per sequence, so each sequence gets what qwen2_prefill on
 * its own rows gives, up to rounding order.
 *   seq_ids    host [n_batch] distinct slots in [0, n_seq)
 *   lens       host [n_batch] rows of each sequence, each > 0
 *   tokens, positions  host [sum of lens]: the rows of sequence b follow
 *              those of sequence b - 1; within a sequence the rules of
 *              qwen2_prefill hold (positions strictly increasing, each in
 *              [0, n_ctx), K/V stored before any row attends)
 *   logits_dev device [n_batch, n_vocab] f32 or NULL: row b is the last
 *              row of sequence b
 *   argmax_dev device [n_batch] int32 or NULL
 * Every check (qwen2_check_prefill_batch) precedes any device work, so a
 * rejected call leaves the cache untouched.  Afterwards qwen2_read_hidden
 * returns n_batch rows.  Asynchronous on `stream`; the host arrays may be
 * reused on return. */
int qwen2_prefill_batch(qwen2_ctx *ctx, int32_t n_batch, const int32_t *seq_ids,
                        const int32_t *lens, const int32_t *tokens, const int32_t *positions,
                        float *logits_dev, int32_t *argmax_dev, void *stream);

/* One decode step for n_batch distinct sequences (row b belongs to
 * seq_ids[b] at positions[b]).
 *   seq_ids, positions  host [n_batch]
 *   tokens_dev          device [n_batch] int32; may be the argmax_dev of the
 *                       previous step (even the same buffer), so a greedy
 *                       loop needs no host round trip.  Ids outside
 *                       [0, n_vocab) are replaced by 0 and latch a device
 *                       flag reported by qwen2_sync_status.
 *   logits_dev          device [n_batch, n_vocab] f32 or NULL
 *   argmax_dev          device [n_batch] int32 or NULL */
int qwen2_decode(qwen2_ctx *ctx, int32_t n_batch, const int32_t *seq_ids, const int32_t *tokens_dev,
                 const int32_t *positions, float *logits_dev, int32_t *argmax_dev, void *stream);

/* next_token_probs (nnterp page, the standardized tap list: the next-token
 * distribution at the last position): the softmax of each of `rows` rows of
 * logits_dev [rows, n_vocab] f32 (as written by a prefill or decode) into
 * probs_dev [rows, n_vocab] f32, p = e^(x - max) / sum e^(x - max).
 * rows in [1, max(n_seq, 8)], else E_ARG.  Enqueued on `stream`; uses a
 * context-owned partial-sum buffer, so calls on one context must not
 * overlap. */
int qwen2_next_token_probs(qwen2_ctx *ctx, const float *logits_dev, int32_t rows,
                           float *probs_dev, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * softmax as qwen2_next_token_probs, with no context.  logits_dev [rows,
 * n_vocab] f32 -> probs_dev [rows, n_vocab] f32, rows in [1, 64], n_vocab >=
 * 1 (else QWEN2_E_ARG).  Its partial sums live in a fixed 8 KiB device array
 * inside the library (one per GPU, held until the process ends), so the call
 * allocates nothing; every call on one GPU shares that array, so calls that
 * overlap on one GPU (different streams, or threads) race and must be
 * ordered by the caller.  Enqueued on `stream` on the current device; the
 * first call on a device also looks up the array's device address
 * (QWEN2_E_HIP if that fails).  Errors are reported by qwen2_last_error(NULL). */
int qwen2_next_token_probs_static(const float *logits_dev, int32_t rows, int32_t n_vocab,
                                  float *probs_dev, void *stream);

/* Stop ids as data (eos and im_end, minfer page, section 5; the Qwen2.5
 * ids are 151643 and 151645): up to 8 ids in [0, n_vocab); n = 0 clears
 * them (the default).  From then on every greedy read-out (prefill, batched
 * prefill, decode) whose id is one of them latches, for its sequence slot,
 * the smallest such read-out position, so a loop that runs ahead on the
 * device can be cut back afterwards.  E_ARG for n outside [0, 8], E_TOKEN for
 * an id out of range.  Synchronous: call it while no call that reads the
 * table is in flight. */
int qwen2_set_stop_ids(qwen2_ctx *ctx, const int32_t *ids, int32_t n);

/* Copies the latched stop positions to out_dev [n_seq] int32 (-1: no stop
 * id read out yet) and, if clear != 0, resets them.  Enqueued on `stream`. */
int qwen2_read_stops(qwen2_ctx *ctx, int32_t *out_dev, int32_t clear, void *stream);

/* Copies the read-out rows of the last prefill/decode (1 row after a
 * prefill, n_batch rows after a batched prefill or a decode) to out_dev
 * [rows, n_embd] f32.
 * which = 0: the last layer's layer_output; 1: final_norm_output (nnterp
 * names).  Enqueued on `stream`. */
int qwen2_read_hidden(qwen2_ctx *ctx, int32_t which, float *out_dev, void *stream);

/* Copies K and V of layer `layer`, sequence `seq`, positions pos0..pos0+n-1
 * between the cache and device buffers k_dev, v_dev [n_head_kv, n, head_dim]
 * f32.  For tests and for moving a sequence's state; bounds are checked. */
int qwen2_kv_read(qwen2_ctx *ctx, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                  float *k_dev, float *v_dev, void *stream);
int qwen2_kv_write(qwen2_ctx *ctx, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                   const float *k_dev, const float *v_dev, void *stream);

/* Synchronises `stream` and reports device-side conditions latched since the
 * last call (QWEN2_E_TOKEN for a decode token id out of range), then clears
 * them.  QWEN2_OK otherwise. */
int qwen2_sync_status(qwen2_ctx *ctx, void *stream);

int qwen2_info(const qwen2_ctx *ctx, qwen2_info_t *out);

/* Per-op timing for benchmarks.  While enabled for a set of op kinds, every
 * launch of such an op is bracketed by two HIP events recorded on the call's
 * stream (at most 16384 launches between two reads).  qwen2_prof_read waits
 * for the recorded events, returns the number of timed launches and their
 * summed duration in milliseconds for one kind, and forgets them.  The GEMV
 * (M <= 8) and MFMA (M > 8) variants of an op share its kind. */
enum {
  QWEN2_OP_EMBED = 0,
  QWEN2_OP_QKV = 1,      /* RMSNorm + fused QKV + bias + RoPE + KV store */
  QWEN2_OP_ATTN = 2,     /* causal GQA attention */
  QWEN2_OP_WO = 3,       /* WO + residual */
  QWEN2_OP_GATEUP = 4,   /* RMSNorm + fused gate/up + SwiGLU */
  QWEN2_OP_DOWN = 5,     /* down + residual */
  QWEN2_OP_LMHEAD = 6,   /* final RMSNorm + lm_head + argmax */
  QWEN2_OP_NORM = 7,     /* standalone RMSNorm of the MFMA path */
  QWEN2_OP_COUNT = 8
};
int qwen2_prof_enable(qwen2_ctx *ctx, uint32_t op_mask /* bit k = op kind k; 0 disables */);
int qwen2_prof_read(qwen2_ctx *ctx, int32_t op, int32_t *launches, double *total_ms);

/* Kernel timing for benchmarks: enqueues `iters` back-to-back launches of
 * one decode-path op (rows <= 8 rows of the context's current activations),
 * layer i % n_layer for launch i, so that a caller's event pair around the
 * call measures the op's average duration with the launch-to-launch
 * overhead amortised.  Cycling through the layers keeps the weight stream
 * coming from HBM rather than a cache.  Only QWEN2_OP_GATEUP is supported
 * (it writes only a scratch buffer, so the model state is unchanged);
 * anything else is QWEN2_E_ARG. */
int qwen2_prof_repeat(qwen2_ctx *ctx, int32_t op, int32_t rows, int32_t iters, void *stream);
/* Device ceilings, measured in the same job as a workload so that its rates
 * can be set against what this device reaches rather than only its spec
 * peaks (8 TB/s HBM, 2.5 PFLOP/s dense f16 MFMA).  No context; errors are
 * reported by qwen2_last_error(NULL).  Enqueued on `stream`; the caller
 * times them with its own events.
 * qwen2_probe_read: n_blocks blocks of 256 threads read the `bytes` (a
 * positive multiple of 16) at buf_dev once, with 16-byte non-temporal loads,
 * and write one fold of the words per wavefront to out_dev [4 n_blocks]
 * uint32.  A buffer larger than the 256 MB Infinity Cache measures HBM.
 * qwen2_probe_mfma: n_blocks blocks of four wavefronts, each issuing
 * 4 iters v_mfma_f32_32x32x16_f16 on register operands (2 * 32 * 32 * 16
 * flop each), and writing one sum per wavefront to out_dev [4 n_blocks] f32.
 * QWEN2_E_ARG for a null pointer, bytes not a positive multiple of 16, iters
 * < 1 or n_blocks outside [1, 65536]. */
int qwen2_probe_read(const void *buf_dev, size_t bytes, int32_t n_blocks, uint32_t *out_dev,
                     void *stream);
int qwen2_probe_mfma(int32_t iters, int32_t n_blocks, float *out_dev, void *stream);

const char *qwen2_last_error(const qwen2_ctx *ctx); /* ctx NULL: the last error of a call
                                                       without a context (qwen2_load,
                                                       qwen2_next_token_probs_static,
                                                       qwen2_probe_read, qwen2_probe_mfma) */
const char *qwen2_strerror(int code);

/* Frees every device allocation of the context (synchronises the device). */
void qwen2_free(qwen2_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* QWEN2_MI355X_H */
