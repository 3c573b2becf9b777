// Host-side validation of hyperparameters and calls.  No HIP here: these
// checks run before anything is enqueued, so a rejected call leaves the KV
// cache and the context unchanged (the minfer page, section 6 and its
// troubleshooting list: a position >= n_ctx is rejected with an error, the
// context is never cut short to fit).
#include <stdio.h>

#include <string>
#include <vector>

#include "../../include/qwen2.h"
#include "validate.h"

namespace q2 {

static int fail(std::string *msg, int code, const char *fmt, long long a = 0, long long b = 0) {
  if (msg) {
    char buf[256];
    snprintf(buf, sizeof buf, fmt, a, b);
    *msg = buf;
  }
  return code;
}

int check_hparams(const qwen2_hparams *hp, std::string *msg) {
  if (!hp) return fail(msg, QWEN2_E_ARG, "null hparams");
  if (hp->n_layer <= 0 || hp->n_embd <= 0 || hp->n_head <= 0 || hp->n_head_kv <= 0 ||
      hp->head_dim <= 0 || hp->n_ff <= 0 || hp->n_vocab <= 0 || hp->n_ctx <= 0 || hp->n_seq <= 0)
    return fail(msg, QWEN2_E_HPARAMS, "every size must be positive");
  if ((long long)hp->n_head * hp->head_dim != hp->n_embd)
    return fail(msg, QWEN2_E_HPARAMS, "n_embd (%lld) != n_head * head_dim (%lld)", hp->n_embd,
                (long long)hp->n_head * hp->head_dim);
  if (hp->n_head % hp->n_head_kv)
    return fail(msg, QWEN2_E_HPARAMS, "n_head %% n_head_kv != 0 (%lld, %lld)", hp->n_head,
                hp->n_head_kv);
  if (hp->n_head / hp->n_head_kv > 8)
    return fail(msg, QWEN2_E_HPARAMS, "query group %lld > 8 is not supported",
                hp->n_head / hp->n_head_kv);
  if (hp->head_dim != 16 && hp->head_dim != 64 && hp->head_dim != 128)
    return fail(msg, QWEN2_E_HPARAMS, "head_dim %lld not in {16, 64, 128}", hp->head_dim);
  if (hp->n_embd % 64)
    return fail(msg, QWEN2_E_HPARAMS, "n_embd %lld is not a multiple of 64", hp->n_embd);
  if (hp->n_embd > 8192)  // (k_rmsnorm_rows: 256 threads x 4 floats x 8 chunks)
    return fail(msg, QWEN2_E_HPARAMS, "n_embd %lld > 8192 is not supported", hp->n_embd);
  if (hp->n_ctx > 131072)  // the decode attention merges at most 2048 64-key chunks
    return fail(msg, QWEN2_E_HPARAMS, "n_ctx %lld > 131072 is not supported", hp->n_ctx);
  if (hp->rope_style != 0 && hp->rope_style != 1)
    return fail(msg, QWEN2_E_HPARAMS, "rope_style %lld: 0 (NonInterleaved) or 1 (Interleaved)",
                hp->rope_style);
  if (!(hp->rope_theta > 0.f) || !(hp->rope_freq_scale > 0.f) || !(hp->rms_eps >= 0.f))
    return fail(msg, QWEN2_E_HPARAMS, "rope_theta, rope_freq_scale must be > 0, rms_eps >= 0");
  if ((long long)hp->n_vocab * hp->n_embd >= (1ll << 40))
    return fail(msg, QWEN2_E_HPARAMS, "vocabulary too large");
  return QWEN2_OK;
}

int check_prefill(const qwen2_hparams *hp, int32_t seq, const int32_t *tokens,
                  const int32_t *positions, int32_t n, std::string *msg) {
  if (!hp || n <= 0 || !tokens || !positions) return fail(msg, QWEN2_E_ARG, "empty prefill or null pointer");
  if (seq < 0 || seq >= hp->n_seq)
    return fail(msg, QWEN2_E_SEQ, "sequence %lld not in [0, %lld)", seq, hp->n_seq);
  for (int32_t i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= hp->n_vocab)
      return fail(msg, QWEN2_E_TOKEN, "token %lld not in [0, %lld)", tokens[i], hp->n_vocab);
  for (int32_t i = 0; i < n; ++i)
    if (positions[i] < 0 || positions[i] >= hp->n_ctx)
      return fail(msg, QWEN2_E_POS, "position %lld not in [0, n_ctx = %lld)", positions[i],
                  hp->n_ctx);
  for (int32_t i = 1; i < n; ++i)
    if (positions[i] <= positions[i - 1])
      return fail(msg, QWEN2_E_ORDER, "positions must increase (%lld after %lld)", positions[i],
                  positions[i - 1]);
  return QWEN2_OK;
}

int check_decode(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                 const int32_t *positions, std::string *msg) {
  if (!hp || n_batch <= 0 || !seq_ids || !positions)
    return fail(msg, QWEN2_E_ARG, "empty decode batch or null pointer");
  for (int32_t b = 0; b < n_batch; ++b)
    if (seq_ids[b] < 0 || seq_ids[b] >= hp->n_seq)
      return fail(msg, QWEN2_E_SEQ, "sequence %lld not in [0, %lld)", seq_ids[b], hp->n_seq);
  std::vector<char> seen(hp->n_seq, 0);
  for (int32_t b = 0; b < n_batch; ++b) {
    if (seen[seq_ids[b]]) return fail(msg, QWEN2_E_SEQ, "sequence %lld repeated in one batch", seq_ids[b]);
    seen[seq_ids[b]] = 1;
  }
  for (int32_t b = 0; b < n_batch; ++b)
    if (positions[b] < 0 || positions[b] >= hp->n_ctx)
      return fail(msg, QWEN2_E_POS, "position %lld not in [0, n_ctx = %lld)", positions[b],
                  hp->n_ctx);
  return QWEN2_OK;
}

int check_prefill_batch(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                        const int32_t *lens, const int32_t *tokens, const int32_t *positions,
                        std::string *msg) {
  if (!hp || n_batch <= 0 || !seq_ids || !lens || !tokens || !positions)
    return fail(msg, QWEN2_E_ARG, "empty prefill batch or null pointer");
  int64_t total = 0;
  for (int32_t b = 0; b < n_batch; ++b) {
    if (lens[b] <= 0) return fail(msg, QWEN2_E_ARG, "sequence %lld of the batch has no rows", b);
    total += lens[b];
  }
  if (total > INT32_MAX) return fail(msg, QWEN2_E_ARG, "more than 2^31 - 1 rows in one batch");
  for (int32_t b = 0; b < n_batch; ++b)
    if (seq_ids[b] < 0 || seq_ids[b] >= hp->n_seq)
      return fail(msg, QWEN2_E_SEQ, "sequence %lld not in [0, %lld)", seq_ids[b], hp->n_seq);
  std::vector<char> seen(hp->n_seq, 0);
  for (int32_t b = 0; b < n_batch; ++b) {
    if (seen[seq_ids[b]]) return fail(msg, QWEN2_E_SEQ, "sequence %lld repeated in one batch", seq_ids[b]);
    seen[seq_ids[b]] = 1;
  }
  int64_t off = 0;
  for (int32_t b = 0; b < n_batch; ++b) {
    int rc = check_prefill(hp, seq_ids[b], tokens + off, positions + off, lens[b], msg);
    if (rc) return rc;
    off += lens[b];
  }
  return QWEN2_OK;
}

}  // namespace q2

extern "C" {

int qwen2_check_hparams(const qwen2_hparams *hp) { return q2::check_hparams(hp, nullptr); }

int qwen2_check_prefill(const qwen2_hparams *hp, int32_t seq, const int32_t *tokens,
                        const int32_t *positions, int32_t n) {
  int rc = q2::check_hparams(hp, nullptr);
  if (rc) return rc;
  return q2::check_prefill(hp, seq, tokens, positions, n, nullptr);
}

int qwen2_check_prefill_batch(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                              const int32_t *lens, const int32_t *tokens,
                              const int32_t *positions) {
  int rc = q2::check_hparams(hp, nullptr);
  if (rc) return rc;
  return q2::check_prefill_batch(hp, n_batch, seq_ids, lens, tokens, positions, nullptr);
}

int qwen2_check_decode(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                       const int32_t *positions) {
  int rc = q2::check_hparams(hp, nullptr);
  if (rc) return rc;
  return q2::check_decode(hp, n_batch, seq_ids, positions, nullptr);
}

const char *qwen2_strerror(int code) {
  switch (code) {
    case QWEN2_OK: return "ok";
    case QWEN2_E_ARG: return "invalid argument";
    case QWEN2_E_HPARAMS: return "unsupported hyperparameters";
    case QWEN2_E_POS: return "position outside [0, n_ctx)";
    case QWEN2_E_TOKEN: return "token id outside [0, n_vocab)";
    case QWEN2_E_SEQ: return "bad or repeated sequence slot";
    case QWEN2_E_ORDER: return "positions of one prefill must strictly increase";
    case QWEN2_E_HIP: return "HIP runtime error";
    case QWEN2_E_OOM: return "out of memory";
    case QWEN2_E_DEBUG: return "a debug check failed (non-finite output or a KV write outside the call's slots)";
    default: return "unknown error";
  }
}

}  // extern "C"
