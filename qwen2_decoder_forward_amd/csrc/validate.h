// Host-side validation shared by the C ABI entry points (no HIP).
#pragma once
#include <stdint.h>

#include <string>

#include "../../include/qwen2.h"

namespace q2 {
int check_hparams(const qwen2_hparams *hp, std::string *msg);
int check_prefill(const qwen2_hparams *hp, int32_t seq, const int32_t *tokens,
                  const int32_t *positions, int32_t n, std::string *msg);
int check_prefill_batch(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                        const int32_t *lens, const int32_t *tokens, const int32_t *positions,
                        std::string *msg);
int check_decode(const qwen2_hparams *hp, int32_t n_batch, const int32_t *seq_ids,
                 const int32_t *positions, std::string *msg);
}  // namespace q2
