"""CPU oracle of the Qwen2 decoder forward pass.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this package.  The GPU library does not,
and this package imports nothing from the GPU library.
"""
from .qwen2_oracle import (F16_TABLE, Hparams, OracleError, Qwen2Oracle, Result,
                           argmax_lowest, decode_f16, hparams_for, linear,
                           rms_norm, rope_angles, rope_interleaved,
                           rope_rotate_half, silu, softmax)

__all__ = ["F16_TABLE", "Hparams", "OracleError", "Qwen2Oracle", "Result",
           "argmax_lowest", "decode_f16", "hparams_for", "linear", "rms_norm",
           "rope_angles", "rope_interleaved", "rope_rotate_half", "silu", "softmax"]
