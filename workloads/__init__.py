"""Seeded synthetic inputs shared by the tests, the smoke check and the bench."""
from .synth import (DecodeCase, PrefillCase, prefill_case, q8_pools, make_case, custom_case, tiny_case, qwen_case,
                    sweep_case, extra_case, skewed_case, long_case, skewed_lengths,
                    SWEEP_B, SWEEP_CTX, EXTRA_POINTS, LONG_POINTS, NAN16)

__all__ = ["DecodeCase", "PrefillCase", "prefill_case", "q8_pools", "make_case", "custom_case", "tiny_case", "qwen_case",
           "sweep_case", "extra_case", "skewed_case", "long_case", "skewed_lengths",
           "SWEEP_B", "SWEEP_CTX", "EXTRA_POINTS", "LONG_POINTS", "NAN16"]
