"""Workload shapes and seeded synthetic inputs (no method arithmetic)."""
from .configs import (BERT_BASE, BY_NAME, CONFIGS, GPT2_DECODE, LONG_CAUSAL,  # noqa: F401
                      PQ_DECODE, TINY, Config, keep_count, scaled)
from .gen import make_decode_inputs, make_inputs, make_prefill_inputs, random_scores  # noqa: F401
