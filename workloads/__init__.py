"""Workload shapes and seeded synthetic inputs (no method arithmetic)."""
from .configs import (ADA_GPT2, ADA_LONG, ADA_SMALL, BERT_BASE, BY_NAME, CONFIGS,  # noqa: F401
                      GPT2_DECODE, LONG_CAUSAL, PQ_DECODE, TINY, AdaConfig, Config, keep_count,
                      scaled)
from .gen import (ada_batch_layers, ada_layers, make_decode_inputs, make_inputs,  # noqa: F401
                  make_prefill_inputs, random_scores)
