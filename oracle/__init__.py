"""CPU fp64 oracle for cascade token/head pruned attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke entry and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library under cascade_token_head_amd/.

Parity status of each function (what pins it, in tests/test_oracle.py):
  bf16_round          exhaustive comparison with torch's fp32->bf16 cast on
                      fp32-representable inputs; hand-worked ties.
  head_attention      torch scaled_dot_product_attention (fp64, CPU);
                      closed forms (Q = 0, n = 1, causal row 0); brute-force
                      scalar loops on tiny shapes; permutation equivariance.
  attention_rows      rows of torch softmax attention (fp64); Q = 0 and
                      causal row 0 closed forms.
  column_sums         column sums of torch softmax probabilities given the
                      exact LSE; Q = 0 harmonic closed form (causal); the
                      columns of one head sum to the number of queries.
  prefill_layer       importance sum = heads x queries; Q = 0 closed forms
                      for the column sums (bidirectional and causal);
                      constant-V head importance; keep=1 reproduces dense
                      multi-head attention written with torch.
  topk / kth_value    brute-force subset check (n <= 10), the independent
                      threshold/filter/eliminate engine, properties, and the
                      hand-worked fixtures in tests/golden/.
  quantize_rows etc.  exhaustive nibble round trip over all 256 codes, error
                      bound |x - s q| <= s/2, amax -> +-127, hand-worked rows
                      in tests/golden/.
  pq_head_attention   threshold 0 -> MSB-only attention; threshold > 1 ->
                      attention over the full int8 cache.
  value_pruned_output one-hot V rows expose every kept probability (and
                      thresholds at the m-th largest keep exactly m rows);
                      threshold 0 -> torch attention; threshold > 1 -> 0;
                      uniform rows at and just above 1/n.
  prune_after_step    truth table for r = 0, 1, 3.
  run_prefill /       parity unpinned beyond the composition of the pinned
  run_decode          parts (the pages print no worked example). Invariants
                      checked: total importance per layer, value pruning
                      leaves importance unchanged, every rolling cut keeps
                      the largest entries (brute force over candidates) and
                      never revives a pruned one, a budget that never cuts
                      reproduces the plain run; per-head pruning reduces to
                      the shared cut for one head and for identical heads,
                      and each head's cut keeps that head's largest entries.
"""
from . import spatten_ref, topk_engine  # noqa: F401
