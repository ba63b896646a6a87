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
                      attention over the full int8 cache; a uniform row whose
                      max p equals the threshold exactly keeps its MSB result
                      (strict test); at a middle threshold the flat head
                      returns p and o of torch's softmax over the full codes
                      and the confident head those over the MSB-only codes.
  decode_attention /  one new token = the last row of causal torch SDPA
  decode_layer        (fp64) over [cache; new k/v], with the new key and
                      value appended in that order; q = 0 gives p = 1/Lc and
                      o = mean of V; two keys whose scores differ by
                      sqrt(dh) ln 3 give p = (3/4, 1/4) (the 1/sqrt(dh)
                      scale); under progressive quantization the stack's
                      importance sums the recomputed probabilities.
  pq_head_attention   with value pruning: V rows 127 e_j (scale 1, code
  (value pruning)     127) expose each kept probability as 127 p (both
                      planes) or 112 p (MSB only); thresholds just below the
                      m-th largest keep m rows; tau = 0 is plain PQ.
  value_pruned_output one-hot V rows expose every kept probability (and
                      thresholds at the m-th largest keep exactly m rows);
                      threshold 0 -> torch attention; threshold > 1 -> 0;
                      uniform rows at and just above 1/n.
  prune_after_step    truth table for r = 0, 1, 3.
  head_attention /    value pruning in prefill: one-hot V rows expose every
  attention_rows      kept probability (torch softmax), extremes, causal
                      row 0, uniform rows at and just above 1/n.
  perhead_prefill_    per-head token pruning in prefill: each head's output
  layer               is torch SDPA over its own keys; one kept key takes all
                      the mass; keeping every key reproduces the dense stack.
  run_prefill_perhead every per-head cut keeps that head's largest
                      importance among its own keys and never revives one;
                      heads choose different keys; on the equal-query
                      inputs (see run_prefill) the whole per-head cascade
                      against its closed form (one softmax per head over its
                      own keys).
  ada_ref (module)    see tests/test_ada_oracle.py: brute force, closed
                      forms, cascade from all / no tokens, a hand-worked
                      case, Proposition 4; run_cascade's sets and Gram pair
                      counts over a four-layer stack against scalar loops
                      over the three steps.
  run_prefill         closed form: with every token's query equal (x[:, 0]
                      = 1, Wq zero outside row 0, Wo writing nothing into
                      column 0) each head's probability rows are one vector
                      softmax (bidirectional) or its prefix-normalised form
                      (causal); the whole cascade - outputs, cumulative token
                      and head importance, token and head cuts, compacted
                      positions - is recomputed from that without a score
                      matrix, on a case where the cumulative and the last
                      layer's importance choose different sets. Also: total
                      importance per layer, keep-all = repeated dense layers.
  run_decode          closed form at q = 0: every cache entry takes 1/Lc per
                      head, so each layer adds the mean V row times Wo, the
                      importance is layers x heads / Lc per step and cuts
                      keep the longest-present entries; checked over five
                      steps with the cut once, rolling, per head and under
                      progressive quantization across the threshold. Also:
                      value pruning leaves importance unchanged, every rolling
                      cut keeps the largest entries (brute force over
                      candidates) and never revives a pruned one, a budget
                      that never cuts reproduces the plain run; per-head
                      pruning reduces to the shared cut for one head and for
                      identical heads, and each head's cut keeps that head's
                      largest entries.
"""
from . import ada_ref, spatten_ref, topk_engine  # noqa: F401
