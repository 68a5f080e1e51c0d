"""CPU oracle for the CEM plan step over an action-conditioned predictor.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark import this package; the HIP product path never
does, and this package imports nothing from it.  It is deliberately plain and
slow: NumPy, float64 for the predictor and the energies, every step in the
order the source describes it.

Source: page "Real-Time Inference for JEPA World Model Architectures with Ray"
(dev48.org).  Section 01, "Where the sixteen seconds actually goes", describes
one planning step: draw candidate action sequences from a Gaussian centred on
the current best guess, push each through the predictor, score the result
against the goal embedding, keep the best ones, re-centre the Gaussian on
them, repeat for ten rounds, execute the first action.  Section 05 adds that
the predictor is frame-causal, so a KV cache across rollout steps is exact.

Parity status of each module (what pins it, besides itself):
  philox    - pinned to rocRAND's Philox-4x32-10 engine (independent source)
              plus bijectivity on a fixed key.
  sampler   - pinned by closed-form special cases and distribution tests.
  predictor - layer pinned to torch.nn.TransformerEncoderLayer (norm_first,
              exact GELU) and scaled_dot_product_attention; mask pinned by
              enumeration; KV-cached rollout pinned to full recompute; the
              composed rollout pinned to a torch.nn module build.
  energy    - closed forms and brute force.
  select    - brute-force sort with ties and NaN.
  refit     - closed forms and Python's statistics module.
  cem       - convergence to the known minimum of a quadratic energy.
"""

from . import cem, energy, philox, predictor, refit, sampler, select  # noqa: F401
