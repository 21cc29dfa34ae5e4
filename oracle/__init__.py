"""CPU oracle for the speculative-sampling verify step and the E2E-TV loss.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct
fp64 restatement of what the pages define. Only the test-suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (``lossless_verify_tv_amd``) never imports,
calls or links anything here, and nothing here imports the product path: the
two share no code, no constants and no helpers. The only module both sides
use is the seeded input generator, which holds none of the method's
arithmetic.

Sources (cited by page title and section throughout):

* P1 -- "Reading Qwen Bebop and DeepSeek DSpark: speculative decoding is
  turning from a trick into systems engineering" (lilfry09.github.io blog
  post), sections "Formulas: what makes a guess worth it" and "Bebop's
  solution: optimise TV directly".
* P2 -- "SpecOPD: Branch-Parallel On-Policy Distillation for Speculative
  Decoding" (paper summary on paper.rainbus.top), section "Acceptance length
  and the E2E-TV objective" and "Method steps", step (6).
* P3 -- "Speculative Decoding and MTP" survey (papers-3lj.pages.dev), sections
  2 (draft/target loop), 3 (probabilistic correctness), 4 (greedy vs
  sampling), 5 (acceptance as overlap), 6 (suffix decay), 7 (speed model).

Modules:

* ``philox``  -- Philox4x64-10 from its published definition.
* ``bf16``    -- bfloat16 decode and round-to-nearest-even encode.
* ``verify``  -- the verify step (scaling, softmax, overlap, accept scan,
  residual / bonus draw, greedy rule, per-request status).
* ``loss``    -- the E2E-TV prefix-product loss and its gradient with respect
  to the draft logits.
* ``objectives`` -- the per-position comparators (per-step TV, CE, KL) with
  their gradients, and every objective with the target given as logits and
  a temperature on both sides.
* ``schedule`` -- confidence-scheduled verify lengths (DSpark).
* ``truncate`` -- top-k / top-p truncation of p and q before the verify step.

Parity status of each function is stated in its module header.
"""

from . import bf16, loss, objectives, philox, schedule, truncate, verify  # noqa: F401
