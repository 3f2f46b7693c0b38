"""CPU oracle for speculative sampling: the plain, slow, obviously correct reference.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and this package imports nothing from the product path: the two share
no code.  Inputs reach both sides from the seeded generators in
``speculative_decoding_forward_amd.synth``, which hold none of the method's
arithmetic.

Sources (the web pages this method is described on):
  [ZSM]  "Accelerating Large Language Model Decoding with Speculative Sampling"
         (zeroshotmind.com explainer of Chen et al.)
  [CANON] "57 Speculative Decoding" (ml-canon summary of Leviathan et al. and Chen et al.)
  [LENS] "Speculative Decoding from Scratch -- How a Tiny Draft Model Speeds Up an
         LLM Without Changing a Single Output" (ta-paperlens walkthrough of Leviathan et al.)
  [GC]   "Speculative Decoding: Getting 3x Speedups Without Changing the Model"
         (General Compute blog)
  [NOTE] "NOTE-159: Accelerating Large Language Model Decoding with Speculative
         Sampling" (anthology-of-the-sota note)

Modules:
  philox   -- Philox4x64-10 and the 24-bit uniforms (counter = (round, j, b, purpose)).
  sampling -- knob transform (temperature / top-k / top-p), inverse-CDF sampling,
              the accept / resample / bonus rule for one sequence row.
  model    -- decoder-only transformer forward with a KV cache (fp64 arithmetic with
              the bf16 rounding points of the spec mirrored).
  rounds   -- the speculative round state machine (draft K, verify, accept, roll back).
  theory   -- closed forms: acceptance rate, expected tokens per target call,
              expected wall-time improvement.

Parity status per function is stated in each module header.  The transformer
architecture itself is not fixed by the pages (they only say "transformer"), so
the layer definition in ``model`` is "parity unpinned" with respect to the pages:
it is pinned only by structural properties and library cross-checks.
"""
