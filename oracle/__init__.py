"""CPU oracle for prefix-pinned sliding-window attention. TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The product path (the HIP library and its
Python binding) never imports or calls it, and it never imports the product:
the two share no code. The only module both sides use is ``synth`` (seeded
input values and workload shapes, no attention arithmetic).

Everything here is plain and slow on purpose: NumPy in float64, no blocking,
no fusion, no reordering beyond what the definitions state.

Sources, cited by title and section throughout this package:

* [PS] "Prefix Sliding 3倍加速" -- the PaperDaily explainer (longzhangge.com)
  of the Prefix Sliding paper on long test-time reasoning: section 03 (the
  visible set A(t) and the generation loop), 04 (cost), 05 (position
  encoding: Continue PE vs Reset PE), 06 (the two-level kernel filter).
* [KV-Lean] the pnsm.cn article on verifying a sliding-window KV cache in
  Lean 4: 1.1 (exactness of the window cache, KV-size formula), 1.2 (bug
  taxonomy), 1.3 (the three phases), 2.1 (reference model: full history with
  window and causal masks), 2.2-2.4 (fixed-length target model, lastWindow,
  Valid, the step identity, slot positions), 3.1-3.4 (cache structure,
  position invariant, step, ring buffer to list), 4.1-4.3 (step lemma,
  run_correct, the drop/append lemma), 5.1-5.2 (not-full pitfalls, truncated
  subtraction), 5.4 (the #guard example), 6.3-6.4 (export-and-compare,
  spec as fuzz oracle).

Modules:

* ``spec``  -- the list model of the cache (lastWindow, step, run, Valid,
  PositionInvariant, ring-to-list view) and the visible-set predicate.
* ``rne``   -- float64 -> bfloat16 / float32 rounding to nearest even, on bits.
* ``rope``  -- rotary position encoding at absolute positions, float64.
* ``attn``  -- the attention reference: full history, -inf logits outside the
  pinned prefix and the window, softmax in float64.
* ``cache`` -- the expected contents of the bounded cache (positions, stored
  K and V bytes) for a given history.

Parity status of each function is stated in its docstring. Every function
here is pinned by a CPU test to something other than itself (worked examples
of the pages, closed forms, library routines, brute force), except where a
docstring says "parity unpinned".
"""
