"""fp64 CPU oracle for grouped shared-prefix attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check of the
package entry point and the CPU-baseline leg of the benchmark use it.

What it computes is the repeated-prefix baseline that Prefix Grouper claims to
reproduce exactly: every group member i is encoded as its own sequence
[P; R_i] with standard causal attention, and the results are mapped back onto
the packed rows [P; R_1; ...; R_G].  Sources (web pages about "Prefix
Grouper: Efficient GRPO Training through Shared-Prefix Forward"):
  * the "prefix-grouper-grpo" page on skillsmp.com, section "Step 1: Set Up
    Standard GRPO Baseline" (each [prefix, response] encoded on its own) and
    "Step 3: Restructure Input Format" (the packed order);
  * the Pith review on pith.science, "What carries the argument" (prefix
    self-attention once, suffix queries see the prefix plus their own
    response, baseline position ids) and "Core claim" (Lemma 2.1: identical
    outputs and gradients).

Modules:
  attention  -- baseline forward/backward of grouped attention (full, or for
                sampled rows), packed position ids, pair counts.
  decoder    -- a small pre-norm decoder evaluated per member sequence, with a
                hand-written backward (for the 4-layer decoder workload).

Parity pins (what ties this oracle to something other than itself) live in
tests/test_oracle_*.py; every function is pinned there unless its docstring
says "parity unpinned".
"""
