"""CPU oracle for the DSpark draft-and-verify round: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, `__graft_entry__.smoke()` and the
CPU-baseline leg of the benchmark use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or generators); the two
meet only in the seeded inputs both of them read.

Every function restates a passage of the DSpark pages (arXiv:2607.05147):

  sample.py      eq (4) and eq (5) of the reading notes (semi-autoregressive
                 factorisation, low-rank Markov head) and the sequential loop
                 of dspark_cycle (caijizhuo page, section 四)
  confidence.py  eq (7) of the reading notes (confidence head) and its
                 sequential temperature scaling
  schedule.py    Algorithm 1 of the reading notes (hardware-aware prefix
                 scheduler), its worked examples, Lemmas 1-2 and Appendix A
  verify.py      the rejection-sampling rule and residual resampling
                 (reading notes, speculative-decoding background and
                 eq (8a)-(8c); caijizhuo page, section 四 steps 5-6)
  round.py       one full round in the order of the end-to-end loop
                 (reading notes, "full decode loop" pseudocode, steps 1-13)

Parity status: every function has a pin in tests/test_oracle_*.py except the
sampler's agreement with the pages' own Markov example, which prints output
probabilities but no inputs; the sampler is pinned in distribution and by
special cases instead (see sample.py).
"""
