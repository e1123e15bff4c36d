"""Plain, slow CPU oracle of the speculative-decoding verify step (fp64).

TEST INFRASTRUCTURE ONLY. The product path never imports, calls or links
anything in this package; only the test suite, the smoke check and the
benchmark's CPU-baseline leg do. It shares no code with the HIP library.

What it computes (each module cites the passage it follows):

* ``philox``    - Philox4x32-10 counter-based uniforms keyed by (seed, sequence
                  id, absolute position).
* ``attention`` - paged-KV attention of the k+1 verify rows, causal inside the
                  draft, written out as the plain definition.
* ``reject``    - the lossless acceptance chain: accept a draft with
                  probability min(1, p/q), resample the first rejected position
                  from the normalised residual max(0, p - q), draw a bonus token
                  from p after full acceptance; decision margins are recorded.
* ``commit``    - the accepted length rolls the committed cache length forward.

Parity pins (tests marked ``not gpu``): every function above is pinned to
something other than itself - a library routine (rocRAND's Philox engine,
torch's scaled-dot-product attention), dense brute force, closed forms,
exhaustive enumeration of the 2^24 uniform grid, and Monte-Carlo checks of the
lossless guarantee. No function here is "parity unpinned".
"""
