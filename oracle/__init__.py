"""fp64 CPU oracle for Jet-Long dynamic bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the library.  It shares no
code with the HIP path.

Parity pins (tests marked "not gpu" in ``tests/test_oracle_*.py``):
  group_size / remote_pos  exhaustive sweep against an exact-rational ceiling,
                           a search for the minimal in-distribution G, the
                           pages' 32K -> 128K example (G = 4), invariants
  rope                     explicit rotation matrices; norm; R(0) = I;
                           R(a) R(b) = R(a + b)
  prefill                  pure-Python brute force; closed forms (q = 0,
                           v = const, d = 2 cosines); G = 1 and w0 >= L equal
                           a library causal attention; w0 = 0 equals causal
                           attention at aliased positions; rows below w0 are
                           plain causal rows
  three_pass               equals the direct routed result to 1e-13
  decode                   brute force with explicit un-rotate / re-rotate;
                           equals the last prefill row at the same L
No function here is "parity unpinned".
"""

from .jetlong import (group_size, remote_pos, rope_theta, rope, prefill,  # noqa: F401
                      prefill_varlen, decode)
