"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from this package.  The product library
(``gated_deltanet_chunked_delta_amd``) never imports it, links it or falls back
to it; the two share no code.

Contents
--------
``ref``      ctypes binding of ``gdn_oracle.c``: the token-by-token fp64
             recurrence (forward) and its reverse-mode derivative (backward).
``chunked``  a numpy fp64 evaluation of the chunked (WY/UT) form, forward and
             backward, used only to check that the chunked algebra equals the
             token recurrence.
``build``    compiles ``gdn_oracle.c`` with gcc into ``liboracle.so``.
"""
