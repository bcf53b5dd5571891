"""CPU oracle (test infrastructure only): plain float64 numpy implementation of
the routing frontend and block-sparse attention, used by the tests, the smoke
check and the benchmark's CPU-baseline leg.  Never imported by the product."""
