"""CPU oracle for int4 compressed-domain decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the benchmark's
CPU-baseline leg. The GPU library never imports, links or calls anything here.

Two independent implementations of the same readings of the pages:
  * ``c_oracle``  - plain C (``tq_oracle.c``), fp32 codec, fp64 attention, OpenMP loops;
  * ``np_oracle`` - NumPy, written separately, used to cross-check the C one.
"""
