"""CPU oracle for the low-bit weight-only matmul -- TEST INFRASTRUCTURE ONLY.

A plain, slow, single-threaded C implementation (``lowbit_oracle.c``) of what
the GPU library computes, carried in double precision, plus this ctypes
loader.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it.  The GPU library never imports, links or calls
anything here, and nothing here imports the GPU library.

Parity status of each function (what pins it; see ``tests/test_oracle_pins.py``):
  f16/bf16 decode and RNE encode .... pinned (numpy float16 / torch bfloat16
                                      over all 65536 bit patterns, ties)
  e4m3 / ue8m0 decode ............... pinned (torch float8_e4m3fn /
                                      float8_e8m0fnu, all bytes)
  w4_unpack / w4_dequant ............ pinned (hand-worked bytes, 16-code
                                      identity, exact rational check)
  w4_matmul ......................... pinned (exact rational brute force,
                                      numpy float64 matmul, one-hot, zero,
                                      power-of-two and K-split invariants)
  lut3_dequant / moe_gemm ........... pinned (hand-worked codebook example,
                                      exact rational brute force, numpy
                                      float64 grouped matmul)
  moe_align ......................... pinned (brute-force invariants: every
                                      slot once, ascending within expert,
                                      padding, block -> expert map)
"""
from .oracle import *  # noqa: F401,F403
