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
  wb_dequant / wb_matmul ............ pinned (closed form over every code of
                                      every width 1..8, exact rational brute
                                      force, numpy float64 matmul, equality
                                      with the INT4 definition at 4 bits)
  quant_act_i8 ...................... pinned (closed forms on grid rows,
                                      ties to even, invariants over rows of
                                      very different magnitudes)
  w4a8_matmul ....................... pinned (exact rational brute force on
                                      the pinned codes, numpy float64 matmul,
                                      on-grid rows equal the W4A16 product,
                                      one-hot and zero-point cases)
  double_to_e4m3 .................... pinned (every finite E4M3 value, the
                                      midpoints between neighbours, saturation,
                                      against torch float8_e4m3fn)
  mxfp8_quant ....................... pinned (closed form of the block
                                      exponent and element codes, torch E4M3
                                      encode of the scaled block)
  exp2_f32 / silu_f32 ............... pinned (exact at integers, within 1 ulp
                                      of libm 2^t, SiLU within the bound that
                                      follows; the routine itself is the
                                      stated Taylor series from ln 2)
  silu_mul_bf16 / silu_mul_quant .... pinned through silu_f32 and
                                      mxfp8_quant (composition checked on
                                      hand cases)
  moe_combine ....................... pinned (one-hot router weights return a
                                      slot row exactly, numpy float64 sum)
  moe_layer ......................... pinned (wiring: all experts non-local
                                      gives 0, one-hot routing reduces to the
                                      stage chain)
"""
from .oracle import *  # noqa: F401,F403
