"""CPU oracle for the 1-bit error-compensated compression stage.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy implementation of what the compression stage computes, written from the
pages' equations.  Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the library under ``momentum_compression_amd`` never
does, and shares no code, table or helper with it.

``cpp/onebit_ref.cpp`` (through ``cref``) is a second, plain C++
implementation of the compressed phase, written apart from the numpy one as
straight loops; the tests hold the two bit-identical and use the C++ one where
whole full-size buffers are checked.

Conventions (each module states the passage it follows):

* All buffers are IEEE binary32 and every elementwise operation is one
  correctly rounded binary32 operation in the order the formula is written
  (numpy float32 arithmetic: round to nearest even, no fused multiply-add,
  subnormals kept).  The pages fix fp32 buffers; decisions that turn floats
  into integers (sign bits, INT8 codes) are taken in that same precision.
* A mean is the real mean of the binary32 inputs, computed exactly with
  Python integers and rounded once to binary32 (``exact.mean_abs_f32``).
* Sign convention: bit = (x >= 0), so +0 and -0 encode +1 and NaN encodes -1.
* Packed words: element j lives in uint32 word j >> 5 at bit j & 31.

Parity status per function is listed in each module header; a function whose
result is pinned only by agreement with the GPU path says "parity unpinned".
"""
