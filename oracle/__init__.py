"""CPU oracle for the OSCAR INT2 KV-cache hot path (decode attention over a BF16 sink |
INT2 history | BF16 recent pool, and the demotion that rotates, clips, quantises and
packs a K/V vector into INT2).

THIS PACKAGE IS TEST INFRASTRUCTURE. Only the test suite, the entry point's smoke check
and the benchmark's CPU-baseline leg may import or call it. The library's GPU path never
routes through it, and it shares no code, header, table or helper with that path.

Everything here is plain, slow fp64 NumPy written from the method's description
(OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization;
the QbitAI article on it describes the rotation R = U * Hadamard * bit-reversal, the
three-segment token pool, the 4-codes-per-byte packing, the scale/zero-point dequant and
the split BF16/INT2 decode joined by an online-softmax merge).

Where the description is silent the module docstrings state the reading taken.

Pinned by the `not gpu` tests: every function here is checked against closed forms,
invariants, brute force or hand-built cases (tests/test_oracle_*.py).
"""

from . import rotation, quant, codebook, clip, pages, groups, attention  # noqa: F401
