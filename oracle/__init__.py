"""CPU oracle for the fused W6A16 FP6 linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct reference against which the
HIP library is checked.  It is written in Python + NumPy with float64
arithmetic and shares no code, tables or helpers with the library under
``weight_only_fp6_amd/``.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.

Contents (all in :mod:`oracle.fp6_oracle`):

* decode tables (explicit, one per format: FP6 e3m2 and e2m3, FP5 e2m2, FP4
  e2m1) and the round-to-nearest-even encoder;
* per-row quantizer (input preparation: W fp32 -> codes + fp16 row scales);
* scalar and vectorised unpackers of the packed layout v3 of every format,
  plus a scalar packer used only to pin the unpackers;
* dequantisation ``fp16_RNE(v(c) * s_n)`` and the float64 GEMM
  ``Y_ref = X . Wdq^T``, plus a naive triple loop used to pin it;
* the acceptance check (per-element and Frobenius tolerances).

:mod:`oracle.sparse24` adds the 2:4-sparse FP6 layer: magnitude pruning, the
compressed (code, position) form, its packed layout and the dense
de-quantised weights (built on the FP6 functions above).

Parity status: every function here (and in :mod:`oracle.sparse24`) is pinned
by ``tests/test_oracle_*.py``
against closed forms, IEEE fp16 decoding, torch's float8_e5m2 rounding,
exact (math.fsum) sums, brute force on tiny inputs and hand-derived packed-byte
fixtures under ``tests/golden/``.  No function is "parity unpinned".
"""

from .fp6_oracle import (  # noqa: F401
    E3M2_VALUES,
    E2M3_VALUES,
    E2M2_VALUES,
    E2M1_VALUES,
    FORMATS,
    tile_bytes,
    packed_bytes,
    unpack_tiles,
    decode,
    encode_rne,
    fp16_rne,
    quantize_rows,
    quantize_rows_sampled,
    pack_scalar,
    unpack_scalar,
    unpack_np,
    dequant_ref,
    gemm_ref,
    gemm_naive,
    tolerance_report,
    TOL_ELEM,
    TOL_FROB,
)
