"""Oracle: plain, slow, CPU reference of the sparse masked MHA forward path.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import or run it.  The HIP product path
never calls into it, and it shares no code, header, table or constant with
the HIP sources.

Sources (cited by page title and section):

* "Accelerating Sparse Transformer Inference on GPU", arXiv catalogue
  record, abstract: STOF maps masked MHA onto row-wise or block-wise kernels
  that read a dedicated storage format, chosen by an analytical model.
* "Accelerating Sparse Transformer Inference on GPU", gist.science
  explainer, Technical summary > Methodology > 1. Unified MHA module: the
  two-level format (BSR outer tiles split into full and partial lists,
  one 64-bit bitmap per 8x8 inner tile of a partial outer tile, skipped
  empty tiles, exact masking) and the two kernels.

Contents:

* ``attention``: fp64 dense masked softmax(Q K^T / sqrt(d)) V.  The method
  reaches exactly this result (skipping an all-masked tile changes no
  value), so the oracle is the plain definition.
* ``encode``: the two-level mask encoding, as a scalar C loop
  (``encode_ref.c``) and a pure-Python twin for small masks.

Parity pins: see tests/test_oracle_attention.py and
tests/test_oracle_encoder.py.  Every function here is pinned; none is
"parity unpinned".
"""
