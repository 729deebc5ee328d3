"""fp64 CPU oracle for the Gated DeltaNet token-mixer hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package; the
product library (``linear_attention_sequence_causal_amd``) never does, and
shares no code with it.

* ``capi``  -- ctypes front end of ``gdn_oracle.c`` (token recurrence, conv,
  localisation and their hand-written reverse modes; the oracle proper).
* ``ref``   -- plain numpy forms for tiny inputs (the page's chunked UT/WY
  evaluation, dense transition products, affine state summaries, per-token
  localisation enumeration) used to pin the oracle to independent results.
"""
