"""CPU oracle for the routed-expert layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy reference of what the layer computes.
Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library (no
kernels, headers, tables or helpers) and never imports it; the seeded input
generator in ``synth`` is the only code both sides use.

What the layer is (the "gracetier" write-up, section 1 "The idea", and the
GB300 write-up's paragraph on the mixture-of-experts design): per token a
router picks the 6 best of 384 experts; the picked experts that are cold are
copied from pinned host memory into their fixed slot of one HBM scratch area
shared by every layer; then one grouped call runs every picked expert's FFN
as if all were resident, and the experts' outputs are added with the routing
weights.  The pages give no formulas; every step below states the reading it
takes, and the modules cite the passage they follow.

Modules
  mx      MXFP4 element and scale decoding (e2m1 codes, e8m0 scales / 32)
  blob    the per-expert byte layout
  route   router logits, top-k selection, routing weights
  ffn     SwiGLU expert FFN and the weighted top-k combine
  gather  the picked-cold set and the scratch copy
  layer   one whole layer end to end
  residency  pick counts, decayed scores and the swap rule of the adaptive
             residency manager; the fingerprint of the byte audit

Offline recipe scripts (they route with the oracle and write the seeded input
recipe's data under synth/): calibrate_zipf, calibrate_verify.

Every function here is pinned by tests against something other than itself
(format tables, brute force on tiny inputs, closed forms, invariants); none is
"parity unpinned".
"""
