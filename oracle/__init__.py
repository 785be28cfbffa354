"""Plain float64 CPU oracle for the Mamba-2 SSD forward pass and the scalar
linear scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``chunked_linear_scan_amd``) and imports nothing from it; both sides only
consume the same seeded host tensors.

Modules
-------
ssd       the SSD recurrence as a token-by-token loop (the definition), plus a
          brute-force unrolled sum, the decay-free linear-attention form, and
          one decode token (ssd_step)
scan      the scalar recurrence h[t] = a[t] h[t-1] + b[t] as a loop, and its
          affine combine
chunked   a float64 mirror of the chunked (state-space duality) algebra, used to
          pin chunk-size invariance before any GPU code exists
lookback  a float64 simulator of the decoupled look-back tile protocol under
          arbitrary tile completion orders, with deliberately broken variants
compare   rel-L2 and first-mismatch reporting

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (closed forms, brute force, hand-worked fixtures in
``tests/golden/``, invariants, and mutants that must be caught).  No function is
"parity unpinned".
"""
