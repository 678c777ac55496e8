"""MI355X (gfx950) selected-token logprob drift library.

* ``binding`` - ctypes binding of the C ABI in ``include/drift.h`` (loads ``libdrift.so``;
  fails loudly when it has not been built).
* ``synth``   - seeded synthetic workloads (random inputs only; no method arithmetic).
* ``build``   - compiles the HIP sources under ``csrc/`` into ``libdrift.so``.
"""
