"""CPU oracle for the memory layers' hot paths -- TEST INFRASTRUCTURE ONLY.

Plain, slow NumPy code in float64 that states what the method computes.  It is
used only by ``tests/``, by ``__graft_entry__.smoke()`` (to check one small GPU
run) and by the ``cpu_baseline`` leg of ``bench.py``.  The product library in
``sparse_key_value_amd`` never imports, calls or links anything here, and this
package imports nothing from it.  Both sides read their inputs from ``synth``.

Modules: ``pkm`` (the memory-layer forward), ``engram`` (hashed n-gram lookup),
``ma`` (Memory Attention token-memory values), ``backward`` (the gather backward and
the sparse update).
"""
