"""Seeded synthetic inputs for the product-key memory forward.

This package is the only code that both the oracle (``oracle/``) and the HIP
path (``sparse_key_value_amd``) consume.  It holds workload shapes and random
number streams, and none of the method's arithmetic: no projection, norm,
scoring, selection, softmax, gather or gate happens here.

Modules
-------
``configs``   the named workloads (shapes, dtypes, switches).
``inputs``    host-side generators (NumPy) for x, W_q, sub-keys, W1, W2,
              uniform gather indices, and the row-addressable value-table
              generator (splitmix64 + Irwin-Hall).
``device``    ctypes wrapper of ``libpkm_synth.so``: the same value-table
              generator on the GPU (the table is up to 128 GiB and is never
              shipped from the host), a streaming-read kernel and a plain copy
              kernel used to calibrate bandwidth counters.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
