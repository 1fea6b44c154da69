"""TurboQuant CPU oracle (test infrastructure, not product code).

Plain, slow, fp64 NumPy implementation of what the codec computes, written
from the method's description and kept independent of the HIP path: it
shares no code, table or constant generator with
``kv_cache_quantization_03_amd``.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.

Parity status of each function is stated in its docstring; the pins that
hold it to something other than itself live in ``tests/test_oracle_*.py``.
"""
from .tq_oracle import *  # noqa: F401,F403
