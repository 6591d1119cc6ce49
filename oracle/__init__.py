"""CPU oracle for causal kernelized linear attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
in this package.  The HIP library and its Python binding never do, and this
package imports nothing from them.

Pins: every function here is pinned in ``tests/test_oracle.py`` against values
fixed by the pages (worked examples stored under ``tests/golden/``), closed
forms, invariants and brute force on tiny inputs; ``tests/test_oracle_mutants.py``
plants mistakes in a copy of the recurrence and checks the pins catch each one;
``tests/test_oracle_bwd.py`` does the same for the backward (``tests/pins_bwd.py``).
"""
from .recurrence import EPS, causal_linear_attention, decode_step, favor_features, feature_map, phi, relu_features
from .chunked import chunked_linear_attention
from .backward import causal_linear_attention_bwd

__all__ = ["EPS", "phi", "relu_features", "favor_features", "feature_map", "causal_linear_attention",
           "decode_step", "chunked_linear_attention", "causal_linear_attention_bwd"]
