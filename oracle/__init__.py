"""CPU oracle of the TwELL ReLU-gated FFN.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code written from the
pages' description of the method.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(the HIP library and its Python binding) never does, and this package never
imports the product.
"""
from .twell_oracle import *  # noqa: F401,F403
from .twell_oracle import __all__  # noqa: F401
