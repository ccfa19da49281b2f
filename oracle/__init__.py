"""fp64 CPU oracle of Grok-1's attention sub-layer core.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
load anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

It is written from the Grok-1 walkthrough pages (see ``grok_oracle``'s module
docstring for the sources) as plain NumPy in float64, with no blocking, fusion
or reordering beyond what those pages state. It shares no code with the HIP
library and imports nothing from it.

Every function is pinned by ``tests/test_oracle_pins.py``. Parity unpinned:
the reference's own bf16 rounding sequence inside attention (whether logits
are rounded to bf16 before the float32 cast, and the bf16 rounding of the
normalised probabilities) is not fixed by the pages beyond the stated
tolerance, so the oracle keeps those steps in float64.
"""
from .grok_oracle import *  # noqa: F401,F403
from .grok_oracle import __all__  # noqa: F401
