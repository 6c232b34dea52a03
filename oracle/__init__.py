"""CPU oracle for the SVDQuant linear layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The library never does.
"""
from .svdq_ref import *  # noqa: F401,F403
from . import svdq_ref  # noqa: F401
