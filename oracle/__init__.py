"""CPU oracle for the SVQ decode-and-multiply path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.
"""
from . import svq_oracle  # noqa: F401
from . import bruteforce  # noqa: F401
