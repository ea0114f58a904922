"""CPU oracle for the DSA indexer, its MISA / HISA variants, and the sparse
attention that consumes the selected indices.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The GPU library never calls it and shares no code with it.

Everything here is plain NumPy in float64 on the exact values of the bf16 /
float32 inputs (``indexer.py``; the consumer in ``attention.py``), plus an
independent pure-Python version for
tiny inputs (``brute.py``) and the matching rules used to compare a GPU result
with the oracle (``check.py``).

Parity status of each function (what pins it to something other than itself)
is listed in the headers of ``indexer.py`` and ``attention.py``.
"""
from . import indexer, attention, brute, check  # noqa: F401
