"""CPU oracle for the SharQ linear hot path (test infrastructure only).

Nothing in the product path may import this package. Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library under ``activation_sparsity_fp4_amd``.
"""

from .sharq_ref import *  # noqa: F401,F403
from .compact_ref import *  # noqa: F401,F403
from .nvfp4_ref import *  # noqa: F401,F403
