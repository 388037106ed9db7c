"""CPU oracle for the IQ4 block-quantised matrix products.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
package: only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or helper with
the HIP library; the only module both sides use is ``synth`` (seeded random numbers).
"""
from .iq4_ref import *  # noqa: F401,F403
from .iq4_ref import __all__ as _nl_all
from .iq4xs_ref import *  # noqa: F401,F403
from .iq4xs_ref import __all__ as _xs_all

__all__ = list(_nl_all) + list(_xs_all)
