"""CPU float64 oracle for paged KV attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library, with which it
shares no code.

Parity pins (closed forms, invariants, library special cases and brute force
that fix each function) live in tests/test_oracle_pins.py,
tests/test_oracle_mutants.py, tests/test_oracle_rope.py and
tests/test_oracle_block_manager.py.  Every function here is pinned; none is
"parity unpinned".
"""

from . import block_manager as _block_manager
from . import rotary as _rotary
from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__ as _pa_all
from .block_manager import *  # noqa: F401,F403
from .rotary import *  # noqa: F401,F403

__all__ = list(_pa_all) + list(_rotary.__all__) + list(_block_manager.__all__)
