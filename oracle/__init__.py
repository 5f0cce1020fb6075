"""CPU oracle for the affine group-quantized W4A16 projection ``y = x · dequant(Wq)ᵀ``.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package.  The HIP library and its
Python binding never import it, and this package imports nothing from them.

Everything here is plain NumPy (fp32 where the format fixes fp32, fp64 for
accumulation) or pure-Python loops for tiny cases; see ``w4a16_oracle`` for
the definitions and the passages of the pages each function follows.

Pinning status: every function in ``w4a16_oracle`` is pinned by
``tests/test_oracle.py`` against closed forms, exact brute force, library
routines or mathematical bounds.  No function is "parity unpinned".
"""

from .w4a16_oracle import *  # noqa: F401,F403
from .w4a16_oracle import __all__  # noqa: F401
