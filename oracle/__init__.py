"""CPU oracle of the flow-matching action-expert denoise loop.

TEST INFRASTRUCTURE ONLY: a plain, slow numpy (fp64) definition of what the
denoise loop computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it.  The HIP library never calls it,
and the two share no code; both consume the seeded inputs of ``synth``.

Pins (what fixes each function independently of itself) live in
``tests/test_oracle_pins.py``; every function here has at least one.  The
pages print no worked numerical example of the expert, so the end-to-end
output at the real model sizes is fixed by these pinned functions, not by a
printed value.
"""
from .denoise import *  # noqa: F401,F403
from .denoise import __all__  # noqa: F401
