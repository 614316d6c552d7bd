"""CPU oracle for the W4A16 / W4A8 group-quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU library never links, imports or falls back to it, and it
shares no code with the GPU library (the two meet only in the seeded input
generators of ``synth``).

See ``oracle/ref.py`` for the functions, their definitions and their pins.
"""
from .ref import *  # noqa: F401,F403
