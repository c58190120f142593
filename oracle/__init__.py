"""Independent CPU oracle for the exact-attention forward and backward passes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP path or its
Python binding.  See ``oracle/attention.py`` (forward) and
``oracle/backward.py`` (gradients) for the definitions, the sources
they follow and the readings taken where the sources are silent.

Every function here is pinned by ``tests/test_oracle_pins.py`` and
``tests/test_oracle_backward.py``; none is "parity unpinned".
"""

from .attention import attention_3pass, attention_online, softmax_probs, visible_mask
from .backward import attention_backward

__all__ = ["attention_3pass", "attention_online", "softmax_probs", "visible_mask", "attention_backward"]
