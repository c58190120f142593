"""Independent CPU oracle for the exact-attention forward and backward passes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP path or its
Python binding.  See ``oracle/attention.py`` (forward) and
``oracle/backward.py`` (gradients) and ``oracle/fp8.py`` (the FP8 forward
pass) for the definitions, the sources they follow and the readings taken
where the sources are silent.

Every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_backward.py`` and ``tests/test_oracle_fp8.py``; none is
"parity unpinned".
"""

from .attention import attention_3pass, attention_online, softmax_probs, visible_mask
from .backward import attention_backward
from .fp8 import attention_fp8, attention_online_fp8, dequantise, e4m3_decode, e4m3_round

__all__ = ["attention_3pass", "attention_online", "softmax_probs", "visible_mask", "attention_backward",
           "attention_fp8", "attention_online_fp8", "dequantise", "e4m3_decode", "e4m3_round"]
