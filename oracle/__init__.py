"""FP64 CPU oracle (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU baseline leg may import
this package.  It shares no code with the HIP library or its binding.
"""
from .softmax_attention import attention, block_terms, visible_pairs  # noqa: F401
from . import layout  # noqa: F401
from . import window  # noqa: F401
from . import a2a  # noqa: F401
