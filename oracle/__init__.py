"""CPU oracle for the group-wise affine quantized linear layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library
(``group_wise_affine_qlinear_amd``) never imports it, and it never imports the
library: the two share no code.
"""
from .qlinear_oracle import *  # noqa: F401,F403
