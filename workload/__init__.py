"""Seeded synthetic workloads for shared-prefix GQA attention.

This package holds only shapes, seeds and random-number draws. It contains
none of the attention arithmetic, so both the CPU oracle (``oracle/``) and
the HIP path (``gqa_attention_agentic_amd``) can take their inputs from it
without sharing any code of the method.
"""

from .configs import Workload, WORKLOADS, get_workload, custom, Branch, Group  # noqa: F401
from .generate import generate, Inputs  # noqa: F401
from .subset import cpu_subset  # noqa: F401
