"""Seeded synthetic inputs for the mixed-precision KV transfer path.

This package only draws random tensors with the shapes and value structure of
the workloads (configuration table in :mod:`workloads.configs`, generators in
:mod:`workloads.gen`).  It holds none of the method's arithmetic: no score, no
tier rule, no quantizer, no payload layout.  Both the CPU oracle and the GPU
path consume exactly the bytes produced here.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from . import gen  # noqa: F401
