"""MI355X-native (gfx950) forward hot path of MiniMax Sparse Attention (MSA).

The compute lives in the HIP/C-ABI library ``libmsa.so`` built from ``csrc/``;
this package only marshals arguments to it (see ``binding``), describes the
workloads (``configs``) and draws seeded synthetic inputs (``inputs``).
"""
from . import configs, inputs  # noqa: F401
