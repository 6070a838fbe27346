"""MI355X (gfx950) batch-1 persistent decode engine for MLA + MoE transformers.

The engine is a HIP library with a C ABI (include/pdm.h); this package is its
thin Python binding (engine.Engine), the build step and the roofline
arithmetic used by the benchmark. Importing the package does not load the
library; Engine() does and fails loudly when it has not been built.
"""
from . import _lib  # noqa: F401
from .engine import Engine, describe_plan, query_sizes  # noqa: F401
