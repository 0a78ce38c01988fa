"""MI355X (gfx950) Kimi Delta Attention core: chunkwise forward, decode step and
segment composition as hand-written HIP kernels behind a C ABI (include/kda.h).

`kda` is the ctypes binding; `inputs` draws the seeded synthetic workloads.
The shared library is loaded on first use and never replaced by a fallback.
"""

from . import inputs  # noqa: F401
from .kda import (  # noqa: F401
    FLAGS_DEFAULT, KDAError, chunk_fwd, load, safe_chunk_size, segment_compose,
    segment_fixup, step, workspace_bytes,
)
