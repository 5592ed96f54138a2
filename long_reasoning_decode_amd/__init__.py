"""MI355X (gfx950) TriAttention KV-cache pruning: HIP kernels behind a C ABI
(include/triattn.h), with a thin ctypes binding in `triattn`."""
from . import triattn  # noqa: F401
