"""TempCache compressed-KV attention step on AMD MI355X (gfx950).

The hot path -- SimHash hashing, bucketed top-1 matching, running-mean merging
into a bounded slot store, and attention with a ln(count) logit bias, plus
AnnCA prompt selection -- runs in hand-written HIP kernels behind the C ABI of
``include/fastar.h`` (``libfastar.so``).  This package is the thin Python
binding: torch provides device memory and streams.
"""

from .binding import (  # noqa: F401
    BF16,
    F32,
    LIB_PATH,
    Cache,
    CacheConfig,
    FastarError,
    annca_attend,
    annca_attend_static,
    annca_select,
    attend_subset,
    hash_codes,
    pq_codes,
    library,
    planes_to_host,
    workspace_bytes,
)
