"""CPU oracle for the TempCache attention step, AnnCA selection, AnnSA,
product-quantization codes, the step inside a chunk's denoising loop, the key projection with its
SimHash codes, and the rotation-corrected M-degree approximation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the HIP library and its Python
binding never do, and there is no CPU fallback built on it.

Pinned by the CPU tests against facts fixed independently of this code: the
Lemma 5.1 closed form (merged attention over identical keys equals dense
attention over the raw tokens), the SimHash collision law, brute-force top-1
search, special cases that reduce to library routines, conservation of
token counts, hand-derived worked examples under ``tests/golden/``.

Parity unpinned: the approximation quality of merging *non-identical* keys
(the pages give only end-to-end video metrics for it), the LRU eviction order
and the rollout generator, which are readings of silent passages and are
checked through invariants (a hand-derived worked example pins the eviction
order to its reading, which the pages themselves do not fix).
"""

from .tempcache import (  # noqa: F401
    CapacityError,
    FrameResult,
    HeadCache,
    TempCacheOracle,
    bf16_round,
    cosine,
    simhash,
    to_storage,
)
from . import annca  # noqa: F401
from . import annsa  # noqa: F401
from . import pq  # noqa: F401
from . import denoise  # noqa: F401
from . import project  # noqa: F401
from . import rope  # noqa: F401
