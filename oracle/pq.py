"""CPU oracle of the quantization-based codes: product quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows (FAST-AR technical summary, gist.science, section
"2. Componentes Principais": the nearest-neighbour search of TempCache and
AnnCA uses "LSH or quantization" to put keys, queries and prompt keys in
buckets).  Readings (the summary names the family only):
  - quantization is product quantization: a table splits the d features into
    M equal contiguous slices; slice m has K = 2^(b/M) centroids, and its
    index is that of the centroid nearest to the slice in Euclidean distance,
    ties to the lowest index;
  - the b-bit code of the table concatenates the M indices, slice m at bits
    [m*b/M, (m+1)*b/M); buckets are equal codes, exactly as for SimHash;
  - codebooks [L][M][K][d/M] are given (seeded draws in the tests), not
    trained here.
"""

from __future__ import annotations

import numpy as np


def pq_codes(x, codebooks):
    """Codes of the rows of ``x`` [n][d] under ``codebooks`` [L][M][K][d/M].

    Returns ``(codes [n][L] uint32, gap [n][L][M] float64)``: ``gap`` is the
    distance between the nearest and the second-nearest centroid of each
    slice (+inf with one centroid), which tells callers where a lower
    precision may legitimately pick another index.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    C = np.asarray(codebooks, dtype=np.float64)
    L, M, K, w = C.shape
    n = x64.shape[0]
    bits = int(round(np.log2(K)))
    assert 1 << bits == K and M * w == x64.shape[1]
    codes = np.zeros((n, L), dtype=np.uint64)
    gap = np.full((n, L, M), np.inf)
    for r0 in range(0, n, 1024):              # rows are independent; bounded memory
        r1 = min(n, r0 + 1024)
        for t in range(L):
            for m in range(M):
                xs = x64[r0:r1, m * w:(m + 1) * w]
                # squared Euclidean distance of every row to every centroid
                dist = ((xs[:, None, :] - C[t, m][None, :, :]) ** 2).sum(axis=2)
                idx = np.argmin(dist, axis=1)          # first minimum: lowest index
                codes[r0:r1, t] |= idx.astype(np.uint64) << np.uint64(m * bits)
                if K > 1:
                    part = np.partition(dist, 1, axis=1)
                    gap[r0:r1, t, m] = part[:, 1] - part[:, 0]
    return codes.astype(np.uint32), gap


def ambiguous_codes(x, codebooks, tol=1e-3):
    """[n][L] bool: some slice's two nearest centroids are within ``tol``
    (relative to the slice's squared norm plus one) of each other."""
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    C = np.asarray(codebooks, dtype=np.float64)
    L, M, K, w = C.shape
    _, gap = pq_codes(x64, C)
    scale = np.stack([(x64[:, m * w:(m + 1) * w] ** 2).sum(axis=1) for m in range(M)], axis=1)
    return (gap < tol * (1.0 + scale[:, None, :])).any(axis=2)
