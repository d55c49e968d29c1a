"""CPU oracle of the key projection with SimHash codes taken in its epilogue.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows (FAST-AR technical summary, gist.science, section
"2. Componentes Principais / A. TempCache", "Mecanismo"): the keys TempCache
hashes, matches and merges are the attention layer's keys, i.e. the linear
projection of each token's hidden state.  Producing a key and hashing it in
one pass is a fusion of two steps that each have a plain definition, so the
oracle is those definitions written out:
  - the stored key is the exact product x W^T rounded once to the key dtype
    (bfloat16, round to nearest, ties to even);
  - its code is SimHash of the stored key (``tempcache.simhash``).

Readings (the summary names no layer details): W in the linear layer's
layout [H*d][D_in] (out features by in features), head h owning out features
[h*d, (h+1)*d); no bias, normalisation or positional rotation, which belong
to the surrounding model.
"""

from __future__ import annotations

import numpy as np

from .tempcache import simhash


def round_bf16_exact(v) -> np.ndarray:
    """Nearest bfloat16 value of each float64 ``v`` (ties to even), as float64.

    A bfloat16 number keeps 8 significant bits: with v = m * 2^e,
    0.5 <= |m| < 1, the result is rint(m * 2^8) * 2^(e - 8), rint rounding
    halves to even.  (Finite values in bfloat16's normal range.)
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def project_keys(X, W, heads, planes):
    """Keys and codes of tokens ``X`` [N][D_in] under ``W`` [H*d][D_in].

    Returns ``(K [H][N][d] float64 holding bfloat16 values, codes
    [H][N][L] uint32, proj [H][N][L][b])``; ``proj`` are the SimHash
    projections of the stored keys (for ambiguity checks).
    """
    x = np.asarray(X, dtype=np.float64)
    w = np.asarray(W, dtype=np.float64)
    d = w.shape[0] // heads
    K = round_bf16_exact(x @ w.T)                       # [N][H*d]
    K = K.reshape(x.shape[0], heads, d).transpose(1, 0, 2)
    codes, proj = zip(*(simhash(K[h], planes) for h in range(heads)))
    return K, np.stack(codes), np.stack(proj)
