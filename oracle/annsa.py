"""CPU oracle of AnnSA: bucket-restricted self-attention over the merged cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows (FAST-AR technical summary, gist.science, section
"2. Componentes Principais / C. AnnSA"): the buckets found for the
cross-attention pruning are reused, and each token's query attends only to the
keys that sit in the same bucket(s), which turns self-attention into a
block-sparse operation.

Readings (where the summary is silent):
  - the keys of the self-attention are the live slots of the TempCache after
    the chunk was merged (mirror keys and values, logit shifted by ln count,
    as for the dense step);
  - a query and a slot share a bucket iff their codes are equal in at least
    one table of one LSH family applied to both (the rule AnnCA applies per
    frame, applied here per query); the family is the caller's, e.g. the
    AnnCA hyperplanes;
  - softmax runs over the shared slots only, at scale 1/sqrt(d); a query that
    shares no bucket with any slot gets a zero output and LSE -inf.
"""

from __future__ import annotations

import math

import numpy as np


def shared_mask(codes_q, codes_k) -> np.ndarray:
    """mask[i][s] = True iff query i and slot s have equal codes in some table.

    ``codes_q`` [n_q][L], ``codes_k`` [n_k][L] (unsigned integer codes).
    """
    codes_q = np.asarray(codes_q, dtype=np.uint64)
    codes_k = np.asarray(codes_k, dtype=np.uint64)
    L = codes_q.shape[1]
    mask = np.zeros((codes_q.shape[0], codes_k.shape[0]), dtype=bool)
    for t in range(L):
        mask |= codes_q[:, t][:, None] == codes_k[:, t][None, :]
    return mask


def annsa_attend(Q, k_hat, v_hat, count, codes_q, codes_k, scale=None):
    """AnnSA of queries ``Q`` [n][d] over slots (k_hat, v_hat [S][d], count [S]).

    Logit of slot s for query i, over the slots that share a bucket with i:
    <q_i, k_hat[s]> * scale + ln(count[s]).  float64 throughout.
    Returns ``(O [n][d], lse [n], n_shared [n])``.
    """
    q = np.asarray(Q, dtype=np.float64)
    k = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v_hat, dtype=np.float64)
    cnt = np.asarray(count, dtype=np.float64)
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(q.shape[1])
    mask = shared_mask(codes_q, codes_k)
    O = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    n_shared = mask.sum(axis=1)
    for i in range(q.shape[0]):
        sel = np.nonzero(mask[i])[0]
        if sel.size == 0:
            continue
        z = (k[sel] @ q[i]) * scale + np.log(cnt[sel])
        zmax = z.max()
        e = np.exp(z - zmax)
        l = e.sum()
        O[i] = (e / l) @ v[sel]
        lse[i] = zmax + math.log(l)
    return O, lse, n_shared
