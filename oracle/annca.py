"""CPU oracle of AnnCA prompt-token selection and sparse cross-attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows (FAST-AR technical summary, gist.science, section
"2. Componentes Principais / B. AnnCA"): latent queries and prompt keys are
projected into one shared LSH space; a prompt token is kept for a frame iff it
shares a bucket with at least one query of that frame; the others are pruned
for that frame.  Readings: the LSH is SimHash with its own hyperplanes (L
tables of b bits); "shares a bucket" means equal codes in at least one table;
the kept tokens are attended with plain softmax attention at scale 1/sqrt(d);
an empty selection gives a zero output.
"""

from __future__ import annotations

import math

import numpy as np

from .tempcache import simhash


def select(codes_q, codes_p) -> np.ndarray:
    """Prompt ids j (ascending) sharing a bucket with any query in any table.

    ``codes_q`` [n_q][L] are the codes of one frame's queries, ``codes_p``
    [n_p][L] the prompt keys' codes.
    """
    codes_q = np.asarray(codes_q)
    codes_p = np.asarray(codes_p)
    L = codes_p.shape[1]
    frame_buckets = [set(int(c) for c in codes_q[:, t]) for t in range(L)]
    keep = [j for j in range(codes_p.shape[0])
            if any(int(codes_p[j, t]) in frame_buckets[t] for t in range(L))]
    return np.array(keep, dtype=np.int64)


def softmax_attention(q, k, v, scale=None):
    """Plain softmax attention in float64: (O [n][d], probabilities [n][m])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(q.shape[1])
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.zeros((q.shape[0], 0))
    z = (q @ k.T) * scale
    e = np.exp(z - z.max(axis=1, keepdims=True))
    P = e / e.sum(axis=1, keepdims=True)
    return P @ v, P


def annca_frame(Q, Kp, Vp, planes, scale=None, codes_q=None, codes_p=None):
    """AnnCA for one frame of queries of one head.

    Returns a dict with the selection, the sparse output, the dense output over
    all prompt tokens and, per query, the dense probability mass that the
    pruning drops (``delta``).
    """
    if codes_q is None:
        codes_q = simhash(Q, planes)[0]
    if codes_p is None:
        codes_p = simhash(Kp, planes)[0]
    sel = select(codes_q, codes_p)
    Kp = np.asarray(Kp, dtype=np.float64)
    Vp = np.asarray(Vp, dtype=np.float64)
    o_sparse, _ = softmax_attention(Q, Kp[sel], Vp[sel], scale)
    o_dense, P = softmax_attention(Q, Kp, Vp, scale)
    dropped = np.ones(Kp.shape[0], dtype=bool)
    dropped[sel] = False
    delta = P[:, dropped].sum(axis=1)
    return {"sel": sel, "o_sparse": o_sparse, "o_dense": o_dense, "delta": delta,
            "codes_q": codes_q, "codes_p": codes_p}
