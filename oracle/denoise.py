"""CPU oracle of the TempCache step inside the denoising loop of a chunk.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows (FAST-AR technical summary, gist.science: the problem
statement, where an autoregressive video diffusion model streams frames and
keeps the keys and values of the frames it has generated in a KV cache; and
section "2. Componentes Principais / A. TempCache", where the current frame's
tokens are matched to the previous frames' cache and merged, attention over a
merged group being shifted by the log of its size, Lemma 5.1).

Readings (the summary does not describe the sampler):
  - a chunk is produced by S denoising steps; at each step the chunk's queries
    attend, in one softmax, over the compressed past (the live slots: logit
    plus ln count) and the chunk's own current keys and values (raw tokens,
    count 1, so no shift);
  - the cache does not change during the steps; once they are done, the
    chunk's final (clean) keys and values are matched and merged frame by
    frame, exactly as in the step without a denoising loop.
"""

from __future__ import annotations

import math

import numpy as np


def attend_with_chunk(Q, k_hat, v_hat, count, K_new, V_new, scale=None):
    """Attention of queries ``Q`` [n][d] over slots plus the chunk's tokens.

    Slots: ``k_hat``, ``v_hat`` [S][d] and ``count`` [S]; logit of slot s is
    <q, k_hat[s]> * scale + ln(count[s]).  Chunk tokens: ``K_new``, ``V_new``
    [T][d]; logit of token j is <q, K_new[j]> * scale.  One softmax over all
    S + T logits; scale defaults to 1/sqrt(d).  float64 throughout.
    Returns ``(O [n][d], lse [n])``; with S + T = 0 the output is zero and the
    log partition function -inf.
    """
    q = np.asarray(Q, dtype=np.float64)
    d = q.shape[1]
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    keys = np.concatenate([np.asarray(k_hat, dtype=np.float64).reshape(-1, d),
                           np.asarray(K_new, dtype=np.float64).reshape(-1, d)])
    vals = np.concatenate([np.asarray(v_hat, dtype=np.float64).reshape(-1, d),
                           np.asarray(V_new, dtype=np.float64).reshape(-1, d)])
    shift = np.concatenate([np.log(np.asarray(count, dtype=np.float64).reshape(-1)),
                            np.zeros(np.asarray(K_new).reshape(-1, d).shape[0])])
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], d)), np.full(q.shape[0], -np.inf)
    z = (q @ keys.T) * scale + shift
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ vals, zmax[:, 0] + np.log(l[:, 0])


def denoise_chunk(cache, Q_steps, K_steps, V_steps, frames, scale=None):
    """One chunk through the denoising loop, then the merge.

    ``cache``: a TempCacheOracle (modified: the final keys and values are
    merged into it).  ``Q_steps``, ``K_steps``, ``V_steps``: [S][H][F*T][d],
    the chunk's tokens at each step, ``frames`` = F frames of T tokens each.
    Returns ``(outs [S][H][F*T][d], lses [S][H][F*T], frame_results)``, where
    step s attends with the cache as it was before the chunk, and
    frame_results are the per-frame results of merging step S-1's tokens.
    """
    S = len(Q_steps)
    H = len(cache.heads)
    outs, lses = [], []
    for s in range(S):
        o_s, l_s = [], []
        for h, hc in enumerate(cache.heads):
            n = hc.n_live
            o, l = attend_with_chunk(Q_steps[s][h], hc.k_hat[:n], hc.v_hat[:n], hc.count[:n],
                                     K_steps[s][h], V_steps[s][h], scale)
            o_s.append(o)
            l_s.append(l)
        outs.append(np.stack(o_s))
        lses.append(np.stack(l_s))
    K, V = np.asarray(K_steps[S - 1]), np.asarray(V_steps[S - 1])
    T = K.shape[1] // frames
    results = [cache.process_frame(K[:, f * T:(f + 1) * T], V[:, f * T:(f + 1) * T])
               for f in range(frames)]
    assert H == K.shape[0]
    return outs, lses, results
