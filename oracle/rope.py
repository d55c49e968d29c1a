"""CPU oracle of the rotation-corrected M-degree approximation over the cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows (LIPAR technical summary, gist.science, section
"2. Metodologia: LIPAR / B. Recuperação de Atenção / 1. Aproximação de
Grau-M"): in causal attention the most recent tokens weigh most, so the
exponential sum of a group of tokens' keys is approximated from only the m
most recent kept tokens, correcting for the rotary position embedding.

Readings (that summary is about pruning; here the group is a TempCache slot):
  - keys enter the cache without their temporal rotation, so temporal
    duplicates stay identical and merge exactly; queries arrive rotated at
    their own frame;
  - the temporal rotation turns features (2p, 2p+1), p < d_t/2, by the angle
    frame * base^(-2p/d_t) (the usual rotary form; the rest of the head is
    left alone);
  - a slot with count c whose m' = min(m, c) most recent members came from
    frames t_1..t_m' (most recent first, a frame repeated once per member)
    contributes m' keys R(t_i) k_hat, each with logit shift ln(c / m'): the
    sum of its c members' exponentials approximated by c / m' times that of
    its m' most recent ones, one softmax over every slot's keys, all with the
    slot's value v_hat.
"""

from __future__ import annotations

import math

import numpy as np


def rope_t(x, frame, d_t, base=10000.0):
    """Rows of ``x`` [n][d] (or one row) rotated to ``frame`` on the first
    ``d_t`` features: pair p = (2p, 2p+1) turns by frame * base^(-2p/d_t)."""
    x = np.array(x, dtype=np.float64)
    one = x.ndim == 1
    if one:
        x = x[None, :]
    fr = np.broadcast_to(np.asarray(frame, dtype=np.float64), (x.shape[0],))
    out = x.copy()
    for p in range(d_t // 2):
        ang = fr * base ** (-2.0 * p / d_t)
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[:, 2 * p], x[:, 2 * p + 1]
        out[:, 2 * p] = a * c - b * s
        out[:, 2 * p + 1] = a * s + b * c
    return out[0] if one else out


def recent_frames(head_cache, m):
    """For each live slot of an oracle HeadCache: the frames of its m most
    recent members, most recent first (members are kept in merge order)."""
    return [[f for f, _ in reversed(head_cache.members[s][-m:])]
            for s in range(head_cache.n_live)]


def mdegree_attend(Q, k_hat, v_hat, count, frames, m, d_t, base=10000.0, scale=None):
    """Attention of rotated queries ``Q`` [n][d] over slots with the M-degree
    approximation (see the module docstring).  ``frames``: per slot, its
    member frames most recent first (at least min(m, count) of them).
    float64 throughout; returns ``(O [n][d], lse [n])``."""
    q = np.asarray(Q, dtype=np.float64)
    d = q.shape[1]
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    keys, vals, shift = [], [], []
    for s in range(len(count)):
        c = int(count[s])
        mm = min(m, c)
        for i in range(mm):
            keys.append(rope_t(k_hat[s], frames[s][i], d_t, base))
            vals.append(np.asarray(v_hat[s], dtype=np.float64))
            shift.append(math.log(c / mm))
    if not keys:
        return np.zeros((q.shape[0], d)), np.full(q.shape[0], -np.inf)
    z = (q @ np.array(keys).T) * scale + np.array(shift)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ np.array(vals), zmax[:, 0] + np.log(l[:, 0])
