"""Seeded synthetic workloads for the TempCache attention step.

The pages evaluate on real autoregressive video (FAST-AR, "Principais
Resultados": Rolling-Forcing and LongVie2 rollouts on LongVBench and
LongVGenBench).  None of that data exists here, so these generators stand in
for it.  They model the redundancy the pages build on ("Redundância de Chave
Temporal", FAST-AR section 1): keys of consecutive frames are often exact or
near copies of each other.

Recipe (all draws float32 from numpy's PCG64, then rounded once to the
storage dtype; "N(0, s)" means standard deviation s):

* frame 0: every key iid N(0, 1);
* frame f >= 1: a seeded permutation of the (static) token positions marks
  floor(p_exact * n + 1/2) positions as exact copies of frame f-1's key at the
  same position, floor(p_pert * n + 1/2) as that key plus N(0, sigma_pert)
  noise, and the rest as fresh N(0, 1) keys.  The categories are per token
  position and shared by all heads (a static patch is static in every head);
  the noise is drawn per head;
* values iid N(0, 1) per token, never copied;
* queries = the token's own key + N(0, sigma_query);
* rollout variant: all positions start static; at every frame >= 1,
  ``moving_per_frame`` still-static positions (chosen uniformly) turn moving
  for good, and moving positions get fresh N(0, 1) keys every frame;
* SimHash hyperplanes: iid N(0, 1), rounded once to the key dtype, one set per
  layer shared by all heads.

Seeds: ``numpy.random.SeedSequence(seed).spawn(6)`` gives independent streams
for hyperplanes, keys, categories, noise, values and queries, so changing one
part never shifts another.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

_STREAMS = ("planes", "keys", "categories", "noise", "values", "queries")


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float data once to the storage dtype and return it as float32.

    ``dtype`` is ``"f32"`` (plain float32 copy) or ``"bf16"`` (round to the
    nearest bfloat16, ties to even, through torch's CPU conversion).  The
    returned float32 array holds values that are exactly representable in the
    storage dtype, so either side may convert it losslessly.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x)
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown storage dtype {dtype!r}")


def make_planes(gen: np.random.Generator, tables: int, bits: int, dim: int,
                dtype: str) -> np.ndarray:
    """SimHash hyperplanes [tables][bits][dim], iid N(0, 1), storage-rounded."""
    raw = gen.standard_normal((tables, bits, dim), dtype=np.float32)
    return round_to_storage(raw, dtype)


def make_codebooks(gen: np.random.Generator, tables: int, subspaces: int, bits: int, dim: int,
                   dtype: str) -> np.ndarray:
    """Product-quantization codebooks [tables][subspaces][2^(bits/subspaces)]
    [dim/subspaces], iid N(0, 1) (the distribution of the fresh keys),
    storage-rounded."""
    k = 1 << (bits // subspaces)
    raw = gen.standard_normal((tables, subspaces, k, dim // subspaces), dtype=np.float32)
    return round_to_storage(raw, dtype)


def denoising_steps(gen: np.random.Generator, x: np.ndarray, steps: int, sigma0: float,
                    dtype: str) -> list:
    """The tokens of a chunk at each of ``steps`` denoising steps: ``x`` plus
    sigma_s * N(0, 1) with sigma_s falling linearly from ``sigma0`` at the
    first step to 0 at the last, which returns ``x`` itself (the clean tokens
    that are merged), each storage-rounded."""
    out = []
    for s in range(steps):
        sig = sigma0 * (steps - 1 - s) / (steps - 1) if steps > 1 else 0.0
        if sig == 0.0:
            out.append(np.array(x, dtype=np.float32))
        else:
            out.append(round_to_storage(
                x + np.float32(sig) * gen.standard_normal(x.shape, dtype=np.float32), dtype))
    return out


@dataclass(frozen=True)
class Workload:
    """Shape, drift mix and LSH settings of one synthetic TempCache workload."""

    name: str
    heads: int
    head_dim: int
    tokens_per_frame: int
    frames_per_chunk: int
    dtype: str               # "f32" or "bf16"
    p_exact: float
    p_pert: float
    tables: int
    bits: int
    threshold: float         # merge iff cosine >= threshold
    budget: int              # slots per head
    prefill_frames: int      # frames merged before the measured chunk
    total_frames: int        # frames in the whole sequence
    moving_per_frame: int = 0
    sigma_pert: float = 0.05
    sigma_query: float = 0.1
    seed: int = 0
    subspaces: int = 0       # 0: SimHash; M > 0: product quantization, M slices

    @property
    def chunk_tokens(self) -> int:
        return self.tokens_per_frame * self.frames_per_chunk

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 head, d=64, 64 tokens/frame, 4 cached frames + 1 query frame, fp32.
    "tiny": Workload("tiny", 1, 64, 64, 1, "f32", 0.70, 0.20, 1, 16, 0.98,
                     256, 4, 5, seed=1000),
    # Lemma variant of "tiny": exact copies or fresh keys only (70/0/30).
    "tiny_lemma": Workload("tiny_lemma", 1, 64, 64, 1, "f32", 0.70, 0.0, 1, 16,
                           0.98, 256, 4, 5, seed=1100),
    # One attention layer shaped like a 1.3B video DiT (30x52 patches/frame).
    "dit1.3b": Workload("dit1.3b", 12, 128, 1560, 3, "bf16", 0.60, 0.30, 4, 32,
                        0.95, 8192, 21, 24, seed=1001),
    # 240-frame streaming rollout at the 1.3B layer shape, 2% static->moving.
    "rollout": Workload("rollout", 12, 128, 1560, 3, "bf16", 0.60, 0.30, 4, 32,
                        0.95, 8192, 0, 240, moving_per_frame=31, seed=1002),
    # The 1.3B layer with product-quantization codes: 4 tables, 4 slices of
    # 32 features, 256 centroids each (32-bit codes); same keys as "dit1.3b".
    "dit1.3b_pq": Workload("dit1.3b_pq", 12, 128, 1560, 3, "bf16", 0.60, 0.30, 4, 32,
                           0.95, 8192, 21, 24, seed=1001, subspaces=4),
    # "tiny" with product-quantization codes: 1 table, 2 slices x 16 centroids.
    "tiny_pq": Workload("tiny_pq", 1, 64, 64, 1, "f32", 0.70, 0.20, 1, 8, 0.98,
                        256, 4, 5, seed=1000, subspaces=2),
    # One attention layer shaped like a 14B video DiT (45x80 patches/frame).
    "dit14b": Workload("dit14b", 40, 128, 3600, 3, "bf16", 0.50, 0.35, 4, 32,
                       0.95, 16384, 21, 24, seed=1003),
}


def _half_up(x: float) -> int:
    return int(math.floor(x + 0.5))


class DriftStream:
    """Frame-by-frame generator of keys, values and queries for a Workload.

    ``next_frame()`` returns ``(K, V, Q, category)`` where K, V, Q are float32
    ``[heads][tokens_per_frame][head_dim]`` arrays of storage-exact values and
    ``category`` is ``int8 [tokens_per_frame]`` (0 exact, 1 perturbed,
    2 fresh, 3 moving).
    """

    def __init__(self, w: Workload):
        self.w = w
        seqs = np.random.SeedSequence(w.seed).spawn(len(_STREAMS))
        self.gen = {name: np.random.Generator(np.random.PCG64(s))
                    for name, s in zip(_STREAMS, seqs)}
        self.frame = 0
        self.prev = None
        self.moving = np.zeros(w.tokens_per_frame, dtype=bool)
        if w.subspaces:
            self._planes = make_codebooks(self.gen["planes"], w.tables, w.subspaces, w.bits,
                                          w.head_dim, w.dtype)
        else:
            self._planes = make_planes(self.gen["planes"], w.tables, w.bits,
                                       w.head_dim, w.dtype)

    def planes(self) -> np.ndarray:
        return self._planes.copy()

    def next_frame(self):
        w = self.w
        H, T, d = w.heads, w.tokens_per_frame, w.head_dim
        g = self.gen
        cat = np.empty(T, dtype=np.int8)
        if self.frame == 0:
            K = round_to_storage(g["keys"].standard_normal((H, T, d),
                                                           dtype=np.float32), w.dtype)
            cat[:] = 2
        else:
            if w.moving_per_frame:
                still = np.flatnonzero(~self.moving)
                k = min(w.moving_per_frame, still.size)
                if k:
                    turn = g["categories"].choice(still, size=k, replace=False)
                    self.moving[turn] = True
            static = np.flatnonzero(~self.moving)
            n = static.size
            perm = g["categories"].permutation(static)
            n_ex = _half_up(w.p_exact * n)
            n_pe = min(_half_up(w.p_pert * n), n - n_ex)
            exact = np.sort(perm[:n_ex])
            pert = np.sort(perm[n_ex:n_ex + n_pe])
            fresh = np.sort(perm[n_ex + n_pe:])
            moving = np.flatnonzero(self.moving)
            K = np.empty((H, T, d), dtype=np.float32)
            K[:, exact] = self.prev[:, exact]
            noise = g["noise"].standard_normal((H, pert.size, d), dtype=np.float32)
            K[:, pert] = round_to_storage(self.prev[:, pert] + np.float32(w.sigma_pert) * noise,
                                          w.dtype)
            newk = np.sort(np.concatenate([fresh, moving]))
            K[:, newk] = round_to_storage(
                g["keys"].standard_normal((H, newk.size, d), dtype=np.float32), w.dtype)
            cat[exact] = 0
            cat[pert] = 1
            cat[fresh] = 2
            cat[moving] = 3
        V = round_to_storage(g["values"].standard_normal((H, T, d), dtype=np.float32),
                             w.dtype)
        qn = g["queries"].standard_normal((H, T, d), dtype=np.float32)
        Q = round_to_storage(K + np.float32(w.sigma_query) * qn, w.dtype)
        self.prev = K
        self.frame += 1
        return K, V, Q, cat

    def frames(self, n: int):
        """Generate ``n`` frames and stack them: K, V, Q [heads][n*T][d]."""
        Ks, Vs, Qs = [], [], []
        for _ in range(n):
            K, V, Q, _ = self.next_frame()
            Ks.append(K)
            Vs.append(V)
            Qs.append(Q)
        return (np.concatenate(Ks, axis=1), np.concatenate(Vs, axis=1),
                np.concatenate(Qs, axis=1))


class ClusterPrompt:
    """Prompt keys in Gaussian clusters and latent queries near two of them.

    Stands in for a long text prompt whose tokens fall into a few semantic
    groups, of which each frame uses only some (FAST-AR, "Esparsidade de
    Cross-Attention" and section 2B).  Per head: ``clusters`` centres iid
    N(0, I_d); ``per_cluster`` prompt keys per centre = centre + N(0, spread);
    prompt values iid N(0, 1); per frame, two distinct clusters are drawn and
    every query of that frame is one of the two centres (uniformly) plus
    N(0, query_noise).  Prompt tokens are ordered cluster by cluster.
    """

    def __init__(self, heads=12, head_dim=128, clusters=8, per_cluster=64,
                 frames=3, queries_per_frame=1560, tables=4, bits=16,
                 spread=0.1, query_noise=0.2, dtype="bf16", seed=1004):
        self.heads, self.head_dim = heads, head_dim
        self.clusters, self.per_cluster = clusters, per_cluster
        self.frames, self.queries_per_frame = frames, queries_per_frame
        self.tables, self.bits, self.dtype = tables, bits, dtype
        seqs = np.random.SeedSequence(seed).spawn(len(_STREAMS))
        g = {name: np.random.Generator(np.random.PCG64(s))
             for name, s in zip(_STREAMS, seqs)}
        H, d = heads, head_dim
        self._planes = make_planes(g["planes"], tables, bits, d, dtype)
        centres = g["keys"].standard_normal((H, clusters, d), dtype=np.float32)
        member = np.repeat(np.arange(clusters), per_cluster)
        kp = centres[:, member] + np.float32(spread) * g["noise"].standard_normal(
            (H, member.size, d), dtype=np.float32)
        self.Kp = round_to_storage(kp, dtype)
        self.Vp = round_to_storage(
            g["values"].standard_normal((H, member.size, d), dtype=np.float32), dtype)
        self.frame_clusters = np.stack(
            [np.stack([g["categories"].choice(clusters, size=2, replace=False)
                       for _ in range(frames)]) for _ in range(H)])  # [H][F][2]
        pick = g["categories"].integers(0, 2, size=(H, frames, queries_per_frame))
        cid = np.take_along_axis(self.frame_clusters[:, :, :], pick, axis=2)  # [H][F][q]
        base = np.stack([centres[h][cid[h].reshape(-1)] for h in range(H)])
        q = base + np.float32(query_noise) * g["queries"].standard_normal(
            base.shape, dtype=np.float32)
        self.Q = round_to_storage(q, dtype)  # [H][F*q][d]

    def planes(self) -> np.ndarray:
        return self._planes.copy()

    @property
    def prompt_tokens(self) -> int:
        return self.clusters * self.per_cluster
