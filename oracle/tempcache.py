"""CPU oracle of the FAST-AR TempCache attention step (plain, slow, obvious).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg may.  It shares
no code with the HIP kernels: it takes plain numpy arrays and follows the
method step by step.

What it follows (FAST-AR technical summary, gist.science, Portuguese page and
its French twin, section "2. Componentes Principais / A. TempCache"):

* each token of the current frame is matched top-1 against what is already
  cached, through a lightweight approximate-nearest-neighbour index (LSH)
  instead of full attention matrices ("Mecanismo");
* matched tokens are merged when their similarity passes a threshold; the
  merged slot keeps the mean of the merged values and attention shifts the
  slot's logit by the group size, which Lemma 5.1 shows is exact for
  identical keys ("Base Teórica");
* the cache stays bounded, so memory and latency stay constant ("Benefício").

The pages leave the concrete choices open; the oracle takes these readings
(each one listed, with its reason, in the design notes of the repository):
SimHash random hyperplanes with L tables of b bits, bit = [<r, x> > 0] packed
LSB first; candidates = union over tables of slots with an equal code; top-1
by cosine against the slot's stored (mirror) key, ties to the lowest slot id;
merge iff cosine >= threshold (the threshold as a binary32 number); the merged
key and value are running means in binary32, one rounded op at a time, tokens
in ascending order; a binary32 master plus a storage-dtype mirror; when the
budget is exceeded, least-recently-updated slots are evicted by
(last frame, slot id); inserts take free ids in ascending order; merged slots
are re-hashed from their new mirror key; attention uses scale 1/sqrt(d) and
adds ln(count) to every slot's logit.

Arithmetic: projections, cosines and attention in float64; slot state in
float32 exactly as the method's update specifies.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


class CapacityError(RuntimeError):
    """More inserts than free plus evictable slots (cannot occur if B >= T_f)."""


# ----------------------------------------------------------------------------
# binary32 -> bfloat16, round to nearest, ties to even (from the format
# definition: keep the top 16 bits of the binary32 pattern; the dropped 16 bits
# decide the rounding, a tie goes to the even kept pattern).
# ----------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round binary32 values to bfloat16 (RNE); returned as float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def to_storage(x, dtype: str) -> np.ndarray:
    """The storage-dtype mirror of binary32 data ("f32" or "bf16")."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# SimHash (random-hyperplane LSH; the pages name LSH as TempCache's ANN, FAST-AR
# section 2A "Mecanismo").
# ----------------------------------------------------------------------------

def simhash(x, planes):
    """Codes of rows of ``x`` under hyperplanes ``planes`` [L][b][d].

    Bit j of table t is 1 iff <planes[t][j], x> > 0 (an exact zero gives 0),
    and bit j is stored as ``1 << j``.  Returns ``(codes [n][L] uint32,
    proj [n][L][b] float64)``; ``proj`` lets callers find bits whose sign is
    ambiguous at a given precision.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    P = np.asarray(planes, dtype=np.float64)
    L, b, d = P.shape
    proj = (x64 @ P.reshape(L * b, d).T).reshape(x64.shape[0], L, b)
    codes = np.zeros((x64.shape[0], L), dtype=np.uint64)
    for j in range(b):
        codes |= (proj[:, :, j] > 0.0).astype(np.uint64) << np.uint64(j)
    return codes.astype(np.uint32), proj


def cosine(x64: np.ndarray, k64: np.ndarray) -> float:
    """cos(x, k) in float64; a zero-norm operand gives 0."""
    nx2 = float(x64 @ x64)
    nk2 = float(k64 @ k64)
    if nx2 == 0.0 or nk2 == 0.0:
        return 0.0
    return float(x64 @ k64) / (math.sqrt(nx2) * math.sqrt(nk2))


@dataclass
class FrameResult:
    """Per-token outcome of one frame for one head."""

    codes: np.ndarray          # [T][L] uint32 codes used for matching
    best_slot: np.ndarray      # [T] int64, -1 if no candidate
    best_cos: np.ndarray       # [T] float64, nan if no candidate
    n_candidates: np.ndarray   # [T] int64, distinct candidate slots
    merged: np.ndarray         # [T] bool
    slot: np.ndarray           # [T] int64, slot the token ended up in
    near_tie: np.ndarray       # [T] bool, decision within 1e-6 of a flip
    evicted: list = field(default_factory=list)
    proj: np.ndarray | None = None


class HeadCache:
    """The bounded, merged KV cache of one attention head."""

    def __init__(self, head_dim, budget, tables, bits, threshold, dtype, planes, subspaces=0):
        self.d = int(head_dim)
        self.B = int(budget)
        self.L = int(tables)
        self.b = int(bits)
        self.dtype = dtype
        # The threshold as the library receives it: a binary32 number.
        self.tau = float(np.float32(threshold))
        # subspaces = 0: SimHash hyperplanes [L][b][d]; M > 0: product
        # quantization codebooks [L][M][2^(b/M)][d/M]
        self.M = int(subspaces)
        if self.M:
            self.planes = np.asarray(planes, dtype=np.float64).reshape(
                self.L, self.M, 1 << (self.b // self.M), self.d // self.M)
        else:
            self.planes = np.asarray(planes, dtype=np.float64).reshape(self.L, self.b, self.d)
        B, d = self.B, self.d
        self.K_m = np.zeros((B, d), dtype=np.float32)
        self.V_m = np.zeros((B, d), dtype=np.float32)
        self.k_hat = np.zeros((B, d), dtype=np.float32)
        self.v_hat = np.zeros((B, d), dtype=np.float32)
        self.count = np.zeros(B, dtype=np.int64)
        self.last = np.zeros(B, dtype=np.int64)
        self.codes = np.zeros((B, self.L), dtype=np.uint32)
        self.n_live = 0
        self.evicted_tokens = 0
        self.tokens_seen = 0
        self.frame = 0
        self.members = [[] for _ in range(B)]      # (frame, token) per slot
        self.buckets = [dict() for _ in range(self.L)]

    def hash(self, x):
        """Codes [n][L] of rows of ``x`` under this cache's LSH or quantizer."""
        if self.M:
            from .pq import pq_codes
            return pq_codes(x, self.planes)[0]
        return simhash(x, self.planes)[0]

    # -- index ---------------------------------------------------------------
    def _rebuild_buckets(self):
        self.buckets = [dict() for _ in range(self.L)]
        for s in range(self.n_live):
            for t in range(self.L):
                self.buckets[t].setdefault(int(self.codes[s, t]), []).append(s)

    def candidates(self, code_row) -> list:
        """Live slots sharing a bucket with ``code_row`` in any table."""
        found = set()
        for t in range(self.L):
            found.update(self.buckets[t].get(int(code_row[t]), ()))
        return sorted(found)

    # -- one frame -------------------------------------------------------------
    def process_frame(self, K, V, codes=None) -> FrameResult:
        """Match, merge, evict, insert and re-hash one frame of new tokens.

        ``K``, ``V``: [T][d] storage-exact values.  ``codes``: optional [T][L]
        codes to use instead of hashing ``K`` here.
        """
        K = np.asarray(K, dtype=np.float32)
        V = np.asarray(V, dtype=np.float32)
        T = K.shape[0]
        if T > self.B:
            raise CapacityError(f"{T} tokens in one frame exceed the budget {self.B}")
        proj = None
        if codes is None:
            if self.M:
                codes = self.hash(K)
            else:
                codes, proj = simhash(K, self.planes)
        codes = np.asarray(codes, dtype=np.uint32).reshape(T, self.L)
        f = self.frame

        # 1. match every token against the state left by earlier frames
        best_slot = np.full(T, -1, dtype=np.int64)
        best_cos = np.full(T, np.nan)
        n_cand = np.zeros(T, dtype=np.int64)
        merged = np.zeros(T, dtype=bool)
        near_tie = np.zeros(T, dtype=bool)
        for i in range(T):
            cands = self.candidates(codes[i])
            n_cand[i] = len(cands)
            if not cands:
                continue
            x = K[i].astype(np.float64)
            coss = [cosine(x, self.k_hat[s].astype(np.float64)) for s in cands]
            j = int(np.argmax(coss))        # first maximum = lowest slot id
            best_slot[i] = cands[j]
            best_cos[i] = coss[j]
            merged[i] = coss[j] >= self.tau
            others = sorted(coss, reverse=True)
            if abs(coss[j] - self.tau) < 1e-6 or (len(others) > 1 and others[0] - others[1] < 1e-6):
                near_tie[i] = True

        # 2. merge: per slot, ascending token order, binary32 running mean
        groups = {}
        for i in range(T):
            if merged[i]:
                groups.setdefault(int(best_slot[i]), []).append(i)
        for s in sorted(groups):
            km = self.K_m[s].copy()
            vm = self.V_m[s].copy()
            c = int(self.count[s])
            for i in groups[s]:
                div = np.float32(c + 1)
                km = km + (K[i] - km) / div
                vm = vm + (V[i] - vm) / div
                c += 1
                self.members[s].append((f, i))
            self.K_m[s], self.V_m[s] = km, vm
            self.count[s] = c
            self.last[s] = f
            self.k_hat[s] = to_storage(km, self.dtype)
            self.v_hat[s] = to_storage(vm, self.dtype)

        # 3. evict least-recently-updated slots if the inserts do not fit
        inserts = [i for i in range(T) if not merged[i]]
        m = len(inserts)
        need = max(0, m - (self.B - self.n_live))
        evicted = []
        if need:
            eligible = [s for s in range(self.n_live) if self.last[s] < f]
            eligible.sort(key=lambda s: (int(self.last[s]), s))
            if len(eligible) < need:
                raise CapacityError("not enough evictable slots")
            evicted = sorted(eligible[:need])
            for s in evicted:
                self.evicted_tokens += int(self.count[s])
                self.members[s] = []

        # 4. insert: free ids (evicted first, then never-used) in ascending order
        free_ids = evicted + list(range(self.n_live, self.B))
        slot = np.where(merged, best_slot, -1).astype(np.int64)
        for r, i in enumerate(inserts):
            s = free_ids[r]
            self.K_m[s] = K[i]
            self.V_m[s] = V[i]
            self.k_hat[s] = to_storage(K[i], self.dtype)
            self.v_hat[s] = to_storage(V[i], self.dtype)
            self.count[s] = 1
            self.last[s] = f
            self.codes[s] = codes[i]
            self.members[s] = [(f, i)]
            slot[i] = s
        self.n_live = self.n_live + m - need

        # 5. re-hash merged slots from their new mirror key, rebuild buckets
        if groups:
            ms = np.array(sorted(groups), dtype=np.int64)
            self.codes[ms] = self.hash(self.k_hat[ms])
        self._rebuild_buckets()
        self.tokens_seen += T
        self.frame += 1
        return FrameResult(codes, best_slot, best_cos, n_cand, merged, slot,
                           near_tie, evicted, proj)

    # -- attention over the merged cache ----------------------------------------
    def attend(self, Q, scale=None, return_probs=False):
        """Softmax attention of ``Q`` [n][d] over the live slots.

        Logit of slot s: <q, k_hat[s]> * scale + ln(count[s]) (scale defaults
        to 1/sqrt(d)); output o = sum_s p_s v_hat[s].  float64 throughout.
        Returns ``(O [n][d], lse [n])`` (and the probabilities if asked).
        """
        q = np.asarray(Q, dtype=np.float64)
        if scale is None or scale == 0:
            scale = 1.0 / math.sqrt(self.d)
        S = self.n_live
        if S == 0:
            O = np.zeros((q.shape[0], self.d))
            lse = np.full(q.shape[0], -np.inf)
            return (O, lse, np.zeros((q.shape[0], 0))) if return_probs else (O, lse)
        k = self.k_hat[:S].astype(np.float64)
        v = self.v_hat[:S].astype(np.float64)
        z = (q @ k.T) * scale + np.log(self.count[:S].astype(np.float64))
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        l = e.sum(axis=1, keepdims=True)
        P = e / l
        O = P @ v
        lse = zmax[:, 0] + np.log(l[:, 0])
        return (O, lse, P) if return_probs else (O, lse)


class TempCacheOracle:
    """Independent per-head caches for ``heads`` heads (heads never interact)."""

    def __init__(self, heads, head_dim, budget, tables, bits, threshold, dtype, planes,
                 subspaces=0):
        self.heads = [HeadCache(head_dim, budget, tables, bits, threshold, dtype, planes,
                                subspaces) for _ in range(heads)]

    @classmethod
    def for_workload(cls, w, planes, heads=None):
        return cls(w.heads if heads is None else heads, w.head_dim, w.budget, w.tables,
                   w.bits, w.threshold, w.dtype, planes, getattr(w, "subspaces", 0))

    def process_frame(self, K, V, codes=None):
        """K, V: [H][T][d]; codes: optional [H][T][L].  Returns per-head results."""
        return [hc.process_frame(K[h], V[h], None if codes is None else codes[h])
                for h, hc in enumerate(self.heads)]

    def attend(self, Q, scale=None):
        outs = [hc.attend(Q[h], scale) for h, hc in enumerate(self.heads)]
        return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])

    def state(self) -> dict:
        """Stacked copies of every head's state arrays."""
        hs = self.heads
        return {
            "K_m": np.stack([h.K_m for h in hs]),
            "V_m": np.stack([h.V_m for h in hs]),
            "k_hat": np.stack([h.k_hat for h in hs]),
            "v_hat": np.stack([h.v_hat for h in hs]),
            "count": np.stack([h.count for h in hs]),
            "last": np.stack([h.last for h in hs]),
            "codes": np.stack([h.codes for h in hs]),       # [H][B][L]
            "n_live": np.array([h.n_live for h in hs]),
            "evicted_tokens": np.array([h.evicted_tokens for h in hs]),
            "frame": hs[0].frame if hs else 0,
        }
