"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Tolerances: hash bits identical except where the float64 projection has
|proj| < 1e-4 (counted); match indices, decisions, counts and the binary32
slot state bit-exact given identical codes; attention outputs within max-abs
2e-2 (bf16) or 1e-4 (fp32); Lemma 5.1 within 1e-5 (fp32).
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_attention_tempcache_amd as fa
from oracle import TempCacheOracle, simhash
from oracle import annca as oannca
from synth import WORKLOADS, ClusterPrompt, DriftStream, denoising_steps, round_to_storage
from tests.helpers import (ambiguous_bit_mask, code_ambiguity_mask, compare_codes, compare_state,
                           mirror_to_f32, oracle_codes_for_device, oracle_state_for_import,
                           to_device)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _cache_for(w, planes, rope_members=0):
    cfg = fa.CacheConfig(w.heads, w.head_dim, w.budget, w.tables, w.bits, w.threshold, w.dtype,
                         w.subspaces, rope_members)
    return fa.Cache(cfg, planes)


def _planes_dev(planes, dtype):
    return to_device(planes, dtype).contiguous()


# ------------------------------------------------------------------ hash

@pytest.mark.parametrize("dtype,H,N,d,L,b", [
    ("bf16", 3, 200, 128, 4, 32),
    ("bf16", 2, 97, 64, 4, 16),
    ("bf16", 1, 33, 128, 3, 20),
    ("bf16", 2, 64, 128, 8, 32),
    ("bf16", 8, 16999, 128, 4, 32),   # more 32-row tiles than one pass of the grid
    ("f32", 1, 64, 64, 1, 16),
    ("f32", 2, 50, 128, 4, 32),
])
def test_hash_matches_oracle(dtype, H, N, d, L, b):
    rng = np.random.default_rng(11 + N)
    from synth import round_to_storage
    x = round_to_storage(rng.standard_normal((H, N, d)).astype(np.float32), dtype)
    planes = round_to_storage(rng.standard_normal((L, b, d)).astype(np.float32), dtype)
    codes = fa.hash_codes(to_device(x, dtype), _planes_dev(planes, dtype), L, b)
    torch.cuda.synchronize()
    got = codes.cpu().numpy().view(np.uint32)
    bad = amb = 0
    for h in range(H):
        ref, _ = simhash(x[h], planes)
        mask = ambiguous_bit_mask(x[h], planes)
        nb, na = compare_codes(got[h].T, ref, mask)
        bad += nb
        amb += na
    print(f"hash {dtype} H={H} N={N} d={d} L={L} b={b}: ambiguous differing bits={amb}")
    assert bad == 0


@pytest.mark.parametrize("dtype,H,N,d,L,M,b", [
    ("bf16", 3, 200, 128, 4, 4, 32),
    ("bf16", 2, 97, 64, 2, 2, 8),
    ("bf16", 1, 33, 128, 1, 1, 8),
    ("bf16", 2, 300, 128, 2, 8, 16),      # 4 centroids a slice: padded blocks
    ("bf16", 1, 100, 128, 3, 1, 3),       # 8 centroids
    ("bf16", 8, 4500, 128, 4, 4, 32),     # more 32-row tiles than one pass of the grid
    ("f32", 1, 64, 64, 2, 2, 8),
    ("f32", 2, 50, 128, 1, 4, 16),
])
def test_pq_codes_match_oracle(dtype, H, N, d, L, M, b):
    from oracle.pq import pq_codes
    from synth import make_codebooks, round_to_storage
    rng = np.random.default_rng(300 + N)
    x = round_to_storage(rng.standard_normal((H, N, d)).astype(np.float32), dtype)
    cb = make_codebooks(rng, L, M, b, d, dtype)
    codes = fa.pq_codes(to_device(x, dtype), to_device(cb, dtype).contiguous(), L, M, b)
    torch.cuda.synchronize()
    got = codes.cpu().numpy().view(np.uint32)
    bad = amb = 0
    for h in range(H):
        ref, _ = pq_codes(x[h], cb)
        nb, na = compare_codes(got[h].T, ref, code_ambiguity_mask(x[h], cb, M))
        bad += nb
        amb += na
    print(f"pq {dtype} H={H} N={N} d={d} L={L} M={M} b={b}: ambiguous differing bits={amb}")
    assert bad == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pq_exact_ties_go_to_the_lowest_index(dtype):
    """Rows equal to a centroid that has a duplicate: both score the same, and
    the lower index must win (positive scores: the winner's score is |c|^2/2).
    The pairs put the copy in the same register group, in the other half of
    the wave, and in a later block of 32 centroids."""
    from synth import make_codebooks
    M, b, d = 4, 32, 128
    w = d // M
    rng = np.random.default_rng(77)
    cb = make_codebooks(rng, 1, M, b, d, dtype)
    pairs = [(1, 2), (4, 9), (6, 37), (8, 255), (12, 13), (33, 100), (40, 44), (0, 31)]
    for a, c in pairs:
        cb[0, :, c] = cb[0, :, a]
    n = 3 * len(pairs)
    x = np.zeros((1, n, d), dtype=np.float32)
    want = np.zeros(n, dtype=np.uint64)
    for i in range(n):
        for m in range(M):
            a = pairs[(i + m) % len(pairs)][0]
            x[0, i, m * w:(m + 1) * w] = cb[0, m, a]
            want[i] |= np.uint64(a) << np.uint64(m * (b // M))
    codes = fa.pq_codes(to_device(x, dtype), to_device(cb, dtype).contiguous(), 1, M, b)
    torch.cuda.synchronize()
    got = codes.cpu().numpy().view(np.uint32)[0, 0]
    from oracle.pq import pq_codes
    ref, _ = pq_codes(x[0], cb)
    assert np.array_equal(ref[:, 0], want.astype(np.uint32))
    assert np.array_equal(got, want.astype(np.uint32))


def test_hash_zero_bits_gives_zero_codes():
    x = torch.randn(2, 40, 128, device="cuda").to(torch.bfloat16)
    planes = torch.zeros(0, dtype=torch.bfloat16, device="cuda")
    codes = fa.hash_codes(x, planes, 3, 0)
    torch.cuda.synchronize()
    assert (codes == 0).all()


# ------------------------------------------------------------------ match / merge

def _run_frames(w, frames, check_every=True, use_gpu_hash=False, rope_members=0):
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    cache = _cache_for(w, planes, rope_members)
    H, T = w.heads, w.tokens_per_frame
    amb_total = 0
    last_q = None
    for f in range(frames):
        K, V, Q, _ = st.next_frame()
        res = orc.process_frame(K, V)
        near = sum(int(r.near_tie.sum()) for r in res)
        assert near == 0, f"frame {f}: {near} near-ties"
        codes = None if use_gpu_hash else oracle_codes_for_device([r.codes for r in res])
        slot_out = torch.full((H, T), -7, dtype=torch.int32, device="cuda")
        merged_out = torch.full((H, T), 7, dtype=torch.uint8, device="cuda")
        cache.match_merge(to_device(K, w.dtype), to_device(V, w.dtype), T, 1, codes=codes,
                          slot_out=slot_out, merged_out=merged_out)
        torch.cuda.synchronize()
        so = slot_out.cpu().numpy()
        mo = merged_out.cpu().numpy()
        for h in range(H):
            np.testing.assert_array_equal(mo[h].astype(bool), res[h].merged, err_msg=f"frame {f} head {h}")
            np.testing.assert_array_equal(so[h], res[h].slot, err_msg=f"frame {f} head {h}")
        if check_every or f == frames - 1:
            gst = cache.export_state()
            compare_state(gst, orc, w.dtype)
            # slot codes: identical except ambiguous bits; re-sync those
            ost = orc.state()
            resync = False
            for h in range(H):
                n = int(ost["n_live"][h])
                mask = code_ambiguity_mask(ost["k_hat"][h, :n], planes, w.subspaces)
                nb, na = compare_codes(gst["codes"][h][:, :n].T, ost["codes"][h, :n], mask)
                assert nb == 0, f"frame {f} head {h}: {nb} non-ambiguous code bits differ"
                amb_total += na
                resync |= na > 0
            if resync:
                cache.import_state({"codes": np.ascontiguousarray(ost["codes"].transpose(0, 2, 1)),
                                    "frame": ost["frame"]})
        last_q = Q
    return orc, cache, amb_total, last_q


@pytest.mark.parametrize("name,overrides,frames", [
    ("tiny", {}, 5),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048), 6),
    ("dit1.3b", dict(heads=3, tokens_per_frame=129, budget=180, seed=77), 8),   # eviction
    ("dit14b", dict(heads=2, tokens_per_frame=250, budget=300, head_dim=64, seed=78), 7),  # eviction
    # 20-bit codes of 3 tables: table 1 straddles two 32-bit words of sign bits
    ("dit1.3b", dict(heads=2, tokens_per_frame=200, budget=1024, tables=3, bits=20, seed=79), 5),
    # 8 tables of 16 bits: the 8-table match path and longer candidate lists
    ("dit1.3b", dict(heads=2, tokens_per_frame=150, budget=600, tables=8, bits=16, seed=80), 5),
    # a frame as large as a budget that is not a multiple of 32 (eviction every frame)
    ("dit1.3b", dict(heads=1, tokens_per_frame=100, budget=100, seed=81), 4),
    # product-quantization codes: fp32 (float64 distances) and bf16 (MFMA scores)
    ("tiny_pq", {}, 5),
    ("dit1.3b_pq", dict(heads=2, tokens_per_frame=300, budget=2048), 5),
    ("dit1.3b_pq", dict(heads=2, tokens_per_frame=200, budget=260, subspaces=8, bits=16,
                        seed=82), 5),                            # 4 centroids a slice, eviction
    # one token per frame into one slot: it merges every frame, or (no
    # repeated keys) evicts the slot every frame
    ("dit1.3b", dict(heads=2, tokens_per_frame=1, budget=1, seed=83), 6),
    ("dit1.3b", dict(heads=2, tokens_per_frame=1, budget=1, p_exact=0.4, p_pert=0.0, seed=83), 10),
    # zero-bit codes: every live slot is in the one bucket, merges and evictions
    ("dit1.3b", dict(heads=2, tokens_per_frame=64, budget=200, bits=0, tables=1, p_exact=0.3,
                     p_pert=0.2, seed=85), 8),
])
def test_match_merge_matches_oracle_given_codes(name, overrides, frames):
    w = WORKLOADS[name].with_(**overrides)
    print(f"match_merge parity: {w.name} {overrides} frames={frames}", flush=True)
    orc, cache, amb, _ = _run_frames(w, frames)
    ev = sum(h.evicted_tokens for h in orc.heads)
    print(f"  ambiguous slot-code bits re-synced: {amb}; evicted tokens: {ev}")


def test_eviction_really_happens_in_the_small_budget_case():
    w = WORKLOADS["dit1.3b"].with_(heads=3, tokens_per_frame=129, budget=180, seed=77)
    orc, cache, _, _ = _run_frames(w, 8, check_every=False)
    assert cache.stats()["evicted_slots"] > 0
    assert sum(h.evicted_tokens for h in orc.heads) > 0


def test_maximum_budget_and_frame_size_with_eviction():
    """The declared maxima: 8192 tokens per frame into 32768 slots per head.
    Half of each frame is fresh, so the budget fills at frame 6 and frames
    6-8 evict; the state after frame 8 is bit-exact and the attention of all
    8192 queries over the 32768 slots matches on 512 sampled queries."""
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=8192, budget=32768, p_exact=0.3,
                                   p_pert=0.2, seed=2024)
    print(f"maximum sizes: T={w.tokens_per_frame} B={w.budget} H={w.heads}", flush=True)
    orc, cache, _, Q = _run_frames(w, 9, check_every=False)
    stats = cache.stats()
    assert stats["evicted_slots"] > 0
    for h in range(w.heads):
        assert orc.heads[h].n_live == w.budget
        assert orc.heads[h].evicted_tokens > 0
    out = cache.attend(to_device(Q, w.dtype))
    torch.cuda.synchronize()
    rows = np.arange(0, w.tokens_per_frame, 16)
    O_ref, _ = orc.attend(Q[:, rows])
    err = np.abs(out.float().cpu().numpy()[:, rows] - O_ref).max()
    print(f"  evicted slots {stats['evicted_slots']}; attend max-abs on {len(rows)} queries {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["dit1.3b", "dit1.3b_pq"])
def test_gpu_hashing_end_to_end_matches_oracle(name):
    """Library hashes the keys itself (bf16 MFMA); decisions still match the oracle."""
    w = WORKLOADS[name].with_(heads=2, tokens_per_frame=256, budget=1024, seed=91)
    _run_frames(w, 5, check_every=False, use_gpu_hash=True)


def test_frame_split_invariance():
    """One call with 3 frames == three calls with one frame each (bit-identical state)."""
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=200, budget=900, seed=5)
    st = DriftStream(w)
    planes = st.planes()
    K, V, _ = st.frames(6)
    a, b = _cache_for(w, planes), _cache_for(w, planes)
    T = w.tokens_per_frame
    kd, vd = to_device(K, w.dtype), to_device(V, w.dtype)
    a.match_merge(kd[:, :3 * T], vd[:, :3 * T], T, 3)
    a.match_merge(kd[:, 3 * T:], vd[:, 3 * T:], T, 3)
    for f in range(6):
        b.match_merge(kd[:, f * T:(f + 1) * T], vd[:, f * T:(f + 1) * T], T, 1)
    torch.cuda.synchronize()
    sa, sb = a.export_state(), b.export_state()
    for key in ("k_master", "v_master", "k_mirror", "v_mirror", "count", "last", "codes",
                "n_live", "evicted_tokens"):
        np.testing.assert_array_equal(sa[key], sb[key], err_msg=key)
    assert sa["frame"] == sb["frame"] == 6


def test_determinism_two_runs():
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=300, budget=700, seed=6)
    outs = []
    for _ in range(2):
        st = DriftStream(w)
        planes = st.planes()
        K, V, _ = st.frames(5)
        c = _cache_for(w, planes)
        c.match_merge(to_device(K, w.dtype), to_device(V, w.dtype), w.tokens_per_frame, 5)
        torch.cuda.synchronize()
        outs.append(c.export_state())
    for key in outs[0]:
        np.testing.assert_array_equal(np.asarray(outs[0][key]), np.asarray(outs[1][key]), err_msg=key)


def test_conservation_on_device():
    w = WORKLOADS["dit1.3b"].with_(heads=3, tokens_per_frame=129, budget=170, seed=8)
    st = DriftStream(w)
    planes = st.planes()
    K, V, _ = st.frames(9)
    c = _cache_for(w, planes)
    c.match_merge(to_device(K, w.dtype), to_device(V, w.dtype), w.tokens_per_frame, 9)
    torch.cuda.synchronize()
    s = c.export_state()
    stats = c.stats()
    for h in range(w.heads):
        n = int(s["n_live"][h])
        assert n <= w.budget
        assert (s["count"][h, :n] >= 1).all()
        assert int(s["count"][h, :n].sum()) + int(s["evicted_tokens"][h]) == 9 * w.tokens_per_frame
    assert stats["tokens_seen"] == 9 * w.tokens_per_frame * w.heads
    assert stats["merged_tokens"] + stats["inserted_tokens"] == stats["tokens_seen"]


# ------------------------------------------------------------------ attend

@pytest.mark.parametrize("name,overrides,frames", [
    ("tiny", {}, 5),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048), 6),
    ("dit1.3b", dict(heads=3, tokens_per_frame=131, budget=1024, head_dim=64, seed=3), 4),
    ("dit14b", dict(heads=2, tokens_per_frame=333, budget=4096, seed=4), 5),
    # one frame into an empty cache: 1..5 key tiles of 64, so every position
    # of the 4-buffer ring is the last tile once
    ("dit1.3b", dict(heads=2, tokens_per_frame=40, budget=1024, seed=40), 1),
    ("dit1.3b", dict(heads=2, tokens_per_frame=100, budget=1024, seed=41), 1),
    ("dit1.3b", dict(heads=2, tokens_per_frame=150, budget=1024, seed=42), 1),
    ("dit1.3b", dict(heads=2, tokens_per_frame=250, budget=1024, seed=43), 1),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=1024, seed=44), 1),
    # one query over one live slot (one token per frame, always merged)
    ("dit1.3b", dict(heads=2, tokens_per_frame=1, budget=5, seed=84), 12),
])
def test_attend_matches_oracle(name, overrides, frames):
    w = WORKLOADS[name].with_(**overrides)
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    Q = None
    for _ in range(frames):
        K, V, Q, _ = st.next_frame()
        orc.process_frame(K, V)
    cache = _cache_for(w, planes)
    cache.import_state(oracle_state_for_import(orc, w.dtype))
    lse = torch.empty((w.heads, Q.shape[1]), dtype=torch.float32, device="cuda")
    out = cache.attend(to_device(Q, w.dtype), lse=lse)
    torch.cuda.synchronize()
    O_ref, lse_ref = orc.attend(Q)
    got = out.float().cpu().numpy()
    err = np.abs(got - O_ref).max()
    lerr = np.abs(lse.cpu().numpy() - lse_ref).max()
    print(f"attend {w.name} {overrides}: n_live={[h.n_live for h in orc.heads]} max-abs={err:.3e} lse={lerr:.3e}")
    assert err <= TOL[w.dtype]
    assert lerr <= (1e-3 if w.dtype == "bf16" else 1e-5) * max(1.0, np.abs(lse_ref).max())


def test_attend_values_one_give_one():
    """Softmax rows sum to one: with every stored value 1 the output is 1."""
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=300, budget=2048, seed=12)
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    for _ in range(4):
        K, V, Q, _ = st.next_frame()
        orc.process_frame(K, V)
    s = oracle_state_for_import(orc, w.dtype)
    s["v_mirror"] = np.full_like(s["v_mirror"], 0x3F80)  # bf16 1.0
    cache = _cache_for(w, planes)
    cache.import_state(s)
    out = cache.attend(to_device(Q, w.dtype))
    torch.cuda.synchronize()
    assert np.abs(out.float().cpu().numpy() - 1.0).max() <= 1e-2


def test_attend_empty_cache_gives_zeros():
    w = WORKLOADS["dit1.3b"].with_(heads=2, budget=256)
    cache = _cache_for(w, DriftStream(w).planes())
    q = torch.randn(2, 70, 128, device="cuda").to(torch.bfloat16)
    lse = torch.zeros(2, 70, device="cuda")
    out = cache.attend(q, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isinf(lse).all()


# ------------------------------------------------------------------ K projection + hash

from oracle import project as oproject  # noqa: E402


@pytest.mark.parametrize("H,d,N,Din,L,b", [
    (2, 128, 300, 256, 4, 32),
    (3, 128, 129, 1536, 4, 32),      # a ragged tile of one token
    (2, 64, 200, 512, 2, 20),        # d = 64, 20-bit codes straddling words
    (12, 128, 1000, 1536, 4, 32),    # the 1.3B layer's head count and width
    (12, 128, 4680, 1536, 4, 32),    # the 1.3B layer's whole chunk (bench.py --workload project)
    (1, 128, 1, 64, 8, 32),          # one token, 8 tables (all 256 planes)
    (2, 128, 700, 96, 3, 16),        # 3 stages: one pass of the copy ring
    (2, 128, 64, 160, 1, 7),         # 5 stages, 7-bit codes
])
def test_project_keys_matches_oracle(H, d, N, Din, L, b):
    print(f"project_keys: H={H} d={d} N={N} Din={Din} L={L} b={b}", flush=True)
    rng = np.random.default_rng(700 + N)
    X = round_to_storage(rng.standard_normal((N, Din), dtype=np.float32), "bf16")
    W = round_to_storage((rng.standard_normal((H * d, Din)) / math.sqrt(Din)).astype(np.float32),
                         "bf16")
    planes = round_to_storage(rng.standard_normal((L, b, d), dtype=np.float32), "bf16")
    cfg = fa.CacheConfig(H, d, 2 * N + 64, L, b, 0.95, "bf16")
    cache = fa.Cache(cfg, planes)
    k, codes = cache.project_keys(to_device(X, "bf16"), to_device(W, "bf16"))
    torch.cuda.synchronize()
    K_ref, c_ref, proj = oproject.project_keys(X, W, H, planes)
    got = k.float().cpu().numpy().astype(np.float64)
    # The stored keys: the bf16 rounding of the product.  fp32 accumulation of
    # Din products errs by at most Din * 2^-24 * sum |x_i w_i| (recursive
    # summation bound), and rounding either sum to bf16 adds at most one unit
    # in the last place; keys near zero are where the first term dominates.
    ulp = np.ldexp(1.0, np.frexp(np.abs(K_ref))[1] - 8)
    acc_err = Din * 2.0 ** -24 * (np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)
    tol = ulp + acc_err.reshape(N, H, d).transpose(1, 0, 2)
    diff = np.abs(got - K_ref)
    assert (diff <= tol).all()
    exact = float((diff == 0).mean())
    assert exact > 0.99
    # codes: a bit may differ only where that change of every key element
    # could move its projection across zero (or |projection| < 1e-4)
    P = planes.astype(np.float64).reshape(L * b, d)
    bound = (tol @ np.abs(P).T).reshape(H, N, L, b) + 1e-4
    amb = np.abs(proj) < bound
    gc = codes.cpu().numpy().view(np.uint32)           # [H][L][N]
    bad = differ = 0
    for j in range(b):
        gbit = (gc.transpose(0, 2, 1) >> j) & 1         # [H][N][L]
        rbit = (c_ref >> j) & 1
        bad += int(((gbit != rbit) & ~amb[..., j]).sum())
        differ += int((gbit != rbit).sum())
    print(f"  exact keys {exact:.5f}, ambiguous bits {int(amb.sum())}, differing bits {differ}")
    assert bad == 0
    # the bound is a worst case; in fact almost every bit agrees
    assert differ <= 1e-3 * amb.size


def test_project_keys_feeds_match_merge():
    """Codes from the fused projection drive the merge like the library's own
    hashing of the same keys, up to ambiguous bits: identical decisions."""
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=256, budget=1024, seed=92)
    st = DriftStream(w)
    planes = st.planes()
    rng = np.random.default_rng(93)
    Din = 256
    W = round_to_storage((rng.standard_normal((w.heads * w.head_dim, Din)) / 16).astype(np.float32),
                         "bf16")
    wd = to_device(W, "bf16")
    a, b_ = _cache_for(w, planes), _cache_for(w, planes)
    for f in range(4):
        X = round_to_storage(rng.standard_normal((w.tokens_per_frame, Din), dtype=np.float32), "bf16")
        if f:
            X[:150] = Xprev[:150]                        # repeated tokens: identical keys, merges
        Xprev = X
        k, codes = a.project_keys(to_device(X, "bf16"), wd)
        v = torch.randn_like(k)
        a.match_merge(k, v, w.tokens_per_frame, 1, codes=codes)
        b_.match_merge(k, v, w.tokens_per_frame, 1)
        torch.cuda.synchronize()
    sa, sb = a.export_state(), b_.export_state()
    for key in ("count", "n_live", "k_master", "v_master"):
        np.testing.assert_array_equal(sa[key], sb[key], err_msg=key)
    assert int(sa["count"].max()) >= 4


# ------------------------------------------------------------------ denoising loop

from oracle import denoise as odenoise  # noqa: E402


@pytest.mark.parametrize("name,overrides,frames,n_new", [
    ("tiny", {}, 4, 0),
    ("tiny", {}, 4, 1),
    ("tiny", {}, 4, 65),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048), 5, 1),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048), 5, 64),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048), 5, 333),
    ("dit1.3b", dict(heads=3, tokens_per_frame=131, budget=1024, head_dim=64, seed=3), 3, 200),
    ("dit1.3b", dict(heads=2, tokens_per_frame=250, budget=1024, seed=43), 1, 0),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=1024, seed=44), 0, 700),  # no slots
])
def test_attend_with_chunk_matches_oracle(name, overrides, frames, n_new):
    w = WORKLOADS[name].with_(**overrides)
    print(f"attend_with_chunk: {w.name} {overrides} frames={frames} n_new={n_new}", flush=True)
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    for _ in range(frames):
        K, V, _, _ = st.next_frame()
        orc.process_frame(K, V)
    H, d = w.heads, w.head_dim
    rng = np.random.default_rng(500 + n_new)
    Q = round_to_storage(rng.standard_normal((H, 257, d), dtype=np.float32), w.dtype)
    # the chunk as a strided view: rows 3 .. 3+n_new of a longer buffer
    buf_k = round_to_storage(rng.standard_normal((H, n_new + 5, d), dtype=np.float32), w.dtype)
    buf_v = round_to_storage(rng.standard_normal((H, n_new + 5, d), dtype=np.float32), w.dtype)
    cache = _cache_for(w, planes)
    if frames:
        cache.import_state(oracle_state_for_import(orc, w.dtype))
    kd, vd = to_device(buf_k, w.dtype), to_device(buf_v, w.dtype)
    lse = torch.empty((H, Q.shape[1]), dtype=torch.float32, device="cuda")
    out = cache.attend_with_chunk(to_device(Q, w.dtype), kd[:, 3:3 + n_new], vd[:, 3:3 + n_new],
                                  lse=lse)
    torch.cuda.synchronize()
    got, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    for h, hc in enumerate(orc.heads):
        n = hc.n_live
        O_ref, lse_ref = odenoise.attend_with_chunk(Q[h], hc.k_hat[:n], hc.v_hat[:n], hc.count[:n],
                                                    buf_k[h, 3:3 + n_new], buf_v[h, 3:3 + n_new])
        err = np.abs(got[h] - O_ref).max()
        lerr = np.abs(gl[h] - lse_ref).max()
        print(f"  head {h}: slots={n} max-abs={err:.3e} lse={lerr:.3e}")
        assert err <= TOL[w.dtype]
        assert lerr <= (1e-3 if w.dtype == "bf16" else 1e-5) * max(1.0, np.abs(lse_ref).max())


def test_attend_with_chunk_without_tokens_is_attend():
    """n_new = 0 runs the plain step: bit-identical outputs."""
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=300, budget=2048, seed=45)
    st = DriftStream(w)
    planes = st.planes()
    cache = _cache_for(w, planes)
    K, V, Q = st.frames(3)
    cache.match_merge(to_device(K, w.dtype), to_device(V, w.dtype), w.tokens_per_frame, 3)
    q = to_device(Q, w.dtype)
    empty = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    a = cache.attend(q)
    b = cache.attend_with_chunk(q, empty, empty)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,overrides", [
    ("tiny", {}),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048, seed=46)),
    ("dit1.3b", dict(heads=2, tokens_per_frame=200, budget=450, seed=47)),  # eviction at the merge
])
def test_denoising_loop_matches_oracle(name, overrides):
    """Three denoising steps over the cache plus the noisy chunk, then the
    clean chunk merged frame by frame: every step's output, the merge
    decisions and the cache state against the oracle."""
    w = WORKLOADS[name].with_(**overrides)
    print(f"denoising loop: {w.name} {overrides}", flush=True)
    prefill, F, S = 3, 2, 3
    orc, cache, _, _ = _run_frames(w, prefill, check_every=False)
    st = DriftStream(w)
    planes = st.planes()
    for _ in range(prefill):
        st.next_frame()
    Kc, Vc, Qc = st.frames(F)
    rng = np.random.default_rng(900)
    Ks = denoising_steps(rng, Kc, S, 0.5, w.dtype)
    Vs = denoising_steps(rng, Vc, S, 0.5, w.dtype)
    Qs = denoising_steps(rng, Qc, S, 0.5, w.dtype)
    outs = [cache.attend_with_chunk(to_device(Qs[s], w.dtype), to_device(Ks[s], w.dtype),
                                    to_device(Vs[s], w.dtype)) for s in range(S)]
    ref_outs, _, res = odenoise.denoise_chunk(orc, Qs, Ks, Vs, frames=F)
    torch.cuda.synchronize()
    for s in range(S):
        err = np.abs(outs[s].float().cpu().numpy() - ref_outs[s]).max()
        print(f"  step {s}: max-abs={err:.3e}")
        assert err <= TOL[w.dtype]
    T, H = w.tokens_per_frame, w.heads
    for f in range(F):
        for r in res[f]:
            assert int(r.near_tie.sum()) == 0
        codes = oracle_codes_for_device([r.codes for r in res[f]])
        slot_out = torch.full((H, T), -7, dtype=torch.int32, device="cuda")
        merged_out = torch.full((H, T), 7, dtype=torch.uint8, device="cuda")
        cache.match_merge(to_device(Kc[:, f * T:(f + 1) * T], w.dtype),
                          to_device(Vc[:, f * T:(f + 1) * T], w.dtype), T, 1, codes=codes,
                          slot_out=slot_out, merged_out=merged_out)
        torch.cuda.synchronize()
        so, mo = slot_out.cpu().numpy(), merged_out.cpu().numpy()
        for h in range(H):
            np.testing.assert_array_equal(mo[h].astype(bool), res[f][h].merged)
            np.testing.assert_array_equal(so[h], res[f][h].slot)
    compare_state(cache.export_state(), orc, w.dtype)


# ------------------------------------------------------------------ rotation-corrected M-degree

from oracle import rope as orope  # noqa: E402


@pytest.mark.parametrize("name,overrides,frames,R", [
    ("tiny", {}, 6, 2),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048, seed=94), 6, 4),
    ("dit1.3b", dict(heads=3, tokens_per_frame=129, budget=180, seed=77), 8, 3),   # eviction
])
def test_member_frames_match_oracle(name, overrides, frames, R):
    w = WORKLOADS[name].with_(**overrides)
    print(f"member frames: {w.name} {overrides} R={R}", flush=True)
    orc, cache, _, _ = _run_frames(w, frames, check_every=False, rope_members=R)
    g = cache.export_state()
    for h, hc in enumerate(orc.heads):
        fr = orope.recent_frames(hc, R)
        for s in range(hc.n_live):
            k = min(R, int(hc.count[s]))
            assert list(g["member_frames"][h, s, :k]) == fr[s][:k], (h, s)


def _rope_state(orc, w, R):
    st = oracle_state_for_import(orc, w.dtype)
    mf = np.zeros((w.heads, w.budget, R), np.int32)
    for h, hc in enumerate(orc.heads):
        for s, fs in enumerate(orope.recent_frames(hc, R)):
            mf[h, s, :len(fs)] = fs
    st["member_frames"] = mf
    return st


@pytest.mark.parametrize("name,overrides,frames,m,d_t", [
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048, seed=95), 6, 1, 32),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048, seed=95), 6, 2, 32),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048, seed=95), 6, 4, 32),
    ("dit1.3b", dict(heads=2, tokens_per_frame=300, budget=2048, seed=95), 6, 3, 128),
    ("dit1.3b", dict(heads=3, tokens_per_frame=131, budget=1024, head_dim=64, seed=3), 5, 4, 16),
    ("dit1.3b", dict(heads=3, tokens_per_frame=129, budget=180, seed=77), 8, 2, 32),  # eviction
    ("dit1.3b", dict(heads=2, tokens_per_frame=40, budget=1024, seed=40), 1, 4, 32),  # one tile
])
def test_attend_rope_matches_oracle(name, overrides, frames, m, d_t):
    w = WORKLOADS[name].with_(**overrides)
    print(f"attend_rope: {w.name} {overrides} frames={frames} m={m} d_t={d_t}", flush=True)
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    for _ in range(frames):
        K, V, _, _ = st.next_frame()
        orc.process_frame(K, V)
    R = 4
    cache = _cache_for(w, planes, R)
    cache.import_state(_rope_state(orc, w, R))
    rng = np.random.default_rng(600 + m)
    Qh = rng.standard_normal((w.heads, 200, w.head_dim))
    Q = round_to_storage(np.stack([orope.rope_t(Qh[h], frames, d_t) for h in range(w.heads)])
                         .astype(np.float32), w.dtype)
    lse = torch.empty((w.heads, Q.shape[1]), dtype=torch.float32, device="cuda")
    out = cache.attend_rope(to_device(Q, w.dtype), m, d_t, lse=lse)
    torch.cuda.synchronize()
    got, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    for h, hc in enumerate(orc.heads):
        n = hc.n_live
        O_ref, lse_ref = orope.mdegree_attend(Q[h], hc.k_hat[:n], hc.v_hat[:n], hc.count[:n],
                                              orope.recent_frames(hc, m), m, d_t)
        err = np.abs(got[h] - O_ref).max()
        lerr = np.abs(gl[h] - lse_ref).max()
        print(f"  head {h}: slots={n} max-abs={err:.3e} lse={lerr:.3e}")
        assert err <= TOL[w.dtype]
        assert lerr <= 1e-3 * max(1.0, np.abs(lse_ref).max())


def test_attend_rope_without_rotation_is_the_cache_step():
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=300, budget=2048, seed=96)
    orc, cache, _, Q = _run_frames(w, 5, check_every=False, rope_members=4)
    q = to_device(Q, w.dtype)
    a = cache.attend(q)
    for m in (1, 4):
        b = cache.attend_rope(q, m, 0)
        torch.cuda.synchronize()
        assert (a.float() - b.float()).abs().max().item() <= 1e-2


def test_attend_rope_empty_cache_gives_zeros():
    w = WORKLOADS["dit1.3b"].with_(heads=2, budget=256)
    cache = _cache_for(w, DriftStream(w).planes(), 2)
    q = torch.randn(2, 70, 128, device="cuda").to(torch.bfloat16)
    lse = torch.zeros(2, 70, device="cuda")
    out = cache.attend_rope(q, 2, 32, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isinf(lse).all()


def test_lemma51_on_gpu_fp32():
    """Full GPU path (hash, match, merge, attend) on exact duplicates = dense attention."""
    w = WORKLOADS["tiny_lemma"]
    st = DriftStream(w)
    planes = st.planes()
    cache = _cache_for(w, planes)
    ks, vs = [], []
    Q = None
    for _ in range(5):
        K, V, Q, _ = st.next_frame()
        cache.match_merge(to_device(K, "f32"), to_device(V, "f32"), w.tokens_per_frame, 1)
        ks.append(K)
        vs.append(V)
    out = cache.attend(to_device(Q, "f32"))
    torch.cuda.synchronize()
    Kr = np.concatenate(ks, axis=1)[0].astype(np.float64)
    Vr = np.concatenate(vs, axis=1)[0].astype(np.float64)
    q = Q[0].astype(np.float64)
    z = q @ Kr.T / math.sqrt(w.head_dim)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    dense = (p / p.sum(axis=1, keepdims=True)) @ Vr
    stats = cache.stats()
    assert stats["live_slots"] < Kr.shape[0]
    err = np.abs(out.cpu().numpy()[0] - dense).max()
    print(f"Lemma 5.1 on GPU: slots={stats['live_slots']} raw={Kr.shape[0]} max-abs={err:.2e}")
    assert err < 1e-5


# ------------------------------------------------------------------ AnnCA

@pytest.mark.parametrize("bits", [16, 20])  # 16: LDS bitmaps; 20: the hash-set path
def test_annca_select_and_sparse_attend_match_oracle(bits):
    cp = ClusterPrompt(heads=2, queries_per_frame=300, frames=3, bits=bits)
    H, F, Nf, Np = 2, 3, 300, cp.prompt_tokens
    planes = cp.planes()
    q_dev = to_device(cp.Q, "bf16")
    kp_dev, vp_dev = to_device(cp.Kp, "bf16"), to_device(cp.Vp, "bf16")
    pl_dev = _planes_dev(planes, "bf16")
    qc = fa.hash_codes(q_dev, pl_dev, cp.tables, cp.bits)
    pc = fa.hash_codes(kp_dev, pl_dev, cp.tables, cp.bits)
    torch.cuda.synchronize()
    # device codes vs oracle codes (ambiguity-tolerant)
    for h in range(H):
        for x, got in ((cp.Q[h], qc[h]), (cp.Kp[h], pc[h])):
            ref, _ = simhash(x, planes)
            nb, _ = compare_codes(got.cpu().numpy().view(np.uint32).T, ref,
                                  ambiguous_bit_mask(x, planes))
            assert nb == 0
    # selection given identical (oracle) codes: exact
    oq = [simhash(cp.Q[h], planes)[0] for h in range(H)]
    op = [simhash(cp.Kp[h], planes)[0] for h in range(H)]
    sel, cnt = fa.annca_select(oracle_codes_for_device(oq), oracle_codes_for_device(op), F)
    out = fa.attend_subset(q_dev, kp_dev, vp_dev, F, sel, cnt)
    dense = fa.attend_subset(q_dev, kp_dev, vp_dev, F)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    got = out.float().cpu().numpy()
    got_dense = dense.float().cpu().numpy()
    for h in range(H):
        for g in range(F):
            rows = slice(g * Nf, (g + 1) * Nf)
            r = oannca.annca_frame(cp.Q[h, rows], cp.Kp[h], cp.Vp[h], planes,
                                   codes_q=oq[h][rows], codes_p=op[h])
            n = int(cnt_h[h, g])
            assert n == r["sel"].size
            np.testing.assert_array_equal(sel_h[h, g, :n], r["sel"])
            assert np.abs(got[h, rows] - r["o_sparse"]).max() <= 2e-2
            assert np.abs(got_dense[h, rows] - r["o_dense"]).max() <= 2e-2
    print(f"AnnCA kept per frame: {cnt_h.tolist()} of {Np}")


def test_annca_with_pq_codes_matches_oracle():
    """AnnCA with product-quantization buckets (4 tables x 4 slices x 16
    centroids): GPU codes against the oracle's, then selection and sparse
    attention given the oracle's codes."""
    from oracle.pq import pq_codes
    from synth import make_codebooks
    cp = ClusterPrompt(heads=2, queries_per_frame=300, frames=3, bits=16)
    H, F, Nf, L, M, b = 2, 3, 300, cp.tables, 4, 16
    cb = make_codebooks(np.random.default_rng(1234), L, M, b, cp.head_dim, "bf16")
    cb_dev = to_device(cb, "bf16").contiguous()
    q_dev = to_device(cp.Q, "bf16")
    kp_dev, vp_dev = to_device(cp.Kp, "bf16"), to_device(cp.Vp, "bf16")
    qc = fa.pq_codes(q_dev, cb_dev, L, M, b)
    pc = fa.pq_codes(kp_dev, cb_dev, L, M, b)
    torch.cuda.synchronize()
    oq = [pq_codes(cp.Q[h], cb)[0] for h in range(H)]
    op = [pq_codes(cp.Kp[h], cb)[0] for h in range(H)]
    for h in range(H):
        for x, got, ref in ((cp.Q[h], qc[h], oq[h]), (cp.Kp[h], pc[h], op[h])):
            nb, _ = compare_codes(got.cpu().numpy().view(np.uint32).T, ref,
                                  code_ambiguity_mask(x, cb, M))
            assert nb == 0
    sel, cnt = fa.annca_select(oracle_codes_for_device(oq), oracle_codes_for_device(op), F)
    out = fa.attend_subset(q_dev, kp_dev, vp_dev, F, sel, cnt)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    got = out.float().cpu().numpy()
    kept = []
    for h in range(H):
        for g in range(F):
            rows = slice(g * Nf, (g + 1) * Nf)
            r = oannca.annca_frame(cp.Q[h, rows], cp.Kp[h], cp.Vp[h], None,
                                   codes_q=oq[h][rows], codes_p=op[h])
            n = int(cnt_h[h, g])
            assert n == r["sel"].size
            np.testing.assert_array_equal(sel_h[h, g, :n], r["sel"])
            if n:
                assert np.abs(got[h, rows] - r["o_sparse"]).max() <= 2e-2
            else:
                assert np.abs(got[h, rows]).max() == 0.0
            kept.append(n)
    print(f"AnnCA with PQ buckets kept per frame: {kept} of {cp.prompt_tokens}")
    assert max(kept) > 0


# ------------------------------------------------------------------ AnnSA

from oracle import annsa as oannsa  # noqa: E402
from synth import round_to_storage  # noqa: E402


def _annsa_cache(overrides, frames):
    return _annsa_cache_w(WORKLOADS["dit1.3b"].with_(**overrides), frames)


def _annsa_cache_w(w, frames):
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    Q = None
    for _ in range(frames):
        K, V, Q, _ = st.next_frame()
        orc.process_frame(K, V)
    cache = _cache_for(w, planes)
    cache.import_state(oracle_state_for_import(orc, w.dtype))
    return w, orc, cache, Q


def _annsa_planes(L, b, d, seed):
    rng = np.random.default_rng(seed)
    return round_to_storage(rng.standard_normal((L, b, d)).astype(np.float32), "bf16")


def _codes_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint32).view(np.int32)).cuda()


def _slot_codes(cache, orc, pl, L, b):
    """The GPU's slot codes (hash_slots), checked against the oracle's SimHash
    except at ambiguous bits; both sides then use these decided codes."""
    w = cache.cfg
    out = torch.empty((w.heads, L, w.budget), dtype=torch.int32, device="cuda")
    cache.hash_slots(to_device(pl, "bf16").contiguous(), L, b, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    per_head, amb = [], 0
    for h in range(w.heads):
        hc = orc.heads[h]
        S = hc.n_live
        ck = np.ascontiguousarray(got[h][:, :S].T)
        if b:
            nb, na = compare_codes(ck, simhash(hc.k_hat[:S], pl)[0], ambiguous_bit_mask(hc.k_hat[:S], pl))
            assert nb == 0
            amb += na
        per_head.append(ck)
    return per_head, amb


@pytest.mark.parametrize("L,b,seed,d", [(4, 6, 50, 128), (4, 12, 51, 128), (1, 4, 52, 128),
                                        (3, 8, 53, 128), (2, 16, 54, 128), (3, 12, 62, 64),
                                        (2, 16, 63, 64)])
def test_annsa_matches_oracle(L, b, seed, d):
    """Outputs within the bf16 bound; queries that share no bucket exactly zero
    with lse = -inf.  Short expected lists (12 and 16 bits) take the listing
    pass, long ones the plain pass; d = 64 rows are 8 features per lane."""
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=300, budget=2048, head_dim=d,
                                         seed=seed), 5)
    pl = _annsa_planes(L, b, w.head_dim, seed)
    H, Nq = w.heads, Q.shape[1]
    cks, amb = _slot_codes(cache, orc, pl, L, b)
    qc = np.zeros((H, L, Nq), np.uint32)
    refs = []
    for h in range(H):
        hc = orc.heads[h]
        S = hc.n_live
        cq = simhash(Q[h], pl)[0]
        qc[h] = cq.T
        refs.append(oannsa.annsa_attend(Q[h], hc.k_hat[:S], hc.v_hat[:S], hc.count[:S], cq, cks[h]))
    lse = torch.empty((H, Nq), dtype=torch.float32, device="cuda")
    out = cache.annsa_attend(to_device(Q, w.dtype), _codes_dev(qc), lse=lse)
    torch.cuda.synchronize()
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    for h, (O, lse_ref, nsh) in enumerate(refs):
        none = nsh == 0
        err = np.abs(got[h] - O).max()
        print(f"annsa L={L} b={b} head {h}: S={orc.heads[h].n_live} shared/query={nsh.mean():.1f} "
              f"({nsh.mean() / orc.heads[h].n_live:.2%}) no-bucket queries={none.sum()} "
              f"max-abs={err:.3e} ambiguous slot bits={amb}")
        assert err <= TOL["bf16"]
        assert (got[h][none] == 0).all() and np.isneginf(glse[h][none]).all()
        if (~none).any():
            lerr = np.abs(glse[h][~none] - lse_ref[~none]).max()
            assert lerr <= 1e-3 * max(1.0, np.abs(lse_ref[~none]).max())


def test_annsa_f32_tiny_matches_oracle():
    w, orc, cache, Q = _annsa_cache_w(WORKLOADS["tiny"], 5)
    pl = _annsa_planes(2, 6, w.head_dim, 58).astype(np.float32)
    out = torch.empty((1, 2, w.budget), dtype=torch.int32, device="cuda")
    cache.hash_slots(torch.from_numpy(pl).cuda().contiguous(), 2, 6, out=out)
    torch.cuda.synchronize()
    hc = orc.heads[0]
    S = hc.n_live
    ck = np.ascontiguousarray(out.cpu().numpy().view(np.uint32)[0][:, :S].T)
    nb, _ = compare_codes(ck, simhash(hc.k_hat[:S], pl)[0], ambiguous_bit_mask(hc.k_hat[:S], pl))
    assert nb == 0
    cq = simhash(Q[0], pl)[0]
    O, lse_ref, nsh = oannsa.annsa_attend(Q[0], hc.k_hat[:S], hc.v_hat[:S], hc.count[:S], cq, ck)
    got = cache.annsa_attend(to_device(Q, "f32"), _codes_dev(cq.T[None]))
    torch.cuda.synchronize()
    err = np.abs(got.cpu().numpy()[0] - O).max()
    print(f"annsa tiny fp32: shared/query={nsh.mean():.1f} max-abs={err:.3e}")
    assert err <= TOL["f32"]


def test_annsa_hash_slots_matches_oracle():
    w, orc, cache, _ = _annsa_cache(dict(heads=2, tokens_per_frame=250, budget=1024, seed=55), 4)
    _, amb = _slot_codes(cache, orc, _annsa_planes(4, 16, w.head_dim, 55), 4, 16)
    print(f"hash_slots: ambiguous differing bits={amb}")


def test_annsa_all_shared_equals_attend():
    """0-bit codes: every query shares the one bucket with every slot, which is
    the dense step over the cache."""
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=300, budget=2048, seed=56), 4)
    H, Nq = w.heads, Q.shape[1]
    q = to_device(Q, w.dtype)
    dense = cache.attend(q)
    cache.hash_slots(torch.zeros(0, dtype=torch.bfloat16, device="cuda"), 2, 0)
    sparse = cache.annsa_attend(q, _codes_dev(np.zeros((H, 2, Nq))))
    torch.cuda.synchronize()
    diff = (sparse.float() - dense.float()).abs().max().item()
    print(f"annsa all-shared vs attend: max-abs {diff:.3e}")
    assert diff <= 1e-2


def test_annsa_overflowing_short_lists_equal_attend():
    """16-bit codes (a short expected list per query) with zero hyperplanes:
    every slot's code is 0, so a query with code 0 shares every slot and its
    list overflows into the second pass; the result is the dense step."""
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=300, budget=2048, seed=61), 4)
    H, Nq = w.heads, Q.shape[1]
    q = to_device(Q, w.dtype)
    dense = cache.attend(q)
    cache.hash_slots(torch.zeros((1, 16, w.head_dim), dtype=torch.bfloat16, device="cuda"), 1, 16)
    sparse = cache.annsa_attend(q, _codes_dev(np.zeros((H, 1, Nq))))
    torch.cuda.synchronize()
    diff = (sparse.float() - dense.float()).abs().max().item()
    print(f"annsa 16-bit all-shared vs attend: max-abs {diff:.3e}")
    # two bf16 outputs of different summation orders (binary32 online softmax
    # against bf16 MFMA weights): the attention output bound applies
    assert diff <= TOL["bf16"]


def test_annsa_nothing_shared_gives_zeros():
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=100, budget=512, seed=57), 3)
    H, Nq = w.heads, Q.shape[1]
    cache.hash_slots(to_device(_annsa_planes(3, 16, w.head_dim, 57), "bf16").contiguous(), 3, 16)
    lse = torch.empty((H, Nq), dtype=torch.float32, device="cuda")
    out = cache.annsa_attend(to_device(Q, w.dtype), _codes_dev(np.full((H, 3, Nq), 0xFFFFFFFF)),
                             lse=lse)
    torch.cuda.synchronize()
    assert (out == 0).all() and torch.isneginf(lse).all()


def test_annsa_refuses_a_stale_index():
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=100, budget=512, seed=59), 2)
    H, Nq = w.heads, Q.shape[1]
    q, qc = to_device(Q, w.dtype), _codes_dev(np.zeros((H, 2, Nq)))
    with pytest.raises(fa.FastarError):
        cache.annsa_attend(q, qc)                      # never indexed
    pl = to_device(_annsa_planes(2, 8, w.head_dim, 59), "bf16").contiguous()
    cache.hash_slots(pl, 2, 8)
    cache.annsa_attend(q, qc)
    with pytest.raises(fa.FastarError):
        cache.annsa_attend(q, _codes_dev(np.zeros((H, 3, Nq))))   # other table count
    K = to_device(np.zeros((H, 100, w.head_dim), np.float32), w.dtype)
    cache.match_merge(K, K, 100, 1)
    with pytest.raises(fa.FastarError):
        cache.annsa_attend(q, qc)                      # the cache changed since
    torch.cuda.synchronize()


def test_rejected_calls_leave_the_state_and_the_annsa_index_intact():
    """Argument errors are found before anything changes: a refused
    match_merge or import leaves the slot state as it was, and an AnnSA index
    built before it stays usable."""
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=100, budget=512, seed=60), 3)
    H, Nq = w.heads, Q.shape[1]
    q, qc = to_device(Q, w.dtype), _codes_dev(np.zeros((H, 2, Nq)))
    cache.hash_slots(to_device(_annsa_planes(2, 8, w.head_dim, 60), "bf16").contiguous(), 2, 8)
    ref = cache.annsa_attend(q, qc).float().cpu()
    before = cache.export_state()
    # more tokens in a frame than the budget: refused on the host
    K = to_device(np.zeros((H, 600, w.head_dim), np.float32), w.dtype)
    with pytest.raises(fa.FastarError):
        cache.match_merge(K, K, 600, 1)
    good = oracle_state_for_import(orc, w.dtype)
    bad_count = {k: v.copy() if isinstance(v, np.ndarray) else v for k, v in good.items()}
    bad_count["count"][1, 5] = 0                       # a live slot with no token
    bad_last = {k: v.copy() if isinstance(v, np.ndarray) else v for k, v in good.items()}
    bad_last["last"][0, 7] = good["frame"]             # updated "at" the next frame
    bad_nlive = {"n_live": np.array([513, 3], np.int32)}
    stale_frame = {"frame": 0}                         # live slots updated at frames 0..2
    for bad in (bad_count, bad_last, bad_nlive, stale_frame):
        with pytest.raises(fa.FastarError):
            cache.import_state(bad)
    after = cache.export_state()
    for k in before:
        np.testing.assert_array_equal(np.asarray(after[k]), np.asarray(before[k]), err_msg=k)
    again = cache.annsa_attend(q, qc).float().cpu()     # the index is still current
    torch.cuda.synchronize()
    assert torch.equal(again, ref)
    assert cache.stats()["refused_frames"] == 0


def test_import_without_frame_keeps_the_frame_counter():
    w, orc, cache, Q = _annsa_cache(dict(heads=2, tokens_per_frame=100, budget=512, seed=61), 3)
    frame = cache.stats()["frame"]
    assert frame == 3
    st = cache.export_state()
    cache.import_state({"codes": st["codes"]})
    assert cache.stats()["frame"] == frame


@pytest.mark.parametrize("tokens", [30, 97])   # 30: evictions span 6 frames; 97: all 20
def test_eviction_across_many_last_update_frames(tokens):
    """Eviction when the evicted slots span several last-update frames: 100
    live slots updated at frames 0..19 (5 each, scattered over the slot ids),
    then a frame of fresh keys that all insert.  The planner walks the
    distinct frames upward for a few of them and falls back to a radix
    select beyond; decisions and state are checked against the oracle."""
    from oracle import HeadCache
    w = WORKLOADS["tiny"].with_(heads=2, budget=100, tokens_per_frame=tokens)
    rng = np.random.default_rng(70 + tokens)
    planes = DriftStream(w).planes()
    orc = TempCacheOracle.for_workload(w, planes)
    for hc in orc.heads:
        hc.n_live = 100
        hc.K_m[:] = rng.standard_normal((100, w.head_dim)).astype(np.float32)
        hc.V_m[:] = rng.standard_normal((100, w.head_dim)).astype(np.float32)
        hc.k_hat[:] = hc.K_m
        hc.v_hat[:] = hc.V_m
        hc.count[:] = rng.integers(1, 4, size=100)
        hc.last[:] = rng.permutation(np.repeat(np.arange(20), 5))
        hc.codes[:] = hc.hash(hc.k_hat)
        hc.frame = 20
        hc._rebuild_buckets()
    cache = _cache_for(w, planes)
    cache.import_state(oracle_state_for_import(orc, w.dtype))
    K = rng.standard_normal((w.heads, tokens, w.head_dim)).astype(np.float32)
    V = rng.standard_normal((w.heads, tokens, w.head_dim)).astype(np.float32)
    res = orc.process_frame(K, V)
    assert all(not r.merged.any() and len(r.evicted) == tokens for r in res)
    slot_out = torch.empty((w.heads, tokens), dtype=torch.int32, device="cuda")
    cache.match_merge(to_device(K, w.dtype), to_device(V, w.dtype), tokens, 1, slot_out=slot_out)
    torch.cuda.synchronize()
    so = slot_out.cpu().numpy()
    for h in range(w.heads):
        np.testing.assert_array_equal(so[h], res[h].slot)
    compare_state(cache.export_state(), orc, w.dtype)
    assert cache.stats()["refused_frames"] == 0


@pytest.mark.parametrize("heads,qpf,frames,bits", [(2, 300, 3, 16), (3, 77, 2, 12), (12, 1560, 3, 16),
                                                   (2, 64, 1, 0)])
def test_fused_annca_equals_hash_select_and_subset_attention(heads, qpf, frames, bits):
    """Hashing the queries and then one attention launch that selects in its
    prologue gives the three-launch path's output bit for bit (same codes, same
    kept lists, same attention kernel) and leaves the hash entry's codes in
    q_codes; on two sampled heads it is also within the bf16 bound of the
    oracle's sparse attention.  bits = 0 keeps every prompt row."""
    cp = ClusterPrompt(heads=heads, queries_per_frame=qpf, frames=frames, bits=bits)
    planes = cp.planes()
    q = to_device(cp.Q, "bf16")
    kp, vp = to_device(cp.Kp, "bf16"), to_device(cp.Vp, "bf16")
    pl = _planes_dev(planes, "bf16") if bits else torch.zeros(0, dtype=torch.bfloat16, device="cuda")
    qc = fa.hash_codes(q, pl, cp.tables, cp.bits)
    pc = fa.hash_codes(kp, pl, cp.tables, cp.bits)
    sel, cnt = fa.annca_select(qc, pc, frames)
    ref = fa.attend_subset(q, kp, vp, frames, sel, cnt)
    qc_fused = torch.full_like(qc, -1)
    got = fa.annca_attend(q, pl, cp.tables, cp.bits, pc, kp, vp, frames, q_codes=qc_fused)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(qc_fused, qc)
    if bits == 0:
        assert (cnt.cpu().numpy() == cp.prompt_tokens).all()
    gq, gp = qc.cpu().numpy().view(np.uint32), pc.cpu().numpy().view(np.uint32)
    out = got.float().cpu().numpy()
    for h in (0, heads - 1):
        for g in range(frames):
            rows = slice(g * qpf, (g + 1) * qpf)
            r = oannca.annca_frame(cp.Q[h, rows], cp.Kp[h], cp.Vp[h], planes,
                                   codes_q=np.ascontiguousarray(gq[h][:, rows].T),
                                   codes_p=np.ascontiguousarray(gp[h].T))
            assert np.abs(out[h, rows] - r["o_sparse"]).max() <= 2e-2


def test_fused_annca_frame_keeping_nothing_gives_zeros():
    cp = ClusterPrompt(heads=2, queries_per_frame=100, frames=2)
    q = to_device(cp.Q, "bf16")
    kp, vp = to_device(cp.Kp, "bf16"), to_device(cp.Vp, "bf16")
    pl = _planes_dev(cp.planes(), "bf16")
    # prompt codes wider than 16 bits match no 16-bit query code
    pc = torch.full((2, cp.tables, cp.prompt_tokens), 1 << 20, dtype=torch.int32, device="cuda")
    got = fa.annca_attend(q, pl, cp.tables, cp.bits, pc, kp, vp, 2)
    torch.cuda.synchronize()
    assert (got == 0).all()


def test_two_launch_annca_with_strided_rows():
    """Queries, keys, values and outputs as row-strided views (each row the
    first 128 of 256 features, heads 2 rows apart): the hash and the attention
    launches read the same strides; the result equals the contiguous call."""
    cp = ClusterPrompt(heads=3, queries_per_frame=200, frames=2)
    pl = _planes_dev(cp.planes(), "bf16")
    q = to_device(cp.Q, "bf16")
    kp, vp = to_device(cp.Kp, "bf16"), to_device(cp.Vp, "bf16")
    pc = fa.hash_codes(kp, pl, cp.tables, cp.bits)
    ref = fa.annca_attend(q, pl, cp.tables, cp.bits, pc, kp, vp, 2)

    def wide(x):  # [H][N][d] -> view of a [H][N][2d] buffer, first d features
        buf = torch.zeros((x.shape[0], x.shape[1], 2 * x.shape[2]), dtype=x.dtype, device=x.device)
        buf[:, :, :x.shape[2]] = x
        return buf[:, :, :x.shape[2]]

    qs, ks, vs = wide(q), wide(kp), wide(vp)
    out = torch.full((3, q.shape[1], 256), 7.0, dtype=torch.bfloat16, device="cuda")
    got = fa.annca_attend(qs, pl, cp.tables, cp.bits, pc, ks, vs, 2, out=out[:, :, :128])
    torch.cuda.synchronize()
    assert qs.stride(1) == 256 and ks.stride(1) == 256
    assert torch.equal(got, ref)
    assert (out[:, :, 128:] == 7.0).all()  # nothing written past each row's 128 features


@pytest.mark.parametrize("nq", [300, 1, 2000])
def test_tail_split_changes_only_the_summation_order(nq):
    """A launch whose (head, query tile) pairs all fit in the last round runs
    them as key-tile quarters plus a combine; a 1023-slot cache (below 16 key
    tiles) never splits.  The same imported state in both: outputs within
    bf16 rounding of each other and of the oracle, log-partitions within
    1e-3 relative.  (Quarters with no key tile, when a head holds fewer than
    four, are covered by the one-frame cases of test_attend_matches_oracle.)"""
    w = WORKLOADS["dit1.3b"].with_(heads=3, tokens_per_frame=220, budget=1024, seed=57)
    st = DriftStream(w)
    planes = st.planes()
    orc = TempCacheOracle.for_workload(w, planes)
    for _ in range(4):
        K, V, _, _ = st.next_frame()
        orc.process_frame(K, V)
    q = np.random.default_rng(5).standard_normal((w.heads, nq, w.head_dim)).astype(np.float32)
    q = round_to_storage(q, "bf16")
    state = oracle_state_for_import(orc, w.dtype)
    outs = {}
    # at most 880 slots are live, so the 1023-slot cache takes the same state
    # with the slot axis (the last of codes, the second of the others) cut
    small = dict(state)
    for k in ("k_master", "v_master", "k_mirror", "v_mirror", "count", "last"):
        small[k] = state[k][:, :1023]
    small["codes"] = state["codes"][:, :, :1023]
    for budget, st_b in ((1024, state), (1023, small)):
        cache = _cache_for(w.with_(budget=budget), planes)
        cache.import_state(st_b)
        lse = torch.empty((w.heads, nq), dtype=torch.float32, device="cuda")
        outs[budget] = (cache.attend(to_device(q, "bf16"), lse=lse), lse)
    torch.cuda.synchronize()
    (o_split, l_split), (o_whole, l_whole) = outs[1024], outs[1023]
    O_ref, lse_ref = orc.attend(q)
    assert (o_split.float() - o_whole.float()).abs().max().item() <= 8e-3
    assert np.abs(o_split.float().cpu().numpy() - O_ref).max() <= TOL["bf16"]
    lim = 1e-3 * max(1.0, np.abs(lse_ref).max())
    assert np.abs(l_split.cpu().numpy() - lse_ref).max() <= lim
    assert (l_split - l_whole).abs().max().item() <= lim
